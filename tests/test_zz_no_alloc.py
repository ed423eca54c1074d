"""The entry point that allocates nothing (nvfp4v_verify_gemm_static) against
nvfp4v_verify_gemm, bitwise, on two calls in a row, the second smaller; both
on the same device, through the C ABI."""

import numpy as np
import pytest

import nvfp4_skinny_gemm_amd as nv
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def make(torch, ctx, n, k, seed):
    w = synth.weights_f32_cuda(n, k, seed=seed, stream="noalloc")
    codes, scales = ctx.quantize(w)
    return ctx.pack(codes, scales, n, k)


def test_static_entry_matches_context_entry(torch_cuda):
    torch = torch_cuda
    ctx = nv.Context(0)
    try:
        # down [5120 x 17408] at 16 rows (split into K pieces: partials and
        # counters in the scratch array), then a smaller call: q|k|v-sized
        # [1024 x 5120] at 5 rows, then 100 rows (two blocks of 64) of the first.
        big = make(torch, ctx, 5120, 17408, 1)
        small = make(torch, ctx, 1024, 5120, 2)
        a_big = torch.from_numpy(synth.activations_bf16(128, 17408, seed=3).view(np.int16)).cuda().view(torch.bfloat16)
        a_small = torch.from_numpy(synth.activations_bf16(128, 5120, seed=4).view(np.int16)).cuda().view(torch.bfloat16)
        for a, packed, n, k, m in ((a_big, big, 5120, 17408, 16), (a_small, small, 1024, 5120, 5),
                                   (a_big, big, 5120, 17408, 100)):
            print("static entry n=%d k=%d m=%d plan: %s" % (n, k, m, ctx.describe_plan(n, k, m)), flush=True)
            want = ctx.verify_gemm(a[:m].contiguous(), packed, n, k, ts=1.5)
            out = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
            got = nv.verify_gemm_static(a[:m].contiguous(), packed, n, k, ts=1.5, out=out)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int32), want.view(torch.int32)), "n=%d k=%d m=%d" % (n, k, m)
        assert ctx.device_status() == nv.OK
    finally:
        ctx.close()


def test_static_entry_argument_errors(torch_cuda):
    torch = torch_cuda
    a = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    packed = torch.zeros(nv.packed_bytes(32, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((4, 32), dtype=torch.float32, device="cuda")
    lib = nv.load()
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert lib.nvfp4v_verify_gemm_static(p(a), 0, 256, p(packed), 32, 1.0, p(out), None) == nv.E_M_RANGE
    assert lib.nvfp4v_verify_gemm_static(p(a), 129, 256, p(packed), 32, 1.0, p(out), None) == nv.E_M_RANGE
    assert lib.nvfp4v_verify_gemm_static(p(a), 4, 250, p(packed), 32, 1.0, p(out), None) == nv.E_SHAPE
    assert lib.nvfp4v_verify_gemm_static(None, 4, 256, p(packed), 32, 1.0, p(out), None) == nv.E_INVALID_ARG
    # K beyond the scratch array's activation block (16 MiB for both copies at 64 rows)
    assert lib.nvfp4v_verify_gemm_static(p(a), 64, 65536 + 256, p(packed), 32, 1.0, p(out), None) == nv.E_WORKSPACE
