"""StairCut's cut on a staircase measured on this GPU: the library's cut and
the oracle's agree on the node count, the kept nodes and the rate for seeded
draft trees, priced by the verify pass itself (two full-size layers, M = 1..32
rows, graph-free timing with HIP events on the pass's stream)."""

import sys

import numpy as np
import pytest

import nvfp4_skinny_gemm_amd as nv
import synth
from oracle import staircut as oc

pytestmark = pytest.mark.gpu

H, I, LAYERS = 5120, 17408, 2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


@pytest.fixture(scope="module")
def measured_staircase(torch_cuda):
    torch = torch_cuda
    from test_gpu_pass import small_stack

    ctx = nv.Context(0)
    try:
        packed, arr = small_stack(torch, ctx, LAYERS, H, I, seed=11)
        h0 = torch.from_numpy(synth.activations_bf16(64, H, seed=1).view(np.int16)).cuda().view(torch.bfloat16)
        ws = torch.empty(nv.pass_workspace_bytes(32, H, I, LAYERS), dtype=torch.uint8, device="cuda")
        h_out = torch.empty((32, H), dtype=torch.bfloat16, device="cuda")
        stream = torch.cuda.current_stream()
        us = np.zeros(32)
        for m in range(1, 33):
            for _ in range(2):
                ctx.verify_pass(arr, H, I, h0[:m], ws, h_out[:m])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                ctx.verify_pass(arr, H, I, h0[:m], ws, h_out[:m])
            e1.record(stream)
            torch.cuda.synchronize()
            us[m - 1] = e0.elapsed_time(e1) * 1e3 / 5
        assert ctx.pass_status() == nv.OK and ctx.device_status() == nv.OK
        log("verify pass of %d layers, us by rows: %s" % (LAYERS, " ".join("%.0f" % x for x in us)))
        assert (us > 0).all()
        return us
    finally:
        ctx.close()


@pytest.mark.parametrize("seed", range(8))
def test_cut_on_measured_staircase(measured_staircase, seed):
    us = measured_staircase
    shape = ("random", "wide", "chain", "random")[seed % 4]
    parent, p = synth.draft_tree(31, seed=seed, stream="gpu-tree", shape=shape)
    n, keep, e, rate = nv.staircut(us, parent, p)
    n2, kept2, e2, rate2 = oc.cut(us, parent, p)
    log("tree %d (%s): keeps %d nodes, %.3f tokens, %.4f tokens/ms" % (seed, shape, n, e, rate))
    assert n == n2
    assert sorted(np.nonzero(keep)[0].tolist()) == kept2
    assert e == pytest.approx(e2, rel=1e-15) and rate == pytest.approx(rate2, rel=1e-15)
