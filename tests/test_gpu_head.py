"""GPU parity of the FP8 output head (the step after the last layer of a
verify pass; TandemLLM manual, "What TandemLLM is", 1.2 "Two levers") against
the CPU oracle: |C_gpu - C| <= 1e-5 * sum_k |a w| per element, the bar of the
NVFP4 GEMM. The HIP path computes exact bf16 weights and fp32 MFMA sums, then
one fp32 product with the row scale, so the error is fp32 summation rounding."""

import os
import sys

import numpy as np
import pytest

import nvfp4_skinny_gemm_amd as nv
import synth

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


@pytest.fixture(scope="module")
def ctx(torch_cuda):
    c = nv.Context(0)
    yield c
    c.close()


def bf16_dev(torch, a_bits):
    return torch.from_numpy(np.ascontiguousarray(a_bits).view(np.int16)).cuda().view(torch.bfloat16)


def check(oracle, c_gpu, c_ref, s_ref, label):
    ok = oracle.within_tolerance(c_gpu, c_ref, s_ref)
    if not ok.all():
        i, j = np.argwhere(~ok)[0]
        raise AssertionError("%s: %d of %d outside 1e-5*S; first at [%d,%d]: gpu=%r ref=%r S=%r"
                             % (label, int((~ok).sum()), ok.size, i, j, float(c_gpu[i, j]),
                                c_ref[i, j], s_ref[i, j]))


# Several row tiles and k-tiles with ragged tails (N % 16, K % 256), one to
# four row blocks of M and two blocks of 64 rows (M = 100), and the degenerate
# single row / single 16-wide k-block.
@pytest.mark.parametrize("n,k,m", [(1, 16, 1), (17, 48, 5), (100, 272, 16), (33, 1040, 17),
                                   (64, 512, 32), (250, 784, 7), (129, 2064, 24), (250, 784, 48),
                                   (129, 2064, 100)])
def test_head_parity_quantised(torch_cuda, ctx, oracle_mod, n, k, m):
    torch = torch_cuda
    log("head parity n=%d k=%d m=%d" % (n, k, m))
    w = synth.weights_f32(n, k, seed=n + k, stream="head")
    codes, scales = nv.fp8_quantize_host(w)
    oc, os_ = oracle_mod.fp8_quantize(w)
    assert np.array_equal(codes, oc) and np.array_equal(scales, os_)
    packed = torch.from_numpy(nv.fp8_pack_host(codes, scales)).cuda()
    a = synth.activations_bf16(m, k, seed=m, stream="head", outliers=True)
    ad = bf16_dev(torch, a)
    c = ctx.fp8_head_gemm(ad, packed, n, k)
    act = ctx.pack_activations(ad)
    c2 = ctx.fp8_head_gemm_pa(act, m, k, packed, n)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle_mod.fp8_gemm(a, codes, scales)
    check(oracle_mod, c.cpu().numpy(), c_ref, s_ref, "fp8 head n=%d k=%d m=%d" % (n, k, m))
    assert torch.equal(c, c2)


@pytest.mark.parametrize("lds", ["0", "1"])
@pytest.mark.parametrize("r", ["1", "2", "4"])
def test_head_tilings_bitwise_equal(torch_cuda, ctx, monkeypatch, r, lds):
    """Every wave sums its rows over all of K in the same order, so neither the
    row tiles per wave nor where the activations are staged (each wave's own
    loads, or one copy per work-group in LDS) change anything in C; one to
    four row blocks of M, ragged N and K."""
    torch = torch_cuda
    n, k = 301, 1296
    codes = synth.fp8_codes(n, k, seed=9)
    scales = synth.fp8_row_scales(n, seed=9)
    packed = torch.from_numpy(nv.fp8_pack_host(codes, scales)).cuda()
    for m in (3, 16, 30, 40, 64):
        ad = bf16_dev(torch, synth.activations_bf16(m, k, seed=m, stream="headr"))
        monkeypatch.setenv("NVFP4V_HEAD_LDS", "0")
        monkeypatch.delenv("NVFP4V_HEAD_R", raising=False)
        base = ctx.fp8_head_gemm(ad, packed, n, k)
        monkeypatch.setenv("NVFP4V_HEAD_R", r)
        monkeypatch.setenv("NVFP4V_HEAD_LDS", lds)
        other = ctx.fp8_head_gemm(ad, packed, n, k)
        torch.cuda.synchronize()
        assert torch.equal(base, other), "m=%d r=%s lds=%s" % (m, r, lds)


@pytest.fixture(scope="module")
def full_head(torch_cuda):
    n, k = 151936, 5120
    codes = synth.fp8_codes(n, k, seed=1)
    scales = synth.fp8_row_scales(n, seed=1)
    packed = torch_cuda.from_numpy(nv.fp8_pack_host(codes, scales)).cuda()
    return n, k, codes, scales, packed


@pytest.mark.parametrize("m", [1, 16, 32, 64, 128])
def test_head_full_size_sampled(torch_cuda, ctx, oracle_mod, full_head, m):
    """The LM head of the 27B stack, 151936 x 5120, at the tree sizes: random
    finite E4M3 codes and row scales; 640 sampled rows (both ends included)
    against the oracle; every output finite."""
    torch = torch_cuda
    n, k, codes, scales, packed = full_head
    log("head full size m=%d" % m)
    a = synth.activations_bf16(m, k, seed=m, stream="headfull")
    c = ctx.fp8_head_gemm(bf16_dev(torch, a), packed, n, k).cpu().numpy()
    assert np.isfinite(c).all()
    cols = np.unique(np.concatenate([[0, 15, 16, n - 1],
                                     synth.rng(5, "headcols").integers(0, n, 636)]))
    c_ref, s_ref = oracle_mod.fp8_gemm(a, codes, scales, cols=cols)
    check(oracle_mod, c[:, cols], c_ref, s_ref, "fp8 head full m=%d" % m)


def test_head_argument_errors(torch_cuda, ctx):
    torch = torch_cuda
    packed = torch.zeros(nv.fp8_packed_bytes(32, 256), dtype=torch.uint8, device="cuda")
    a = torch.zeros((129, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.Nvfp4vError) as e:
        ctx.fp8_head_gemm(a, packed, 32, 256)
    assert e.value.status == nv.E_M_RANGE
    # a K that is not a multiple of 16 is the library's shape error
    a200 = torch.zeros((4, 200), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.Nvfp4vError) as e:
        ctx.fp8_head_gemm(a200, packed, 32, 200)
    assert e.value.status == nv.E_SHAPE
    # a tensor that does not match the sizes passed is refused by the binding
    # before its address reaches the library
    with pytest.raises(ValueError):
        ctx.fp8_head_gemm(a[:4], packed, 32, 200)
    with pytest.raises(ValueError):
        ctx.verify_gemm(a[:4], packed, 32, 128)
    with pytest.raises(ValueError):
        ctx.fp8_head_gemm(a[:4], packed[:100], 32, 256)
