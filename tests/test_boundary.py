"""The C-ABI boundary on the CPU: the library loads, exports what the header
declares, validates arguments before any HIP call, and its host-side format
code (quantiser, E4M3 encoder) matches the oracle byte for byte."""

import ctypes
import os

import numpy as np
import pytest

import nvfp4_skinny_gemm_amd as nv
import synth


@pytest.fixture(scope="module")
def lib():
    return nv.load()


def test_exports_every_declared_symbol(lib):
    names = nv.exported_names()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name


def test_strerror(lib):
    for code in range(0, -11, -1):
        assert nv.strerror(code) and nv.strerror(code) != "unknown status"
    assert nv.strerror(-99) == "unknown status"


def test_packed_bytes():
    assert nv.packed_bytes(17408, 5120) == 17408 * 5120 // 2 + 17408 * 5120 // 16
    assert nv.packed_bytes(5120, 17408) == 50135040
    assert nv.packed_bytes(151936, 5120) == 437575680
    assert nv.packed_bytes(512, 256) == 73728
    assert nv.packed_bytes(17, 48) == 2 * 1 * 2304   # padded to 32 rows x 256 k
    assert nv.packed_bytes(0, 256) == 0
    assert nv.packed_bytes(16, 40) == 0


class _CtxFields(ctypes.Structure):
    # mirrors the leading fields of struct nvfp4v_ctx (csrc/internal.h)
    _fields_ = [("device", ctypes.c_int), ("num_cus", ctypes.c_int), ("last_hip", ctypes.c_int),
                ("partials", ctypes.c_void_p), ("partial_floats", ctypes.c_size_t),
                ("counters", ctypes.c_void_p), ("n_counters", ctypes.c_size_t)]


_KEEP = []


class FakeCtx:
    """A host block standing in for a context with an empty workspace and 256 CUs:
    every call made with it must return from its host-side checks, before any
    HIP call. Kept alive for the whole module."""

    def __init__(self):
        self.fields = _CtxFields(0, 256, 0, None, 0, None, 0)
        self.ptr = ctypes.cast(ctypes.pointer(self.fields), ctypes.c_void_p)
        _KEEP.append(self)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# These tests hand fake device addresses to the library; they are host-only and
# never run where a GPU could receive a launch.
host_only = pytest.mark.skipif(_gpu_visible(), reason="host-only argument checks")


def fake_dev(addr=0x1000):
    return ctypes.c_void_p(addr)


@host_only
def test_verify_gemm_argument_errors(lib):
    ctx = FakeCtx().ptr
    a, w, c = fake_dev(0x10000), fake_dev(0x20000), fake_dev(0x30000)
    f = lib.nvfp4v_verify_gemm
    assert f(None, a, 8, 256, w, 512, 1.0, c, None) == nv.E_INVALID_ARG
    assert f(ctx, None, 8, 256, w, 512, 1.0, c, None) == nv.E_INVALID_ARG
    assert f(ctx, a, 8, 256, None, 512, 1.0, c, None) == nv.E_INVALID_ARG
    assert f(ctx, a, 8, 256, w, 512, 1.0, None, None) == nv.E_INVALID_ARG
    assert f(ctx, a, 0, 256, w, 512, 1.0, c, None) == nv.E_M_RANGE
    assert f(ctx, a, 65, 256, w, 512, 1.0, c, None) == nv.E_M_RANGE
    assert f(ctx, a, 8, 250, w, 512, 1.0, c, None) == nv.E_SHAPE
    assert f(ctx, a, 8, 0, w, 512, 1.0, c, None) == nv.E_SHAPE
    assert f(ctx, a, 8, 256, w, 0, 1.0, c, None) == nv.E_SHAPE
    assert f(ctx, fake_dev(0x10008), 8, 256, w, 512, 1.0, c, None) == nv.E_ALIGN
    assert f(ctx, a, 8, 256, fake_dev(0x20004), 512, 1.0, c, None) == nv.E_ALIGN
    assert f(ctx, a, 8, 256, w, 512, 1.0, fake_dev(0x30002), None) == nv.E_ALIGN
    # a zero-sized workspace cannot hold split-K partials
    assert f(ctx, a, 8, 17408, w, 5120, 1.0, c, None) == nv.E_WORKSPACE


@host_only
def test_fault_injection(lib, monkeypatch):
    ctx = FakeCtx().ptr
    monkeypatch.setenv("NVFP4V_FAULT", "launch")
    out = ctypes.c_void_p()
    assert lib.nvfp4v_create(ctypes.byref(out), 0) == nv.E_FAULT
    assert lib.nvfp4v_pack(ctx, fake_dev(), fake_dev(), 16, 128, fake_dev(0x40000), None) == nv.E_FAULT
    assert lib.nvfp4v_quantize(ctx, fake_dev(), 16, 128, fake_dev(), fake_dev(), None) == nv.E_FAULT
    assert lib.nvfp4v_staircase(ctx, 16, 128, 1, 2, 0, 1, 0, fake_dev()) == nv.E_FAULT


@host_only
def test_other_argument_errors(lib):
    ctx = FakeCtx().ptr
    assert lib.nvfp4v_create(None, 0) == nv.E_INVALID_ARG
    out = ctypes.c_void_p()
    assert lib.nvfp4v_create(ctypes.byref(out), -1) == nv.E_INVALID_ARG
    assert lib.nvfp4v_pack(ctx, fake_dev(), fake_dev(), 16, 100, fake_dev(), None) == nv.E_SHAPE
    assert lib.nvfp4v_pack(ctx, fake_dev(), fake_dev(), 16, 128, fake_dev(0x1001), None) == nv.E_ALIGN
    assert lib.nvfp4v_unpack(ctx, fake_dev(0x1004), 16, 128, fake_dev(), fake_dev(), None) == nv.E_ALIGN
    assert lib.nvfp4v_quantize(ctx, fake_dev(), 16, 24, fake_dev(), fake_dev(), None) == nv.E_SHAPE
    us = (ctypes.c_double * 4)()
    assert lib.nvfp4v_staircase(ctx, 16, 128, 0, 2, 0, 1, 0, us) == nv.E_M_RANGE
    assert lib.nvfp4v_staircase(ctx, 16, 128, 3, 2, 0, 1, 0, us) == nv.E_M_RANGE
    assert lib.nvfp4v_staircase(ctx, 16, 128, 1, 65, 0, 1, 0, us) == nv.E_M_RANGE
    assert lib.nvfp4v_staircase(ctx, 16, 128, 1, 2, 0, 0, 0, us) == nv.E_INVALID_ARG
    buf = ctypes.create_string_buffer(8)
    assert lib.nvfp4v_describe_plan(ctx, 16, 128, 0, buf, 8) == nv.E_M_RANGE
    assert lib.nvfp4v_device_status(None) == nv.E_INVALID_ARG
    assert nv.strerror(nv.E_DISPATCH) != "unknown status"


def test_host_quantiser_matches_oracle(oracle_mod):
    w = synth.weights_f32(300, 512, seed=0, stream="boundary")
    w[0, :16] = 0.0
    w[1, :16] = np.float32(1e-5)
    w[2, :16] = np.float32(5000.0)
    w[3, :16] = -np.float32(1e-9)
    w[3, 0] = 6.0
    w[4, :16] = np.float32([6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -1.25, -1.75, -2.5, -3.5, -5, 0])
    w[5, :16] *= np.float32(2.0 ** -12)
    w[6, 16:32] = np.float32(6.375)
    w[7] *= np.float32(1e-3)
    w[8] *= np.float32(300.0)
    codes, scales = nv.quantize_host(w)
    oc, os_ = oracle_mod.quantize(w)
    assert np.array_equal(scales, os_)
    assert np.array_equal(codes, oc)


def test_host_quantiser_rejects_nonfinite():
    w = np.zeros((2, 32), np.float32)
    w[1, 5] = np.inf
    with pytest.raises(nv.Nvfp4vError) as ei:
        nv.quantize_host(w)
    assert ei.value.status == nv.E_NONFINITE


def test_host_e4m3_encoder_matches_oracle(oracle_mod):
    g = np.random.default_rng(5)
    x = np.concatenate([np.exp2(g.uniform(-14, 10, 20000)), synth.tiny_scale_values(64, 256).ravel()])
    vals = np.array([oracle_mod.e4m3_value(b) for b in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, vals, mids, [448.0, 460.0, 464.0, 500.0, 0.0]]).astype(np.float32)
    x = np.concatenate([x, -x])
    got = nv.encode_e4m3_host(x)
    ref = np.array([oracle_mod.e4m3_encode(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, ref)
    with pytest.raises(nv.Nvfp4vError):
        nv.encode_e4m3_host(np.float32([1.0, np.nan]))


def test_fp8_host_quantiser_matches_oracle(oracle_mod):
    w = synth.weights_f32(37, 272, seed=11, stream="fp8q")
    w[3] = 0.0
    w[5, 7] = -w[5].__abs__().max() * 2
    codes, scales = nv.fp8_quantize_host(w)
    oc, os_ = oracle_mod.fp8_quantize(w)
    assert np.array_equal(codes, oc)
    assert np.array_equal(scales.view(np.uint32), os_.view(np.uint32))
    w[1, 1] = np.nan
    with pytest.raises(nv.Nvfp4vError):
        nv.fp8_quantize_host(w)


def test_fp8_pack_layout():
    """The packed head re-read with the layout the header states: 16-row x 256-k
    tiles of 4096 bytes; load p, lane r + 16 h holds row r, k = 64 h + 16 p + b;
    then fp32 row scales padded to whole row tiles."""
    n, k = 37, 784
    codes = synth.fp8_codes(n, k, seed=2)
    scales = synth.fp8_row_scales(n, seed=2)
    packed = nv.fp8_pack_host(codes, scales)
    nrt, nkt = (n + 15) // 16, (k + 255) // 256
    assert packed.size == nv.fp8_packed_bytes(n, k) == nrt * nkt * 4096 + nrt * 64
    t = packed[:nrt * nkt * 4096].reshape(nrt, nkt, 4, 4, 16, 16)  # rt, kt, p, h, r, b
    full = np.zeros((nrt * 16, nkt * 256), np.uint8)
    for rt in range(nrt):
        for kt in range(nkt):
            blk = t[rt, kt].transpose(2, 1, 0, 3).reshape(16, 256)  # r, (h, p, b)
            full[rt * 16:(rt + 1) * 16, kt * 256:(kt + 1) * 256] = blk
    assert np.array_equal(full[:n, :k], codes)
    assert not full[n:].any() and not full[:, k:].any()
    sc = packed[nrt * nkt * 4096:].view(np.float32)
    assert np.array_equal(sc[:n], scales) and not sc[n:].any()


def test_fp8_head_argument_errors(lib):
    assert nv.fp8_packed_bytes(0, 16) == 0 and nv.fp8_packed_bytes(4, 24) == 0
    assert nv.fp8_packed_bytes(1, 16) == 4096 + 64
    assert lib.nvfp4v_fp8_head_gemm(None, None, 1, 16, None, 1, None, None) == nv.E_INVALID_ARG
    assert lib.nvfp4v_fp8_head_gemm_pa(None, None, 1, 16, None, 1, None, None) == nv.E_INVALID_ARG
    with pytest.raises(nv.Nvfp4vError):
        nv.fp8_pack_host(np.zeros((2, 24), np.uint8), np.zeros(2, np.float32))
