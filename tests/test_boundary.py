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
    for code in range(0, -12, -1):
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


_KEEP = []


class FakeCtx:
    """A zeroed host block of the full size of struct nvfp4v_ctx (empty
    workspace, no device buffers) with its CU count set to 256: every call made
    with it must return from its host-side checks, before any HIP call. Kept
    alive for the whole module."""

    def __init__(self):
        size = int(nv.load().nvfp4v_ctx_size())
        assert size >= 64
        self.buf = ctypes.create_string_buffer(size)  # zero-filled
        # leading fields of the struct: int device, int num_cus
        ctypes.c_int.from_buffer(self.buf, 4).value = 256
        self.ptr = ctypes.cast(self.buf, ctypes.c_void_p)
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
    assert f(ctx, a, 129, 256, w, 512, 1.0, c, None) == nv.E_M_RANGE
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
    assert lib.nvfp4v_create(ctypes.byref(out), 0, None) == nv.E_FAULT
    assert lib.nvfp4v_pack(ctx, fake_dev(), fake_dev(), 16, 128, fake_dev(0x40000), None) == nv.E_FAULT
    assert lib.nvfp4v_quantize(ctx, fake_dev(), 16, 128, fake_dev(), fake_dev(), None) == nv.E_FAULT
    assert lib.nvfp4v_staircase(ctx, 16, 128, 1, 2, 0, 1, 0, fake_dev()) == nv.E_FAULT


@host_only
def test_other_argument_errors(lib):
    ctx = FakeCtx().ptr
    assert lib.nvfp4v_create(None, 0, None) == nv.E_INVALID_ARG
    out = ctypes.c_void_p()
    assert lib.nvfp4v_create(ctypes.byref(out), -1, None) == nv.E_INVALID_ARG
    assert lib.nvfp4v_pack(ctx, fake_dev(), fake_dev(), 16, 100, fake_dev(), None) == nv.E_SHAPE
    assert lib.nvfp4v_pack(ctx, fake_dev(), fake_dev(), 16, 128, fake_dev(0x1001), None) == nv.E_ALIGN
    assert lib.nvfp4v_unpack(ctx, fake_dev(0x1004), 16, 128, fake_dev(), fake_dev(), None) == nv.E_ALIGN
    assert lib.nvfp4v_quantize(ctx, fake_dev(), 16, 24, fake_dev(), fake_dev(), None) == nv.E_SHAPE
    us = (ctypes.c_double * 4)()
    assert lib.nvfp4v_staircase(ctx, 16, 128, 0, 2, 0, 1, 0, us) == nv.E_M_RANGE
    assert lib.nvfp4v_staircase(ctx, 16, 128, 3, 2, 0, 1, 0, us) == nv.E_M_RANGE
    assert lib.nvfp4v_staircase(ctx, 16, 128, 1, 129, 0, 1, 0, us) == nv.E_M_RANGE
    assert lib.nvfp4v_staircase(ctx, 16, 128, 1, 2, 0, 0, 0, us) == nv.E_INVALID_ARG
    buf = ctypes.create_string_buffer(8)
    assert lib.nvfp4v_describe_plan(ctx, 16, 128, 0, buf, 8) == nv.E_M_RANGE
    assert lib.nvfp4v_device_status(None) == nv.E_INVALID_ARG
    n = ctypes.c_uint64(0)
    assert lib.nvfp4v_f16_redone(None, ctypes.byref(n)) == nv.E_INVALID_ARG
    assert lib.nvfp4v_f16_redone(ctx, None) == nv.E_INVALID_ARG
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


TABLE_PATH = os.path.join(os.path.dirname(nv.__file__), "tables", "gfx950.txt")


def plan(lib, ctx, n, k, m):
    buf = ctypes.create_string_buffer(256)
    assert lib.nvfp4v_describe_plan(ctx, n, k, m, buf, 256) == nv.OK
    return buf.value.decode()


def test_tile_table_file_changes_the_plan(lib, tmp_path):
    """A table file loaded into a context changes its plans for the GEMMs its
    rules hold and leaves the others on the built-in table; NULL goes back."""
    ctx = FakeCtx().ptr
    base_o, base_down = plan(lib, ctx, 5120, 5120, 16), plan(lib, ctx, 5120, 17408, 16)
    assert "r=2 " in base_o and "ksplit=1" in base_o
    f = tmp_path / "o_only.txt"
    f.write_text("arch gfx950\n# o at 9..16 rows on one R = 8 work-group per 8 row tiles, 2 K pieces\n"
                 "rule 300 330 10 30 9 16 reg 8 2\n")
    assert lib.nvfp4v_load_tile_table(ctx, str(f).encode()) == nv.OK
    got = plan(lib, ctx, 5120, 5120, 16)
    assert "r=8 " in got and "ksplit=2" in got and got != base_o
    assert plan(lib, ctx, 5120, 5120, 8) == plan(lib, FakeCtx().ptr, 5120, 5120, 8)  # M outside the rule
    assert plan(lib, ctx, 5120, 17408, 16) == base_down  # another shape
    assert lib.nvfp4v_load_tile_table(ctx, None) == nv.OK
    assert plan(lib, ctx, 5120, 5120, 16) == base_o


def test_checked_in_table_is_the_built_in_one(lib):
    """Loading tables/gfx950.txt (the file the build compiles in) changes no plan."""
    ctx, ref = FakeCtx().ptr, FakeCtx().ptr
    assert lib.nvfp4v_load_tile_table(ctx, TABLE_PATH.encode()) == nv.OK
    for n, k in ((151936, 5120), (15360, 5120), (5120, 5120), (34816, 5120), (5120, 17408), (17408, 5120),
                 (512, 256), (10240, 5120)):
        for m in (1, 8, 9, 16, 17, 32, 33, 48, 49, 64):
            assert plan(lib, ctx, n, k, m) == plan(lib, ref, n, k, m), (n, k, m)


@pytest.mark.parametrize("text", [
    "rule 1 * 1 * 1 64 reg 2 1\n",                    # no arch line
    "arch gfx942\nrule 1 * 1 * 1 64 reg 2 1\n",       # another arch
    "arch gfx950\nrule 1 * 1 * 1 64 wmma 2 1\n",      # unknown kernel
    "arch gfx950\nrule 1 * 1 * 1 64 reg 3 1\n",       # R with no kernel
    "arch gfx950\nrule 1 * 1 * 1 64 lds 2 1\n",       # lds R = 2 is built up to 32 rows only
    "arch gfx950\nrule 1 * 1 * 1 65 reg 2 1\n",       # more than 64 rows in a register-variant launch
    "arch gfx950\nrule 1 * 1 * 65 129 wide 2 1\n",    # M beyond the API's range
    "arch gfx950\nrule 1 * 1 * 1 32 wide 2 1\n",      # the wide unit is built from 33 rows
    "arch gfx950\nrule 5 4 1 * 1 64 reg 2 1\n",       # empty range
    "arch gfx950\nrule 1 * 1 * 1 64 reg 2 0\n",       # no K split
    "arch gfx950\nrule 1 * 1 * 1 64 reg 2\n",         # missing field
    "arch gfx950\nrule 1 * 1 * x 64 reg 2 1\n",       # not a number
    "arch gfx950\n" + "rule 1 * 1 * 1 64 reg 2 1\n" * 65,  # too many rules
], ids=["no-arch", "arch", "kernel", "r", "lds-r", "m", "wide-m", "wide-lo", "range", "ks", "fields", "number",
        "count"])
def test_bad_tile_table_is_refused(lib, tmp_path, text):
    ctx = FakeCtx().ptr
    f = tmp_path / "bad.txt"
    f.write_text(text)
    before = plan(lib, ctx, 5120, 5120, 16)
    assert lib.nvfp4v_load_tile_table(ctx, str(f).encode()) == nv.E_TABLE
    assert plan(lib, ctx, 5120, 5120, 16) == before  # the previous table stays
    out = ctypes.c_void_p()
    assert lib.nvfp4v_create(ctypes.byref(out), 0, str(f).encode()) == nv.E_TABLE
    assert not out.value


def test_wide_rows_in_one_launch(lib, tmp_path):
    """Above 64 rows the built-in table gives gate or up alone (1088 row tiles)
    and gate|up fused (2176) one launch of the wide unit, and every other shape
    one launch per block of 64 rows; a table file can move a shape to the wide
    unit."""
    ctx = FakeCtx().ptr
    for m in (65, 100, 128):
        assert "wide-m" in plan(lib, ctx, 17408, 5120, m) and "launches" not in plan(lib, ctx, 17408, 5120, m)
        assert "wide-m" in plan(lib, ctx, 34816, 5120, m) and "ksplit=1" in plan(lib, ctx, 34816, 5120, m)
        assert "launches=2 (64-row blocks)" in plan(lib, ctx, 5120, 17408, m)
        assert "launches=2 (64-row blocks)" in plan(lib, ctx, 5120, 5120, m)
    assert "wide-m" not in plan(lib, ctx, 17408, 5120, 64)
    f = tmp_path / "down_wide.txt"
    f.write_text("arch gfx950\nrule 300 330 60 70 65 128 wide 2 4\n")
    assert lib.nvfp4v_load_tile_table(ctx, str(f).encode()) == nv.OK
    got = plan(lib, ctx, 5120, 17408, 100)
    assert "wide-m" in got and "mblocks=7" in got and "ksplit=4" in got and "launches" not in got


def test_missing_tile_table_file(lib, tmp_path):
    ctx = FakeCtx().ptr
    assert lib.nvfp4v_load_tile_table(ctx, str(tmp_path / "none.txt").encode()) == nv.E_TABLE
    assert lib.nvfp4v_load_tile_table(None, None) == nv.E_INVALID_ARG


def test_pass_modes():
    """Two schedules, chain (0, the default) and persistent (1); any other mode
    is rejected and leaves the context's mode unchanged."""
    lib = nv.load()
    ctx = FakeCtx().ptr
    assert lib.nvfp4v_get_pass_mode(ctx) == nv.PASS_CHAIN
    assert lib.nvfp4v_set_pass_mode(ctx, nv.PASS_PERSISTENT) == nv.OK
    assert lib.nvfp4v_get_pass_mode(ctx) == nv.PASS_PERSISTENT
    for bad in (-1, 2, 3, 99):
        assert lib.nvfp4v_set_pass_mode(ctx, bad) == nv.E_INVALID_ARG
        assert lib.nvfp4v_get_pass_mode(ctx) == nv.PASS_PERSISTENT
    assert lib.nvfp4v_set_pass_mode(None, nv.PASS_CHAIN) == nv.E_INVALID_ARG


@host_only
def test_tree_attention_host_checks():
    """Tree-verify attention: shape, range, tree and alignment checks return
    before anything reaches the GPU."""
    lib = nv.load()
    ctx = FakeCtx().ptr
    dev = fake_dev()
    par = np.array([-1, 0, 1, 1], np.int32)
    pp = ctypes.c_void_p(par.ctypes.data)

    def call(m=4, ctx_len=10, hq=2, hkv=2, d=128, parent=pp, scale=0.1, cap=64, q=dev, o=dev, ws=dev):
        return lib.nvfp4v_tree_attention(ctx, q, dev, dev, cap, ctx_len, m, hq, hkv, d, parent, scale, o, ws,
                                         1 << 20, None)

    assert lib.nvfp4v_tree_attention(None, dev, dev, dev, 64, 10, 4, 2, 2, 128, pp, 0.1, dev, dev, 1 << 20,
                                     None) == nv.E_INVALID_ARG
    assert call(q=None) == nv.E_INVALID_ARG
    assert call(parent=None) == nv.E_INVALID_ARG
    assert call(d=64) == nv.E_SHAPE
    assert call(hq=3) == nv.E_SHAPE
    assert call(hq=130, hkv=65) == nv.E_SHAPE
    assert call(ctx_len=61) == nv.E_SHAPE
    assert call(cap=48) == nv.E_SHAPE
    assert call(m=0) == nv.E_M_RANGE
    assert call(m=33) == nv.E_M_RANGE
    assert call(hq=16, hkv=2, m=5) == nv.E_M_RANGE
    bad = np.array([-1, 0, 2, 1], np.int32)  # row 2 is its own parent
    assert call(parent=ctypes.c_void_p(bad.ctypes.data)) == nv.E_INVALID_ARG
    bad0 = np.array([0, 0, 1, 1], np.int32)
    assert call(parent=ctypes.c_void_p(bad0.ctypes.data)) == nv.E_INVALID_ARG
    assert call(scale=float("inf")) == nv.E_INVALID_ARG
    assert call(o=fake_dev(0x1004)) == nv.E_ALIGN


def test_attention_sizes():
    # caches: cap * Hkv * 128 bf16 each
    assert nv.kv_cache_bytes(64, 40) == 64 * 40 * 128 * 2
    assert nv.kv_cache_bytes(48, 40) == 0 and nv.kv_cache_bytes(64, 40, 64) == 0 and nv.kv_cache_bytes(0, 1) == 0
    # workspace: 1024 bytes of tickets + one record per (head, chunk) and 16
    # query columns, at most one chunk per 352 positions and 64 chunks per head
    one = nv.tree_attention_workspace_bytes(100, 16, 40, 40)
    rec1 = (16 * 2 + 8 * 64 * 4) * 4  # one 16-column block
    assert one == 1024 + 40 * 1 * rec1
    assert nv.tree_attention_workspace_bytes(32768, 16, 40, 40) == 1024 + 40 * 64 * rec1
    rec2 = (32 * 2 + 2 * 8 * 64 * 4) * 4
    assert rec2 == 2 * rec1  # two blocks in one record, or two work-groups' records
    assert nv.tree_attention_workspace_bytes(1000, 17, 40, 40) == 1024 + 40 * 3 * rec2  # 1017 positions
    assert nv.tree_attention_workspace_bytes(10, 33, 40, 40) == 0
    assert nv.tree_attention_workspace_bytes(10, 4, 40, 40, 64) == 0


@host_only
def test_kv_write_host_checks():
    lib = nv.load()
    ctx = FakeCtx().ptr
    dev = fake_dev()

    def call(n=4, pos0=0, hkv=2, d=128, cap=64, k=dev):
        return lib.nvfp4v_kv_write(ctx, k, dev, n, pos0, hkv, d, cap, dev, dev, None)

    assert lib.nvfp4v_kv_write(None, dev, dev, 4, 0, 2, 128, 64, dev, dev, None) == nv.E_INVALID_ARG
    assert call(k=None) == nv.E_INVALID_ARG
    assert call(d=64) == nv.E_SHAPE
    assert call(hkv=0) == nv.E_SHAPE
    assert call(cap=40) == nv.E_SHAPE
    assert call(n=0) == nv.E_SHAPE
    assert call(pos0=61) == nv.E_SHAPE
    assert call(k=fake_dev(0x1008)) == nv.E_ALIGN
