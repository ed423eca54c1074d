"""Tree-verify attention on the GPU against the oracle (fp64), element by
element within the tolerance the oracle derives (oracle.attention.within_tolerance),
through the C ABI; caches written by nvfp4v_kv_write over slots pre-filled with
NaN bit patterns (so a read past the last position would show)."""

import math

import numpy as np
import pytest

import nvfp4_skinny_gemm_amd as nv
import synth
from oracle import attention as att

pytestmark = pytest.mark.gpu


def log(msg):
    print("[attn] " + msg, flush=True)


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


def dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def build_cache(torch, ctx, k, v, ctx_len, m, cap):
    """Caches of `cap` positions, NaN everywhere, then the context rows and the
    tree rows written by two kv_write calls."""
    hkv, P, d = k.shape
    nbytes = nv.kv_cache_bytes(cap, hkv, d)
    kc = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    vc = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    rows_k = dev_bf16(torch, np.transpose(k, (1, 0, 2)))  # [P][hkv][d]
    rows_v = dev_bf16(torch, np.transpose(v, (1, 0, 2)))
    if ctx_len > 0:
        ctx.kv_write(rows_k[:ctx_len].contiguous(), rows_v[:ctx_len].contiguous(), 0, cap, kc, vc)
    ctx.kv_write(rows_k[ctx_len:].contiguous(), rows_v[ctx_len:].contiguous(), ctx_len, cap, kc, vc)
    return kc, vc


def run_case(torch, ctx, ctx_len, m, hq, hkv, shape, seed, heads=None, cap_extra=0):
    q, k, v = synth.attention_inputs(m, hq, hkv, ctx_len, seed=seed)
    parent = synth.tree_parent_rows(m, seed=seed, shape=shape)
    cap = (ctx_len + m + 31) // 32 * 32 + cap_extra
    log("T=%d M=%d Hq=%d Hkv=%d tree=%s cap=%d plan=%s" % (ctx_len, m, hq, hkv, shape, cap,
                                                           ctx.tree_attention_plan(ctx_len, m, hq, hkv)))
    kc, vc = build_cache(torch, ctx, k, v, ctx_len, m, cap)
    scale = 1.0 / math.sqrt(128)
    o1 = ctx.tree_attention(dev_bf16(torch, q), kc, vc, cap, ctx_len, hkv, parent, scale=scale)
    o2 = ctx.tree_attention(dev_bf16(torch, q), kc, vc, cap, ctx_len, hkv, parent, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), "not bitwise reproducible"
    o = o1.cpu().numpy()
    assert np.isfinite(o).all()
    group = hq // hkv
    if heads is None:
        heads = list(range(hkv))
    qh = [kv * group + gq for kv in heads for gq in range(group)]
    ref, a, e = att.tree_attention(q[:, qh], k[heads], v[heads], parent, ctx_len, scale)
    ok = att.within_tolerance(o[:, qh], ref, a, e)
    err = np.abs(o[:, qh] - ref) / (a + 1e-30)
    log("  worst |err| / A = %.3g (tolerance floor 2e-5)" % err.max())
    assert ok.all(), "%d of %d outputs outside tolerance; worst |err|/A %.3g" % ((~ok).sum(), ok.size, err.max())
    return o


CASES = [
    # (ctx_len, M, Hq, Hkv, tree)
    (0, 1, 4, 4, "chain"),      # the root alone: O = its own value
    (0, 8, 4, 4, "random"),     # tree only: the mask decides everything
    (1, 5, 2, 2, "wide"),
    (31, 16, 4, 4, "random"),   # one chunk, ragged group
    (200, 17, 2, 2, "random"),  # two column blocks
    (1000, 32, 4, 4, "random"),
    (999, 7, 8, 2, "random"),   # grouped query heads: 4 per key/value head, 28 columns
    (4101, 16, 2, 1, "chain"),  # 2 query heads on one key/value head, 32 columns, many chunks
    (333, 24, 1, 1, "wide"),
]


@pytest.mark.parametrize("case", CASES, ids=["T%d-M%d-%dx%d-%s" % c for c in CASES])
def test_tree_attention_against_oracle(torch_cuda, ctx, case):
    ctx_len, m, hq, hkv, shape = case
    run_case(torch_cuda, ctx, ctx_len, m, hq, hkv, shape, seed=sum(case[:4]), cap_extra=64 if m == 7 else 0)


@pytest.mark.parametrize("ctx_len,m", [(1024, 16), (1024, 32), (32768, 16), (32768, 32)])
def test_full_size_heads_sampled(torch_cuda, ctx, ctx_len, m):
    """40 heads of 128 (the stand-in layer's q, k and v of 5120 each) at 1k and
    32k of context; the oracle checks heads 0, 17 and 39."""
    run_case(torch_cuda, ctx, ctx_len, m, 40, 40, "random", seed=m, heads=[0, 17, 39])


def test_sibling_rows_do_not_see_each_other(torch_cuda, ctx):
    """Without context, a star tree's leaves see only the root and themselves:
    changing one leaf's key and value leaves every other row's output bitwise
    unchanged."""
    torch = torch_cuda
    m, hq, hkv = 6, 2, 2
    q, k, v = synth.attention_inputs(m, hq, hkv, 0, seed=11)
    parent = np.array([-1, 0, 0, 0, 0, 0], np.int32)
    outs = []
    for variant in range(2):
        k2, v2 = k.copy(), v.copy()
        if variant:
            k2[:, 3] ^= 0x0101
            v2[:, 3] ^= 0x0101
        kc, vc = build_cache(torch, ctx, k2, v2, 0, m, 32)
        outs.append(ctx.tree_attention(dev_bf16(torch, q), kc, vc, 32, 0, hkv, parent).cpu())
    for i in range(m):
        same = torch.equal(outs[0][i].view(torch.int32), outs[1][i].view(torch.int32))
        assert same == (i != 3), "row %d" % i


def test_graph_replay_equals_eager(torch_cuda, ctx):
    torch = torch_cuda
    ctx_len, m, hq, hkv = 700, 16, 8, 8
    q, k, v = synth.attention_inputs(m, hq, hkv, ctx_len, seed=5)
    parent = synth.tree_parent_rows(m, seed=5)
    cap = 736
    kc, vc = build_cache(torch, ctx, k, v, ctx_len, m, cap)
    qd = dev_bf16(torch, q)
    ws = torch.zeros(nv.tree_attention_workspace_bytes(ctx_len, m, hq, hkv), dtype=torch.uint8, device="cuda")
    eager = ctx.tree_attention(qd, kc, vc, cap, ctx_len, hkv, parent, ws=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ctx.tree_attention(qd, kc, vc, cap, ctx_len, hkv, parent, ws=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.tree_attention(qd, kc, vc, cap, ctx_len, hkv, parent, ws=ws, out=out)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), "replay %d" % rep


@pytest.mark.parametrize("case", [(1000, 32, 4, 4), (3000, 17, 40, 40), (5000, 24, 8, 8), (600, 8, 4, 1)],
                         ids=["T1000-M32", "T3000-M17-40h", "T5000-M24", "T600-grouped"])
def test_column_split_is_bitwise_neutral(torch_cuda, ctx, monkeypatch, case):
    """Two column blocks in one work-group, or one work-group per block (each
    then streams the chunk's keys and values itself, two groups in flight per
    wave): every column's scores, softmax and sums are computed in the same
    order, so at equal chunking O is bitwise the same; and it agrees with the
    oracle either way (the split also graph-replays)."""
    torch = torch_cuda
    ctx_len, m, hq, hkv = case
    q, k, v = synth.attention_inputs(m, hq, hkv, ctx_len, seed=11)
    parent = synth.tree_parent_rows(m, seed=11)
    cap = (ctx_len + m + 31) // 32 * 32
    kc, vc = build_cache(torch, ctx, k, v, ctx_len, m, cap)
    qd = dev_bf16(torch, q)
    # equal chunking both ways (within the workspace's bound of one chunk per 352 positions)
    monkeypatch.setenv("NVFP4V_ATTN_CHUNKS", str(min(3, -(-(ctx_len + m) // 352))))
    outs = []
    for split in ("0", "1"):
        monkeypatch.setenv("NVFP4V_ATTN_SPLIT", split)
        ws = torch.zeros(nv.tree_attention_workspace_bytes(ctx_len, m, hq, hkv), dtype=torch.uint8, device="cuda")
        outs.append(ctx.tree_attention(qd, kc, vc, cap, ctx_len, hkv, parent, scale=1.0 / math.sqrt(128), ws=ws))
        torch.cuda.synchronize()
        if split == "1":
            out = torch.empty_like(outs[-1])
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                ctx.tree_attention(qd, kc, vc, cap, ctx_len, hkv, parent, scale=1.0 / math.sqrt(128), ws=ws,
                                   out=out)
            for rep in range(2):
                out.zero_()
                g.replay()
                torch.cuda.synchronize()
                assert torch.equal(out.view(torch.int32), outs[-1].view(torch.int32)), "replay %d" % rep
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    o_ref, o_abs, o_e = att.tree_attention(q, k, v, parent, ctx_len, 1.0 / math.sqrt(128))
    ok = att.within_tolerance(outs[1].cpu().numpy(), o_ref, o_abs, o_e)
    assert ok.all(), "%d of %d outside the tolerance" % ((~ok).sum(), ok.size)


def test_argument_errors(torch_cuda, ctx):
    import ctypes

    torch = torch_cuda
    lib = nv.load()
    cap, hq, hkv, m = 64, 2, 2, 4
    q = torch.zeros((m, hq, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(nv.kv_cache_bytes(cap, hkv), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    o = torch.empty((m, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros(nv.tree_attention_workspace_bytes(10, m, hq, hkv), dtype=torch.uint8, device="cuda")
    par = np.array([-1, 0, 1, 1], np.int32)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def call(m_=m, ctx_len=10, hq_=hq, hkv_=hkv, d=128, parent=par, scale=0.1, ws_bytes=None, cap_=cap, qp=None):
        wb = ws.numel() if ws_bytes is None else ws_bytes
        return lib.nvfp4v_tree_attention(ctx._h, qp if qp is not None else P(q), P(kc), P(vc), cap_, ctx_len, m_, hq_,
                                         hkv_, d, ctypes.c_void_p(parent.ctypes.data), scale, P(o), P(ws), wb, None)

    assert call() == nv.OK
    torch.cuda.synchronize()
    assert call(d=64) == nv.E_SHAPE
    assert call(hq_=3) == nv.E_SHAPE
    assert call(ctx_len=61) == nv.E_SHAPE          # ctx_len + m > cap
    assert call(cap_=48) == nv.E_SHAPE             # not a multiple of 32
    assert call(m_=33, parent=np.array([-1] + [0] * 32, np.int32)) == nv.E_M_RANGE
    # 8 query heads per key/value head x 5 rows = 40 query columns > 32
    assert call(m_=5, hq_=16, hkv_=2, parent=np.array([-1, 0, 0, 0, 0], np.int32)) == nv.E_M_RANGE
    assert call(parent=np.array([0, 0, 1, 1], np.int32)) == nv.E_INVALID_ARG
    assert call(parent=np.array([-1, 0, 3, 1], np.int32)) == nv.E_INVALID_ARG
    assert call(scale=float("nan")) == nv.E_INVALID_ARG
    assert call(ws_bytes=100) == nv.E_WORKSPACE
    assert call(qp=ctypes.c_void_p(q.data_ptr() + 2)) == nv.E_ALIGN
    torch.cuda.synchronize()

