"""The chained verify pass on the GPU.

Only layer 0's GEMMs see inputs drawn by the generator, so the oracle checks
those directly. Deeper layers are checked by properties that hold at any size:
- the pass equals the composition of single verify_gemm / glue calls, bitwise;
- graph replays equal the eager pass, bitwise;
- every glue kernel equals the oracle's glue, bitwise, on generator inputs;
- activations stay finite with an O(1) RMS through the 64-layer stack.
"""

import math
import sys

import numpy as np
import pytest

import nvfp4_skinny_gemm_amd as nv
import synth
from conftest import f16_copy_expected

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


def f32(x):
    return float(np.float32(x))


def test_glue_kernels_match_oracle(torch_cuda, ctx, oracle_mod):
    torch = torch_cuda
    g = np.random.default_rng(11)
    x = (g.standard_normal((16, 3 * 512)) * 40).astype(np.float32)
    y = (g.standard_normal((16, 3 * 512)) * 40).astype(np.float32)
    xd, yd = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
    c = f32(1 / math.sqrt(5120))
    got = ctx.glue_scale(xd[:, 1024:], c).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle_mod.glue_scale(x[:, 1024:], c))
    c2 = f32(1 / math.sqrt(2 * 5120))
    got = ctx.glue_sum(xd[:, :512], yd[:, 512:1024], c2).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle_mod.glue_sum(x[:, :512], y[:, 512:1024], c2))


def small_stack(torch, ctx, layers, H, I, seed=0):
    packed = []
    for l in range(layers):
        mats = {}
        for name, parts, n, k in (("qkv", ("q", "k", "v"), 3 * H, H), ("o", ("o",), H, H),
                                  ("gate_up", ("gate", "up"), 2 * I, H), ("down", ("down",), H, I)):
            w = torch.cat([synth.weights_f32_cuda(n // len(parts), k, seed=seed,
                                                  stream="t%d/%s" % (l, p)) for p in parts])
            if name == "gate_up":  # gate and up interleaved in 16-row tiles
                w = torch.stack([w[: n // 2].reshape(n // 32, 16, k), w[n // 2:].reshape(n // 32, 16, k)],
                                dim=1).reshape(n, k)
            codes, scales = ctx.quantize(w)
            mats[name] = ctx.pack(codes, scales, n, k)
        packed.append(mats)
    arr = (nv.Layer * layers)()
    for l, m in enumerate(packed):
        arr[l] = nv.Layer(m["qkv"].data_ptr(), m["o"].data_ptr(), m["gate_up"].data_ptr(),
                          m["down"].data_ptr(), 1.0, 1.0, 1.0, 1.0)
    return packed, arr


def manual_chain(torch, ctx, packed, h0, H, I):
    c_h, c_i, c_2 = f32(1 / math.sqrt(H)), f32(1 / math.sqrt(I)), f32(1 / math.sqrt(2 * H))
    h = h0
    outs = []
    for mats in packed:
        qkv = ctx.verify_gemm(h, mats["qkv"], 3 * H, H)
        o = ctx.verify_gemm(ctx.glue_scale(qkv[:, 2 * H:], c_h), mats["o"], H, H)
        gu = ctx.verify_gemm(ctx.glue_scale(o, c_h), mats["gate_up"], 2 * I, H)
        t = gu.view(gu.shape[0], I // 16, 2, 16)  # plain GEMM output follows the interleaved rows
        gate, up = t[:, :, 0].reshape(-1, I).contiguous(), t[:, :, 1].reshape(-1, I).contiguous()
        d = ctx.verify_gemm(ctx.glue_sum(gate, up, c_2), mats["down"], H, I)
        h = ctx.glue_scale(d, c_i)
        outs.append(h)
    return outs


MODES = [pytest.param(nv.PASS_CHAIN, id="chain"), pytest.param(nv.PASS_PERSISTENT, id="persistent")]


@pytest.fixture
def mode_ctx(ctx, request):
    ctx.set_pass_mode(request.param)
    yield ctx
    ctx.set_pass_mode(nv.PASS_CHAIN)


@pytest.mark.parametrize("mode_ctx", MODES, indirect=True)
@pytest.mark.parametrize("m", [1, 8, 16, 33, 64, 65, 120, 128])
def test_pass_equals_composition(torch_cuda, mode_ctx, m):
    torch, ctx = torch_cuda, mode_ctx
    H, I, L = 256, 512, 3
    packed, arr = small_stack(torch, ctx, L, H, I)
    h0 = torch.from_numpy(synth.activations_bf16(128, H, seed=3).view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(m, H, I, L), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    trace = torch.empty((L, m, H), dtype=torch.bfloat16, device="cuda")
    ctx.verify_pass(arr, H, I, h0[:m], ws, h_out, trace=trace)
    assert ctx.pass_status() == nv.OK
    log("pass mode %d, grid %d work-groups" % (ctx.get_pass_mode(), ctx.last_pass_grid()))
    ref = manual_chain(torch, ctx, packed, h0[:m], H, I)
    for l in range(L):
        assert torch.equal(trace[l].view(torch.int16), ref[l].view(torch.int16)), "layer %d" % l
    assert torch.equal(h_out.view(torch.int16), ref[-1].view(torch.int16))
    # the workspace holds the last layer's fp32 outputs, q|k|v first, in one
    # region per block of 64 rows (each the size of a 64-row pass workspace)
    last = packed[-1]
    h_prev = ref[-2] if L > 1 else h0[:m]
    qkv = ctx.verify_gemm(h_prev, last["qkv"], 3 * H, H)
    region = nv.pass_workspace_bytes(64, H, I, L)
    for r0 in range(0, m, 64):
        mc = min(64, m - r0)
        base = (r0 // 64) * region
        got = ws[base:base + mc * 3 * H * 4].view(torch.float32).view(mc, 3 * H)
        assert torch.equal(got, qkv[r0:r0 + mc]), "rows %d.." % r0


@pytest.mark.parametrize("plan", ["n:r=1,ks=2", "n:r=2,ks=1"])
@pytest.mark.parametrize("m", [8, 24])
def test_chain_pass_with_lds_plans(torch_cuda, ctx, monkeypatch, plan, m):
    """The chained pass on the activations-in-LDS GEMM variant (fused scale and
    gate/up pair epilogues included) equals the composition of single calls."""
    torch = torch_cuda
    H, I, L = 512, 1024, 2
    monkeypatch.setenv("NVFP4V_PLAN", plan)
    packed, arr = small_stack(torch, ctx, L, H, I, seed=5)
    h0 = torch.from_numpy(synth.activations_bf16(64, H, seed=3).view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(m, H, I, L), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    trace = torch.empty((L, m, H), dtype=torch.bfloat16, device="cuda")
    ctx.verify_pass(arr, H, I, h0[:m], ws, h_out, trace=trace)
    ref = manual_chain(torch, ctx, packed, h0[:m], H, I)
    for l in range(L):
        assert torch.equal(trace[l].view(torch.int16), ref[l].view(torch.int16)), "layer %d" % l


@pytest.mark.parametrize("mode_ctx", MODES, indirect=True)
def test_pass_longer_than_one_launch(torch_cuda, mode_ctx):
    """40 layers: the persistent kernel runs 32 layers per launch, so the chain
    crosses a launch boundary; still bitwise the composition of single calls."""
    torch, ctx = torch_cuda, mode_ctx
    H, I, L, m = 256, 512, 40, 16
    packed, arr = small_stack(torch, ctx, L, H, I, seed=9)
    h0 = torch.from_numpy(synth.activations_bf16(64, H, seed=8).view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(m, H, I, L), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    trace = torch.empty((L, m, H), dtype=torch.bfloat16, device="cuda")
    ctx.verify_pass(arr, H, I, h0[:m], ws, h_out, trace=trace)
    assert ctx.pass_status() == nv.OK
    ref = manual_chain(torch, ctx, packed, h0[:m], H, I)
    for l in range(L):
        assert torch.equal(trace[l].view(torch.int16), ref[l].view(torch.int16)), "layer %d" % l
    assert torch.equal(h_out.view(torch.int16), ref[-1].view(torch.int16))


@pytest.mark.parametrize("mode_ctx", MODES, indirect=True)
def test_graph_replays_equal_eager(torch_cuda, mode_ctx):
    torch, ctx = torch_cuda, mode_ctx
    H, I, L, m = 512, 1024, 4, 16
    packed, arr = small_stack(torch, ctx, L, H, I, seed=1)
    h0 = torch.from_numpy(synth.activations_bf16(64, H, seed=4).view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(m, H, I, L), dtype=torch.uint8, device="cuda")
    eager = torch.zeros((m, H), dtype=torch.bfloat16, device="cuda")
    ctx.verify_pass(arr, H, I, h0[:m], ws, eager)
    torch.cuda.synchronize()
    assert ctx.pass_status() == nv.OK, "eager pass gave up at site %d" % ctx.pass_error_site()
    assert torch.isfinite(eager.float()).all() and eager.float().abs().sum() > 0
    out = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ctx.verify_pass(arr, H, I, h0[:m], ws, out)
    torch.cuda.current_stream().wait_stream(s)
    assert ctx.pass_status() == nv.OK, "side-stream pass gave up at site %d" % ctx.pass_error_site()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.verify_pass(arr, H, I, h0[:m], ws, out)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert ctx.pass_status() == nv.OK, "replay %d gave up at site %d" % (rep, ctx.pass_error_site())
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay %d" % rep
        # unrelated eager work between replays
        ctx.verify_gemm(h0[:m], packed[0]["qkv"], 3 * H, H)
        torch.cuda.synchronize()


@pytest.mark.parametrize("m", [8, 16, 24, 32, 100, 120])
def test_graph_replays_equal_eager_full_size(torch_cuda, ctx, m):
    """Full-size layers in the chained schedule, whose tile table splits K at
    these row counts (down at 8; gate|up and down at 16; down at 24 and 32) and
    exchanges the partial sums through one XCD's L2: graph replays equal the
    eager pass bitwise, with split eager GEMMs on the same context in between
    (they share the arrival counters), and no row block reports pieces on two
    XCDs. Above 64 rows the pass runs one 64-row block after the other."""
    torch = torch_cuda
    H, I, L = 5120, 17408, 2
    packed, arr = small_stack(torch, ctx, L, H, I, seed=3)
    h0 = torch.from_numpy(synth.activations_bf16(128, H, seed=8).view(np.int16)).cuda().view(torch.bfloat16)
    d_in = torch.from_numpy(synth.activations_bf16(128, I, seed=9).view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(m, H, I, L), dtype=torch.uint8, device="cuda")
    eager = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    ctx.verify_pass(arr, H, I, h0[:m], ws, eager)
    torch.cuda.synchronize()
    d_ref = ctx.verify_gemm(d_in[:m], packed[1]["down"], H, I).clone()
    log("M=%d down plan: %s" % (m, ctx.describe_plan(H, I, m)))
    out = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ctx.verify_pass(arr, H, I, h0[:m], ws, out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.verify_pass(arr, H, I, h0[:m], ws, out)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay %d" % rep
        d = ctx.verify_gemm(d_in[:m], packed[1]["down"], H, I)
        torch.cuda.synchronize()
        assert torch.equal(d.view(torch.int32), d_ref.view(torch.int32)), "eager down after replay %d" % rep
    assert ctx.device_status() == 0


def align256(x):
    return (x + 255) // 256 * 256


def act_packed_bytes(m, k):
    return ((k + 255) // 256) * ((m + 15) // 16) * 8 * 1024


def unpack_act(buf, m, k):
    """Packed activations (the layout the GEMM kernels read) -> bf16 bits [m, k]."""
    mb = (m + 15) // 16
    rows = np.arange(m)[:, None]
    ks = np.arange(k)[None, :]
    kt, rem = ks >> 8, ks & 255
    h, q, e = rem >> 6, (rem >> 3) & 7, rem & 7
    off = ((kt * mb + (rows >> 4)) * 8 + q) * 1024 + ((rows & 15) + 16 * h) * 16 + 2 * e
    return buf.view(np.uint16)[off // 2]


def workspace_views(ws, m, H, I, L):
    """fp32 outputs of the last layer and each layer's packed input blocks:
    (bf16 copy, fp16 copy) per block."""
    sizes = [m * 3 * H * 4, m * H * 4, m * 2 * I * 4, m * H * 4]
    C, off = [], 0
    for sz in sizes:
        C.append(ws[off:off + sz].view(np.float32))
        off += align256(sz)
    act_bytes = [act_packed_bytes(m, H)] * 3 + [act_packed_bytes(m, I)]
    stride = sum(2 * align256(b) for b in act_bytes)
    acts, acts16 = [], []
    for l in range(L + 1):
        blk, blk16, o = [], [], off + l * stride
        for b in act_bytes:
            blk.append(ws[o:o + b])
            blk16.append(ws[o + align256(b):o + align256(b) + b])
            o += 2 * align256(b)
        acts.append(blk)
        acts16.append(blk16)
    return C, acts, acts16


@pytest.mark.parametrize("mode_ctx", MODES, indirect=True)
@pytest.mark.parametrize("m", [1, 8, 9, 16, 24, 32])
def test_full_size_phases_against_oracle(torch_cuda, mode_ctx, oracle_mod, m):
    """Two full-size layers (H = 5120, I = 17408), at M in every regime of the
    tile table up to two row blocks (1..8, 9..16, 17..32). For the last layer, every
    GEMM's fp32 output is checked against the oracle on 384 sampled weight
    rows, fed with the packed activations the kernels read, taken back from
    the workspace; every glue step (and the hand-over between layers) is
    checked bitwise against the oracle's glue on the fp32 outputs."""
    torch, ctx = torch_cuda, mode_ctx
    log("full-size pass, mode %d, M = %d" % (ctx.get_pass_mode(), m))
    run_and_check_last_layer(torch, ctx, oracle_mod, m, 5120, 17408, 2, seed=2, sample=384)


def run_and_check_last_layer(torch, ctx, oracle_mod, m, H, I, L, seed, sample):
    """Run the pass and check the last layer: every GEMM's fp32 output against
    the oracle on `sample` weight rows (all rows if None), fed with the packed
    activations the kernels read, taken back from the workspace; every glue
    step and the hand-over between layers bitwise against the oracle's glue.
    Returns the trace."""
    packed, arr = small_stack(torch, ctx, L, H, I, seed=seed)
    a0 = synth.activations_bf16(64, H, seed=0, stream="pass/h0")
    h0 = torch.from_numpy(a0.view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(m, H, I, L), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    trace = torch.empty((L, m, H), dtype=torch.bfloat16, device="cuda")
    ctx.verify_pass(arr, H, I, h0[:m], ws, h_out, trace=trace)
    assert ctx.pass_status() == nv.OK, "pass gave up at site %d" % ctx.pass_error_site()
    torch.cuda.synchronize()
    assert torch.isfinite(trace.float()).all(), "non-finite activations in the pass"
    C, acts, acts16 = workspace_views(ws.cpu().numpy(), m, H, I, L)
    for j in range(4):
        assert np.isfinite(C[j]).all(), "non-finite fp32 output of GEMM %d" % j
    last = L - 1
    if ctx.get_pass_mode() == nv.PASS_CHAIN:
        # the chained launches compute from the fp16 copies the packing kernel
        # and the epilogues write beside the bf16 ones
        for l in range(L + 1):
            for j, kk in enumerate((H, H, H, I)):
                if l == L and j:
                    break
                assert np.array_equal(unpack_act(acts16[l][j], m, kk),
                                      f16_copy_expected(unpack_act(acts[l][j], m, kk))), (l, j)
    h_in = unpack_act(acts[last][0], m, H)
    assert np.array_equal(unpack_act(acts[0][0], m, H), a0[:m].view(np.uint16))
    if L > 1:
        assert np.array_equal(h_in, trace[last - 1].view(torch.int16).cpu().numpy().view(np.uint16))
    ins = [h_in, unpack_act(acts[last][1], m, H), unpack_act(acts[last][2], m, H),
           unpack_act(acts[last][3], m, I)]
    outs = [C[0].reshape(m, 3 * H), C[1].reshape(m, H), C[2].reshape(m, 2 * I), C[3].reshape(m, H)]
    # glue: o_in, g_in, d_in and the layer's output h
    c_h, c_i, c_2 = f32(1 / math.sqrt(H)), f32(1 / math.sqrt(I)), f32(1 / math.sqrt(2 * H))
    assert np.array_equal(ins[1], oracle_mod.glue_scale(np.ascontiguousarray(outs[0][:, 2 * H:]), c_h))
    assert np.array_equal(ins[2], oracle_mod.glue_scale(outs[1], c_h))
    assert np.array_equal(ins[3], oracle_mod.glue_sum(np.ascontiguousarray(outs[2][:, :I]),
                                                      np.ascontiguousarray(outs[2][:, I:]), c_2))
    hq = h_out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(hq, oracle_mod.glue_scale(outs[3], c_i))
    # GEMMs: (sampled) rows of each projection against the oracle
    rng = np.random.default_rng(17)
    mats = [("qkv", ("q", "k", "v"), H, H), ("o", ("o",), H, H), ("gate_up", ("gate", "up"), I, H),
            ("down", ("down",), H, I)]
    for j, (name, parts, n_part, k) in enumerate(mats):
        n = n_part * len(parts)
        rows = np.arange(n) if sample is None else np.sort(rng.choice(n, sample, replace=False))
        w_rows = np.empty((len(rows), k), np.float32)
        for pi, part in enumerate(parts):
            sel = (rows // n_part) == pi
            if not sel.any():
                continue
            w = synth.weights_f32_cuda(n_part, k, seed=seed, stream="t%d/%s" % (last, part))
            w_rows[sel] = w[torch.from_numpy(rows[sel] % n_part).cuda()].cpu().numpy()
            del w
        oc, osc = oracle_mod.quantize(w_rows)
        c_ref, s_ref = oracle_mod.gemm(ins[j], oc, osc)
        ok = oracle_mod.within_tolerance(outs[j][:, rows], c_ref, s_ref)
        assert ok.all(), "%s: %d of %d checked outputs outside 1e-5*S" % (name, (~ok).sum(), ok.size)
    return trace


@pytest.mark.parametrize("mode_ctx", MODES, indirect=True)
@pytest.mark.parametrize("shape", [(256, 512, 3), (2048, 8192, 2), (1040, 2064, 2), (3072, 5120, 2)],
                         ids=["tiny", "split-pieces", "ragged", "leftover-units"])
@pytest.mark.parametrize("m", [1, 8, 16, 17, 32])
def test_cut_pass_against_oracle(torch_cuda, mode_ctx, oracle_mod, shape, m):
    """Both schedules: the last layer's GEMMs (every row) against the oracle and
    its glue bitwise. "tiny" leaves most work-groups without work,
    "split-pieces" spreads row blocks over several work-groups (partial sums in
    k order), "ragged" has row tiles and k-tiles that do not fill a row block
    or a k-tile, "leftover-units" has row counts that are not a multiple of
    four row tiles. The same pass again is bitwise identical."""
    torch, ctx = torch_cuda, mode_ctx
    H, I, L = shape
    log("pass mode %d H=%d I=%d L=%d M=%d" % (ctx.get_pass_mode(), H, I, L, m))
    t1 = run_and_check_last_layer(torch, ctx, oracle_mod, m, H, I, L, seed=4, sample=None)
    t2 = run_and_check_last_layer(torch, ctx, oracle_mod, m, H, I, L, seed=4, sample=64)
    assert torch.equal(t1.view(torch.int16), t2.view(torch.int16)), "pass not deterministic"


@pytest.mark.parametrize("mode_ctx", MODES, indirect=True)
def test_ragged_k_pass_against_oracle(torch_cuda, mode_ctx, oracle_mod):
    """H and I not multiples of the 256-wide k-tile: the padding of every
    activation block is zeroed before the pass (stale workspace bytes would
    otherwise meet the zero padding weights as 0 x NaN)."""
    torch, ctx = torch_cuda, mode_ctx
    for m in (1, 16):
        run_and_check_last_layer(torch, ctx, oracle_mod, m, 1040, 2064, 2, seed=6, sample=None)


@pytest.mark.parametrize("mode_ctx", MODES, indirect=True)
@pytest.mark.parametrize("m", [16, 32])
def test_cut_pass_longer_than_one_launch(torch_cuda, mode_ctx, oracle_mod, m):
    """40 layers: two persistent launches (32 + 8 layers); the last layer is
    checked against the oracle and the whole trace is deterministic."""
    torch, ctx = torch_cuda, mode_ctx
    t1 = run_and_check_last_layer(torch, ctx, oracle_mod, m, 256, 512, 40, seed=9, sample=None)
    t2 = run_and_check_last_layer(torch, ctx, oracle_mod, m, 256, 512, 40, seed=9, sample=None)
    assert torch.equal(t1.view(torch.int16), t2.view(torch.int16))
    assert torch.isfinite(t1.float()).all()


@pytest.mark.parametrize("mode_ctx", MODES, indirect=True)
def test_cut_pass_large_m_falls_back(torch_cuda, mode_ctx):
    """M > 32 in the persistent mode runs the chained launches: bitwise the
    composition."""
    torch, ctx = torch_cuda, mode_ctx
    H, I, L, m = 256, 512, 2, 40
    packed, arr = small_stack(torch, ctx, L, H, I)
    h0 = torch.from_numpy(synth.activations_bf16(64, H, seed=3).view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(m, H, I, L), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    ctx.verify_pass(arr, H, I, h0[:m], ws, h_out)
    ref = manual_chain(torch, ctx, packed, h0[:m], H, I)
    assert torch.equal(h_out.view(torch.int16), ref[-1].view(torch.int16))


@pytest.mark.parametrize("mode_ctx", MODES, indirect=True)
def test_full_stack_stays_finite_and_bounded(torch_cuda, mode_ctx):
    """64 layers at full size, M = 16: the linear glue keeps the RMS O(1)."""
    torch, ctx = torch_cuda, mode_ctx
    H, I, L, m = 5120, 17408, 64, 16
    log("building 64-layer stack")
    packed, arr = small_stack(torch, ctx, L, H, I, seed=7)
    h0 = torch.from_numpy(synth.activations_bf16(64, H, seed=0, stream="pass/h0").view(np.int16)).cuda()
    h0 = h0.view(torch.bfloat16)
    ws = torch.empty(nv.pass_workspace_bytes(m, H, I, L), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    trace = torch.empty((L, m, H), dtype=torch.bfloat16, device="cuda")
    ctx.verify_pass(arr, H, I, h0[:m], ws, h_out, trace=trace)
    torch.cuda.synchronize()
    t = trace.float()
    assert torch.isfinite(t).all()
    rms = t.pow(2).mean(dim=(1, 2)).sqrt().cpu().numpy()
    log("rms by layer: first %.3f last %.3f max %.3f" % (rms[0], rms[-1], rms.max()))
    assert rms.max() < 8.0 and rms.min() > 0.125


@pytest.mark.parametrize("m", [12, 40])
def test_padding_rows_leave_the_fp16_path(torch_cuda, ctx, m):
    """The staged GEMM variants (activations through LDS) read whole 16-row
    blocks, so the rows beyond M hold whatever the workspace held. With NaN
    bit patterns there (a workspace filled with 0xFF) the pass gives the same
    h as on a zeroed workspace, bitwise, and no unit falls back to the bf16
    copy unless the activations themselves carry a marker (M = 12: gate|up
    and down staged; M = 40: o staged, three row blocks)."""
    torch = torch_cuda
    H, I, L = 5120, 17408, 2
    packed, arr = small_stack(torch, ctx, L, H, I, seed=4)
    a0 = synth.activations_bf16(64, H, seed=0, stream="pass/h0")
    h0 = torch.from_numpy(a0.view(np.int16)).cuda().view(torch.bfloat16)
    outs, redone = [], []
    for fill in (0x00, 0xFF):
        ws = torch.full((nv.pass_workspace_bytes(m, H, I, L),), fill, dtype=torch.uint8, device="cuda")
        h_out = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
        before = ctx.f16_redone()
        ctx.verify_pass(arr, H, I, h0[:m], ws, h_out)
        redone.append(ctx.f16_redone() - before)
        outs.append(h_out.view(torch.int16).cpu().numpy())
        C, acts, acts16 = workspace_views(ws.cpu().numpy(), m, H, I, L)
        markers = sum(int((unpack_act(acts16[l][j], m, kk) == 0x7FFF).sum())
                      for l in range(L) for j, kk in enumerate((H, H, H, I)))
        log("M=%d fill 0x%02X: %d units recomputed, %d markers" % (m, fill, redone[-1], markers))
        if markers == 0:
            assert redone[-1] == 0, (m, fill, redone[-1])
    assert np.array_equal(outs[0], outs[1]), m


@pytest.mark.parametrize("m", [8, 24, 40])
def test_pass_with_markers_equals_composition(torch_cuda, ctx, m):
    """Values of h0 outside the fp16 copy's exact range (tiny, large, bf16
    subnormal) become markers in the first layer's input; its launches then
    test their sums and compute those units again from the bf16 copy. The
    pass still equals the composition of single calls bitwise, run after run
    (the marker words are cleared between passes), and a following pass
    without markers recomputes nothing."""
    torch = torch_cuda
    H, I, L = 256, 512, 3
    packed, arr = small_stack(torch, ctx, L, H, I)
    base = synth.activations_bf16(128, H, seed=3)
    marked = base.copy()
    g = np.random.default_rng(m)
    specials = (np.array([1e-12, -3e-9, 300.0, -1e5], np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for r in range(m):
        marked[r, g.choice(H, 2, replace=False)] = g.choice(np.concatenate([specials, [0x0001]]).astype(np.uint16), 2)
    ws = torch.empty(nv.pass_workspace_bytes(m, H, I, L), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((m, H), dtype=torch.bfloat16, device="cuda")
    for name, a in (("marked", marked), ("marked again", marked), ("plain", base)):
        h0 = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        before = ctx.f16_redone()
        ctx.verify_pass(arr, H, I, h0[:m], ws, h_out)
        redone = ctx.f16_redone() - before
        ref = manual_chain(torch, ctx, packed, h0[:m], H, I)
        log("M=%d %s: %d units recomputed" % (m, name, redone))
        assert torch.equal(h_out.view(torch.int16), ref[-1].view(torch.int16)), (m, name)
        assert (redone > 0) == (name != "plain"), (m, name, redone)
