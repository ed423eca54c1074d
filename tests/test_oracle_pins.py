"""Pins for the CPU oracle: each test ties it to something other than itself.

- E2M1 / E4M3 decode: exhaustive, against a hand-written value table (E2M1) and
  against torch's float8_e4m3fn conversion as a library routine (E4M3).
- Encoders and the quantiser: brute-force argmin over the decoded grid with the
  tie rule, on random values, every midpoint and its fp64 neighbours.
- GEMM: the hand-computed 2x16x2 worked example (tests/golden), row
  independence, exact scaling, one-hot extraction, a scale-exponent bump, and a
  dense fp64 matmul of the decoded weights (numpy as the library routine).
- bf16 rounding and the chain glue: against torch's bf16 conversion.
"""

import math

import numpy as np
import pytest
import torch

from conftest import read_golden

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX E2M1 magnitudes by code


def lib_e4m3_values():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ---------------------------------------------------------------- decode ----
def test_e2m1_exhaustive(oracle_mod):
    for code in range(16):
        mag = E2M1_TABLE[code & 7]
        expect = math.copysign(mag, -1.0) if code & 8 else mag
        got = oracle_mod.e2m1_value(code)
        assert got == expect and math.copysign(1.0, got) == math.copysign(1.0, expect)


def test_e4m3_exhaustive_against_library(oracle_mod):
    ref = lib_e4m3_values()
    for byte in range(256):
        got = oracle_mod.e4m3_value(byte)
        if np.isnan(ref[byte]):
            assert np.isnan(got), hex(byte)
        else:
            assert got == ref[byte], hex(byte)
            assert math.copysign(1.0, got) == math.copysign(1.0, ref[byte])


@pytest.mark.parametrize("byte,value", [(0x38, 1.0), (0x3C, 1.5), (0x04, 2.0 ** -7), (0x01, 2.0 ** -9),
                                        (0x08, 2.0 ** -6), (0x7E, 448.0), (0xFE, -448.0)])
def test_e4m3_anchors(oracle_mod, byte, value):
    assert oracle_mod.e4m3_value(byte) == value


def test_e4m3_specials(oracle_mod):
    assert np.isnan(oracle_mod.e4m3_value(0x7F)) and np.isnan(oracle_mod.e4m3_value(0xFF))
    z = oracle_mod.e4m3_value(0x80)
    assert z == 0.0 and math.copysign(1.0, z) == -1.0


# ---------------------------------------------------------------- encode ----
def brute_e4m3(x):
    """Nearest finite E4M3 magnitude (ties to even mantissa), saturating at 448."""
    vals = lib_e4m3_values()[:0x7F]  # 0x00..0x7E, all finite non-negative
    ax = abs(x)
    if ax >= 448.0:
        b = 0x7E
    else:
        d = np.abs(vals - ax)
        best = np.flatnonzero(d == d.min())
        b = int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])
    return b | (0x80 if math.copysign(1.0, x) < 0 else 0)


def e4m3_probe_points():
    vals = lib_e4m3_values()[:0x7F]
    pts = list(vals)
    for a, b in zip(vals[:-1], vals[1:]):
        mid = (a + b) / 2
        pts += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf)]
    pts += [448.0, 460.0, 464.0, 470.0, 1e6, 2.0 ** -10, 2.0 ** -10 * 1.0000001, 1e-30]
    g = np.random.default_rng(1)
    pts += list(np.exp2(g.uniform(-12, 10, 4000)))
    return pts


def test_e4m3_encode_bruteforce(oracle_mod):
    for x in e4m3_probe_points():
        for v in (x, -x):
            assert oracle_mod.e4m3_encode(v) == brute_e4m3(v), repr(v)


def brute_e2m1(q):
    aq = abs(q)
    if aq > 6.0:
        c = 7
    else:
        d = [abs(aq - v) for v in E2M1_TABLE]
        m = min(d)
        best = [i for i, di in enumerate(d) if di == m]
        c = best[0] if len(best) == 1 else [i for i in best if i % 2 == 0][0]
    return c | (8 if math.copysign(1.0, q) < 0 else 0)


def test_e2m1_encode_bruteforce(oracle_mod):
    pts = list(E2M1_TABLE)
    for a, b in zip(E2M1_TABLE[:-1], E2M1_TABLE[1:]):
        mid = (a + b) / 2
        pts += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf)]
    pts += [6.5, 100.0, 1e-300, 0.0]
    pts += list(np.random.default_rng(2).uniform(0, 7, 3000))
    for x in pts:
        for v in (x, -x):
            assert oracle_mod.e2m1_encode(v) == brute_e2m1(v), repr(v)
    # ties go to the even mantissa
    assert [oracle_mod.e2m1_encode(t) for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)] == [0, 2, 2, 4, 4, 6, 6]


# ------------------------------------------------------------- quantiser ----
def brute_quantize(w):
    n, k = w.shape
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, k // 16), np.uint8)
    lib = lib_e4m3_values()
    for j in range(n):
        for b in range(k // 16):
            blk = w[j, b * 16:(b + 1) * 16].astype(np.float64)
            amax = float(np.max(np.abs(blk)))
            sb = brute_e4m3(amax / 6.0)
            scales[j, b] = sb
            s = lib[sb]
            for t in range(16):
                c = 0 if s == 0 else brute_e2m1(float(blk[t]) / s)
                kk = b * 16 + t
                codes[j, kk >> 1] |= (c << 4) if kk & 1 else c
    return codes, scales


def test_quantize_bruteforce(oracle_mod):
    g = np.random.default_rng(3)
    w = g.standard_normal((24, 64)).astype(np.float32)
    w[0, :16] = 0.0                                   # s = 0 -> all codes 0
    w[1, :16] = np.float32(1e-5)                      # absmax/6 below half the smallest subnormal
    w[2, :16] = np.float32(5000.0)                    # scale saturates at 448, codes at 6
    w[3, :16] = -np.float32(1e-9); w[3, 0] = 6.0      # tiny negatives -> -0 (code 8)
    w[4, :16] = np.float32([6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -1.25, -1.75, -2.5, -3.5, -5, 0])
    w[5, :16] *= np.float32(2.0 ** -12)               # subnormal scales
    w[6, 16:32] = np.float32(6.375)                   # absmax/6 = 1.0625: an exact E4M3 tie
    codes, scales = oracle_mod.quantize(w)
    c2, s2 = brute_quantize(w)
    assert np.array_equal(scales, s2)
    assert np.array_equal(codes, c2)
    assert scales[0, 0] == 0 and not codes[0, :8].any()
    assert scales[2, 0] == 0x7E
    assert codes[3, 0] & 0xF == 7 and all((codes[3, 1:8] & 0xF) == 8) and all((codes[3, 0:8] >> 4) == 8)
    assert scales[6, 1] == 0x38  # 1.0625 ties between 1.0 and 1.125 -> even mantissa (1.0)


def test_quantize_rejects_nonfinite(oracle_mod):
    w = np.zeros((1, 16), np.float32)
    w[0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle_mod.quantize(w)
    w[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle_mod.quantize(w)


def test_quantize_thread_invariant(oracle_mod):
    w = np.random.default_rng(4).standard_normal((37, 96)).astype(np.float32)
    a = oracle_mod.quantize(w, threads=1)
    b = oracle_mod.quantize(w, threads=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ GEMM ----
def golden_example():
    g = read_golden("worked_example_2x16x2.txt")
    hexrow = lambda key: np.array([int(v, 16) for v in g[key]])
    codes = np.stack([hexrow("codes_row0"), hexrow("codes_row1")]).astype(np.uint8)
    scales = np.stack([hexrow("scale_row0"), hexrow("scale_row1")]).astype(np.uint8)
    a = np.stack([hexrow("a_row0"), hexrow("a_row1")]).astype(np.uint16)
    c = np.array([[float(v) for v in g["c_row0"]], [float(v) for v in g["c_row1"]]])
    s = np.array([[float(v) for v in g["s_row0"]], [float(v) for v in g["s_row1"]]])
    return a, codes, scales, c, s


def test_worked_example(oracle_mod):
    a, codes, scales, c_ref, s_ref = golden_example()
    c, s = oracle_mod.gemm(a, codes, scales)
    assert np.array_equal(c, c_ref)
    assert np.array_equal(s, s_ref)


def test_worked_example_nibble_order_matters(oracle_mod):
    a, codes, scales, c_ref, _ = golden_example()
    swapped = ((codes >> 4) | (codes << 4)).astype(np.uint8)
    c, _ = oracle_mod.gemm(a, swapped, scales)
    assert c[1, 1] == 400.0 / 128.0 and c[1, 1] != c_ref[1, 1]


def random_problem(m, n, k, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((m, k)).astype(np.float32)
    a = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    codes = g.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = g.integers(0x10, 0x58, (n, k // 16), dtype=np.uint8)
    return a, codes, scales


def bf16_to_f64(a):
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def test_row_independence(oracle_mod):
    a, codes, scales = random_problem(5, 7, 64, 10)
    c5, s5 = oracle_mod.gemm(a, codes, scales)
    for i in range(5):
        c1, s1 = oracle_mod.gemm(a[i:i + 1], codes, scales)
        assert np.array_equal(c1[0], c5[i]) and np.array_equal(s1[0], s5[i])


def test_exact_scaling_and_ts(oracle_mod):
    a, codes, scales = random_problem(3, 9, 48, 11)
    c, s = oracle_mod.gemm(a, codes, scales)
    a2 = (a.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # bf16 exponent + 1 = times 2 (no zeros here)
    assert not ((a & 0x7F80) == 0).any()
    c2, _ = oracle_mod.gemm(a2, codes, scales)
    assert np.array_equal(c2, 2 * c)
    c3, s3 = oracle_mod.gemm(a, codes, scales, ts=0.25)
    assert np.array_equal(c3, 0.25 * c) and np.array_equal(s3, 0.25 * s)


def test_one_hot_extracts_weights(oracle_mod):
    a, codes, scales = random_problem(1, 6, 32, 12)
    k = 32
    onehot = np.zeros((k, k), np.uint16)
    onehot[np.arange(k), np.arange(k)] = 0x3F80  # bf16 1.0
    c, _ = oracle_mod.gemm(onehot, codes, scales)
    w = oracle_mod.decode(codes, scales)
    assert np.array_equal(c, w.T)
    # and the decoded weights agree with the library fp8 / the E2M1 table element by element
    lib = lib_e4m3_values()
    for j in range(6):
        for kk in range(k):
            nib = (codes[j, kk // 2] >> (4 * (kk % 2))) & 0xF
            mag = E2M1_TABLE[nib & 7] * (-1 if nib & 8 else 1)
            assert w[j, kk] == mag * lib[scales[j, kk // 16]]


def test_scale_exponent_bump_doubles_block(oracle_mod):
    a, codes, scales = random_problem(4, 5, 64, 13)
    c, _ = oracle_mod.gemm(a, codes, scales)
    bumped = scales.copy()
    bumped[:, 2] += 0x08  # E4M3 exponent field + 1 (all scales normal and < 0x58 here)
    c2, _ = oracle_mod.gemm(a, codes, bumped)
    w = oracle_mod.decode(codes, scales)
    af = bf16_to_f64(a)
    block = af[:, 32:48] @ w[:, 32:48].T
    np.testing.assert_allclose(c2, c + block, rtol=1e-12, atol=1e-12)


def test_dense_matmul_crosscheck(oracle_mod):
    a, codes, scales = random_problem(6, 33, 160, 14)
    c, s = oracle_mod.gemm(a, codes, scales, ts=1.75)
    w = oracle_mod.decode(codes, scales, ts=1.75)
    af = bf16_to_f64(a)
    ref = np.matmul(af, w.T)
    assert np.all(np.abs(c - ref) <= 1e-12 * s)
    np.testing.assert_allclose(s, np.abs(af) @ np.abs(w).T, rtol=1e-12)


def test_k_permutation_invariance(oracle_mod):
    a, codes, scales = random_problem(3, 4, 64, 15)
    c, s = oracle_mod.gemm(a, codes, scales)
    # permute whole 16-blocks (so scales move with their codes) and the matching A columns
    perm_blocks = [2, 0, 3, 1]
    cols = np.concatenate([np.arange(b * 16, b * 16 + 16) for b in perm_blocks])
    codes_p = np.concatenate([codes[:, b * 8:b * 8 + 8] for b in perm_blocks], axis=1)
    scales_p = scales[:, perm_blocks]
    c2, _ = oracle_mod.gemm(a[:, cols], codes_p, scales_p)
    assert np.all(np.abs(c2 - c) <= 1e-13 * s)


def test_nan_scale_propagates(oracle_mod):
    a, codes, scales = random_problem(2, 3, 32, 16)
    scales[1, 1] = 0x7F
    c, _ = oracle_mod.gemm(a, codes, scales)
    assert np.isnan(c[:, 1]).all() and not np.isnan(c[:, [0, 2]]).any()


def test_sampled_cols_match_full(oracle_mod):
    a, codes, scales = random_problem(4, 40, 96, 17)
    c, s = oracle_mod.gemm(a, codes, scales)
    cols = np.array([39, 0, 17, 17, 5])
    cs, ss = oracle_mod.gemm(a, codes, scales, cols=cols)
    assert np.array_equal(cs, c[:, cols]) and np.array_equal(ss, s[:, cols])


def test_gemm_thread_invariant(oracle_mod):
    a, codes, scales = random_problem(3, 50, 64, 18)
    c1, _ = oracle_mod.gemm(a, codes, scales, threads=1)
    c7, _ = oracle_mod.gemm(a, codes, scales, threads=7)
    assert np.array_equal(c1, c7)


def test_tolerance_rule(oracle_mod):
    c = np.array([1.0, 0.0, np.nan, 2.0])
    s = np.array([10.0, 0.0, 1.0, 1.0])
    ok = oracle_mod.within_tolerance(np.array([1.0 + 9e-5, -0.0, np.nan, np.inf]), c, s)
    assert ok.tolist() == [True, True, True, False]
    ok = oracle_mod.within_tolerance(np.array([1.0 + 2e-4, 1e-30, 0.0, 2.0]), c, s)
    assert ok.tolist() == [False, False, False, True]


# ------------------------------------------------------- bf16 and glue ------
def torch_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_against_library(oracle_mod):
    g = np.random.default_rng(19)
    bits = g.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    ties = (g.integers(0, 2 ** 16, 2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([bits, ties]).view(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1e-45])])
    got = oracle_mod.bf16_from_f32(x)
    ref = torch_bf16_bits(x)
    finite = ~np.isnan(x)
    assert np.array_equal(got[finite], ref[finite])
    assert np.all((got[~finite] & 0x7F80) == 0x7F80) and np.all((got[~finite] & 0x7F) != 0)


def test_glue_against_library(oracle_mod):
    g = np.random.default_rng(20)
    x = (g.standard_normal(50000) * 30).astype(np.float32)
    y = (g.standard_normal(50000) * 30).astype(np.float32)
    cst = np.float32(1.0 / math.sqrt(5120.0))
    assert np.array_equal(oracle_mod.glue_scale(x, cst), torch_bf16_bits(x * cst))
    c2 = np.float32(1.0 / math.sqrt(2 * 5120.0))
    ref = torch_bf16_bits((x * c2) + (y * c2))
    assert np.array_equal(oracle_mod.glue_sum(x, y, c2), ref)
