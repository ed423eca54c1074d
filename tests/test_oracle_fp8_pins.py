"""Pins of the oracle's FP8 output head (quantiser and GEMM) against things
other than the oracle itself: torch's float8_e4m3fn decode (a library routine),
brute-force nearest-value search on that table, exact closed forms, and a dense
fp64 matmul. The head's format is a reading of the TandemLLM manual, "What
TandemLLM is", 1.2 "Two levers" (the output head is kept in FP8): OCP E4M3 codes
with one fp32 scale per output row."""
import numpy as np
import pytest
import torch

import synth


def e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


TAB = e4m3_table()


def brute_code(x):
    neg = bool(np.signbit(x))
    ax = abs(float(x))
    if ax >= 448.0:
        mag = 0x7E
    else:
        d = np.abs(TAB[:0x7F] - ax)
        cand = np.nonzero(d == d.min())[0]
        mag = int(cand[0]) if cand.size == 1 else int([c for c in cand if c % 2 == 0][0])
    return mag | (0x80 if neg else 0)


def brute_quantize(w):
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    scales = np.zeros(n, np.float32)
    for j in range(n):
        s = np.float32(np.max(np.abs(w[j].astype(np.float64))) / 448.0)
        scales[j] = s
        if s != 0:
            for kk in range(k):
                codes[j, kk] = brute_code(float(w[j, kk]) / float(s))
    return codes, scales


def special_rows(k):
    rows = []
    rows.append(np.zeros(k, np.float32))                       # all-zero row: s = 0, codes +0
    r = np.zeros(k, np.float32)
    r[0] = 112.0                                               # s = 0.25 exactly
    r[1], r[2] = 0.25 * 1.0625, 0.25 * 1.1875                  # ties between grid points
    r[3], r[4] = -0.25 * 1.0625, -0.0                          # negative tie, negative zero
    r[5] = 0.25 * 2.0 ** -10                                   # below half the smallest subnormal
    r[6] = 0.25 * 3 * 2.0 ** -10                               # tie between subnormal codes 1 and 2
    rows.append(r)
    g = np.zeros(k, np.float32)
    g[:126] = TAB[1:127][:k] if k >= 126 else TAB[1:1 + k]     # every positive grid value (x 2^-3 below)
    g *= 0.125
    rows.append(g)
    return np.stack(rows)


@pytest.mark.parametrize("seed", [0, 1])
def test_fp8_quantize_bruteforce(oracle_mod, seed):
    k = 160
    w = np.concatenate([special_rows(k), synth.weights_f32(5, k, seed=seed, stream="fp8pin")])
    codes, scales = oracle_mod.fp8_quantize(w)
    bc, bs = brute_quantize(w)
    assert np.array_equal(scales.view(np.uint32), bs.view(np.uint32))
    assert np.array_equal(codes, bc)


def test_fp8_quantize_closed_forms(oracle_mod):
    k = 160
    w = special_rows(k)
    codes, scales = oracle_mod.fp8_quantize(w)
    assert scales[0] == 0 and not codes[0].any()
    assert scales[1] == 0.25
    assert list(codes[1, :7]) == [0x7E, 0x38, 0x3A, 0xB8, 0x80, 0x00, 0x02]
    # the grid row: absmax 448/8 gives s = 1/8, so every grid value comes back unchanged
    assert scales[2] == 0.125
    assert np.array_equal(codes[2, :126], np.arange(1, 127, dtype=np.uint8))
    assert codes[2, 125] == 0x7E


def test_fp8_quantize_rejects_nonfinite(oracle_mod):
    w = np.zeros((2, 32), np.float32)
    w[1, 3] = np.inf
    with pytest.raises(ValueError):
        oracle_mod.fp8_quantize(w)


def fp8_problem(m, n, k, seed):
    codes = synth.fp8_codes(n, k, seed=seed)
    scales = synth.fp8_row_scales(n, seed=seed)
    a = synth.activations_bf16(m, k, seed=seed, stream="fp8pin")
    return a, codes, scales


def bf16_to_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_fp8_gemm_dense_crosscheck(oracle_mod):
    a, codes, scales = fp8_problem(5, 40, 272, seed=3)
    c, s = oracle_mod.fp8_gemm(a, codes, scales)
    w = scales.astype(np.float64)[:, None] * TAB[codes]
    ref = bf16_to_f64(a) @ w.T
    sref = np.abs(bf16_to_f64(a)) @ np.abs(w).T
    assert np.allclose(s, sref, rtol=1e-12, atol=0)
    assert np.all(np.abs(c - ref) <= 1e-12 * sref)


def test_fp8_gemm_one_hot_extracts_weights(oracle_mod):
    k, n = 48, 9
    _, codes, scales = fp8_problem(1, n, k, seed=4)
    eye = np.zeros((k, k), np.float32)
    np.fill_diagonal(eye, 1.0)
    a = oracle_mod.bf16_from_f32(eye)
    c, _ = oracle_mod.fp8_gemm(a, codes, scales)
    assert np.array_equal(c.T, scales.astype(np.float64)[:, None] * TAB[codes])


def test_fp8_gemm_cols_and_row_scale_linearity(oracle_mod):
    a, codes, scales = fp8_problem(3, 30, 96, seed=5)
    c, s = oracle_mod.fp8_gemm(a, codes, scales)
    cols = np.array([29, 0, 7, 7, 13])
    cc, ss = oracle_mod.fp8_gemm(a, codes, scales, cols=cols)
    assert np.array_equal(cc, c[:, cols]) and np.array_equal(ss, s[:, cols])
    c2, _ = oracle_mod.fp8_gemm(a, codes, scales * np.float32(2.0))
    assert np.array_equal(c2, 2.0 * c)
