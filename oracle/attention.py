"""Oracle of tree-verify attention (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
CPU-baseline leg may import this module; the product (the HIP library and its
binding) never does, and the two share no code.

What the pages fix. The served model mixes 48 Gated DeltaNet layers with 16
attention layers (TandemLLM manual, "What TandemLLM is", 1.1 "The test
environment"). One forward pass checks every guess of the draft tree at once
(1.2 "Two levers"), so each attention layer of the verify pass runs its M rows
(the root token and the tree's nodes) against the committed context, and the
cost is measured per context length from 1k to 32k tokens (release post, the
paragraph on what checking 8 to 32 guesses costs). The pages give neither the
head layout nor the attention formula; the plain reading, written out here:

* scaled dot-product attention with a softmax over the visible keys, fp64;
* row i of the tree sees every context position 0 .. T-1 and the tree rows on
  its own path to the root, itself included (the tokens it would follow if
  its branch were accepted), and no other tree row;
* the tree rows' keys and values sit at positions T + j of the same cache;
* grouped query heads: query head h reads key/value head h // (Hq / Hkv).

Inputs are bf16 bit patterns (uint16); everything is computed in fp64:
  s_j  = scale * sum_d q[d] k_j[d]          over the visible positions j
  p_j  = exp(s_j - max s) / sum_j' exp(s_j' - max s)
  O[d] = sum_j p_j v_j[d]
and, for the parity tolerance, A[d] = sum_j p_j |v_j[d]| and
E = max_j scale * sum_d |q[d] k_j[d]| (the size of the largest score's terms).
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 (exact: a bf16 is the top half of an fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def visible_rows(parent_rows) -> np.ndarray:
    """vis[i][j]: tree row i sees tree row j (j on i's path to the root, or j = i).
    parent_rows[0] = -1 (the root row); parent_rows[i] < i for i >= 1."""
    m = len(parent_rows)
    vis = np.zeros((m, m), dtype=bool)
    for i in range(m):
        j = i
        while j >= 0:
            vis[i, j] = True
            j = int(parent_rows[j])
    return vis


def tree_attention(q_bits, k_bits, v_bits, parent_rows, ctx_len: int, scale: float):
    """q_bits [M][Hq][D], k_bits / v_bits [Hkv][>= ctx_len + M][D] (position T + i
    holds tree row i). Returns (O, A, E): O and A [M][Hq][D], E [M][Hq], fp64."""
    q = bf16_to_f64(q_bits)
    m, hq, d = q.shape
    hkv = k_bits.shape[0]
    assert hq % hkv == 0, "query heads must be a multiple of key/value heads"
    group = hq // hkv
    k = bf16_to_f64(k_bits[:, : ctx_len + m])
    v = bf16_to_f64(v_bits[:, : ctx_len + m])
    vis = visible_rows(parent_rows)
    out = np.zeros((m, hq, d))
    absout = np.zeros((m, hq, d))
    emax = np.zeros((m, hq))
    for i in range(m):
        pos = np.concatenate([np.arange(ctx_len), ctx_len + np.nonzero(vis[i])[0]])
        for h in range(hq):
            kv = h // group
            kk, vv = k[kv, pos], v[kv, pos]
            terms = kk * q[i, h][None, :]
            s = scale * terms.sum(axis=1)
            p = np.exp(s - s.max())
            p /= p.sum()
            out[i, h] = p @ vv
            absout[i, h] = p @ np.abs(vv)
            emax[i, h] = scale * np.abs(terms).sum(axis=1).max()
    return out, absout, emax


def within_tolerance(o_gpu, o, a, e, rel: float = 2e-5):
    """|O_gpu - O| <= (rel + 4 * 2^-24 * D * E) * A + 1e-30 per element.

    Derivation (fp32 arithmetic on the device): a score's dot product over D
    terms carries at most ~D * 2^-24 * E of rounding; a shift of every score by
    at most delta changes each softmax weight by a factor within exp(+-2 delta),
    hence O by at most ~(4 delta) * A for small delta. `rel` covers the rest,
    relative to A: the exponentials (a few ulp), the split of each weight into
    two bf16 terms (2^-17) and the fp32 sums over positions and chunks."""
    d = o.shape[-1]
    bound = (rel + 4.0 * 2.0 ** -24 * d * e)[..., None] * a + 1e-30
    return np.abs(np.asarray(o_gpu, np.float64) - o) <= bound
