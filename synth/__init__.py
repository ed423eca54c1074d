"""Seeded synthetic inputs for the NVFP4 verify GEMM.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no E2M1/E4M3 encoding or decoding, no quantiser, no GEMM,
no chain glue). Both the CPU oracle and the HIP path take their inputs from
here; each side then applies its own quantiser / encoder.

Streams. Every tensor is drawn from its own counter-based Philox stream keyed by
(seed, tag, *ids), so any tensor, and any weight row of it, can be regenerated
alone. Weight rows are drawn in blocks of ``ROW_BLOCK`` rows, each block with its
own key, so a sampled parity check can regenerate only the rows it needs.

Distributions (the plainest readings where a recipe leaves a step open):
  * activations: fp64 N(0,1) -> fp32 -> bf16 (round-to-nearest-even, done by
    torch's dtype conversion). Optional outlier columns: round(0.001 * K)
    distinct column indices, drawn without replacement; those columns are
    multiplied by 20 in fp32 before the bf16 rounding. Row i of an M-row draw
    is the same for every M (rows nest).
  * weights for quantisation: fp32 N(0,1) (fp64 draw, rounded to fp32).
  * "tiny" weights given directly in the 4-bit format: code bytes uniform over
    0..255 (so each nibble is uniform over the 16 codes) and one scale *value*
    per 16 elements, 2^u with u ~ U(-4, 2) continuous, as fp32; each side
    encodes that value to E4M3 itself.
"""

from __future__ import annotations

import hashlib

import numpy as np

ROW_BLOCK = 256
MAX_ROWS = 128  # activations are drawn as 128 rows (row i is the same for any M); callers slice


def _key(seed: int, tag: str, *ids: int) -> int:
    h = hashlib.sha256(repr((int(seed), str(tag)) + tuple(int(i) for i in ids)).encode())
    return int.from_bytes(h.digest()[:16], "little")


def rng(seed: int, tag: str, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=_key(seed, tag, *ids)))


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def outlier_columns(k: int, seed: int = 0, stream: str = "act") -> np.ndarray:
    count = int(round(0.001 * k))
    if count == 0:
        return np.zeros(0, np.int64)
    g = rng(seed, stream + "/outliers", k)
    return np.sort(g.choice(k, size=count, replace=False)).astype(np.int64)


def activations_f32(m: int, k: int, seed: int = 0, stream: str = "act",
                    outliers: bool = True) -> np.ndarray:
    """fp32 activations [m, k] before the bf16 rounding (rows nest across m)."""
    if m > MAX_ROWS:
        raise ValueError("at most %d rows" % MAX_ROWS)
    g = rng(seed, stream, k)
    x = g.standard_normal((MAX_ROWS, k)).astype(np.float32)[:m]
    if outliers:
        cols = outlier_columns(k, seed, stream)
        x[:, cols] *= np.float32(20.0)
    return np.ascontiguousarray(x)


def activations_bf16(m: int, k: int, seed: int = 0, stream: str = "act",
                     outliers: bool = True) -> np.ndarray:
    """bf16 bit patterns (uint16) [m, k]."""
    return _to_bf16_bits(activations_f32(m, k, seed, stream, outliers))


def weights_f32(n: int, k: int, seed: int = 0, stream: str = "w", rows=None) -> np.ndarray:
    """fp32 N(0,1) weights [n, k], or only the listed rows (same values)."""
    if rows is None:
        out = np.empty((n, k), np.float32)
        for b0 in range(0, n, ROW_BLOCK):
            b1 = min(n, b0 + ROW_BLOCK)
            g = rng(seed, stream, n, k, b0 // ROW_BLOCK)
            out[b0:b1] = g.standard_normal((b1 - b0, k)).astype(np.float32)
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, k), np.float32)
    cache = {}
    for idx, r in enumerate(rows):
        blk = int(r) // ROW_BLOCK
        if blk not in cache:
            b0 = blk * ROW_BLOCK
            b1 = min(n, b0 + ROW_BLOCK)
            g = rng(seed, stream, n, k, blk)
            cache = {blk: g.standard_normal((b1 - b0, k)).astype(np.float32)}
        out[idx] = cache[blk][int(r) - blk * ROW_BLOCK]
    return out


def tiny_codes(n: int, k: int, seed: int = 0, stream: str = "tiny") -> np.ndarray:
    """Code bytes [n, k/2], uniform over 0..255 (each nibble uniform over 16 codes)."""
    g = rng(seed, stream + "/codes", n, k)
    return g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)


def tiny_scale_values(n: int, k: int, seed: int = 0, stream: str = "tiny") -> np.ndarray:
    """Scale values [n, k/16] = 2^u, u ~ U(-4, 2), as fp32 (to be E4M3-encoded)."""
    g = rng(seed, stream + "/scales", n, k)
    u = g.uniform(-4.0, 2.0, size=(n, k // 16))
    return np.exp2(u).astype(np.float32)


# ---- device-side draws (fast, for the full-size benchmark stack) -----------
def cuda_generator(seed: int, tag: str, *ids: int):
    import torch

    g = torch.Generator(device="cuda")
    g.manual_seed(_key(seed, tag, *ids) & ((1 << 63) - 1))
    return g


def weights_f32_cuda(n: int, k: int, seed: int = 0, stream: str = "w", out=None):
    """fp32 N(0,1) weights [n, k] drawn on the GPU with torch's Philox generator."""
    import torch

    g = cuda_generator(seed, stream, n, k)
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device="cuda")
    out.normal_(0.0, 1.0, generator=g)
    return out


def fp8_codes(n: int, k: int, seed: int = 0, stream: str = "fp8") -> np.ndarray:
    """Uniformly random finite OCP E4M3 bytes u8[n, k] (0x7F and 0xFF, the NaNs, excluded)."""
    r = rng(seed, stream, n, k).integers(0, 254, size=(n, k), dtype=np.uint8)
    return r + (r >= 0x7F).astype(np.uint8)


def fp8_row_scales(n: int, seed: int = 0, stream: str = "fp8s") -> np.ndarray:
    """fp32 row scales [n] spread over 2^-14 .. 2^-6 (|w| / 448 for weights of a few 1e-3 to 1e-1)."""
    return np.exp2(rng(seed, stream, n).uniform(-14.0, -6.0, size=n)).astype(np.float32)


def draft_tree(n: int, seed: int = 0, stream: str = "tree", shape: str = "random"):
    """A synthetic draft tree of n nodes for StairCut's cut: (parent int32[n],
    p_accept float64[n]). Parents come before their children (-1 = the root).
    shape "random": each node hangs under the root or an earlier node, chosen
    uniformly; "chain": node v under v - 1; "wide": under the root or one of
    the first three nodes. Each node's children share an acceptance mass
    m ~ U(0.3, 0.98) split by uniform weights, so the probabilities of siblings
    sum to m <= 1 (siblings are different tokens at one position)."""
    g = rng(seed, stream, n)
    if shape == "chain":
        parent = np.arange(-1, n - 1, dtype=np.int32)
    elif shape == "wide":
        parent = np.array([-1] + [int(g.integers(-1, min(v, 3))) for v in range(1, n)], np.int32)
    else:
        parent = np.array([int(g.integers(-1, v)) for v in range(n)], np.int32)
    p = np.zeros(n, np.float64)
    for u in range(-1, n):
        kids = np.nonzero(parent == u)[0]
        if kids.size == 0:
            continue
        mass = g.uniform(0.3, 0.98)
        w = g.uniform(0.05, 1.0, kids.size)
        p[kids] = mass * w / w.sum()
    return parent, p


def attention_inputs(m: int, hq: int, hkv: int, ctx_len: int, d: int = 128, seed: int = 0,
                     stream: str = "attn"):
    """Tree-verify attention inputs as bf16 bit patterns: queries [m][hq][d] and
    keys / values [hkv][ctx_len + m][d] (positions ctx_len + i are tree row
    i's), all N(0, 1) like the projections' outputs after the linear glue."""
    g = rng(seed, stream, m, hq, hkv, ctx_len, d)
    q = _to_bf16_bits(g.standard_normal((m, hq, d), dtype=np.float32))
    k = _to_bf16_bits(g.standard_normal((hkv, ctx_len + m, d), dtype=np.float32))
    v = _to_bf16_bits(g.standard_normal((hkv, ctx_len + m, d), dtype=np.float32))
    return q, k, v


def tree_parent_rows(m: int, seed: int = 0, shape: str = "random", stream: str = "attn-tree"):
    """Parent rows of an m-row verify tree: row 0 is the root (-1), rows 1..m-1
    the nodes of draft_tree(m - 1) (a node under the root hangs from row 0)."""
    if m == 1:
        return np.array([-1], np.int32)
    parent, _ = draft_tree(m - 1, seed=seed, stream=stream, shape=shape)
    return np.concatenate([[-1], parent.astype(np.int64) + 1]).astype(np.int32)


def staircase_us(max_rows: int = 64, seed: int = 0, stream: str = "stairs", base: float = 3800.0,
                 step_rows: int = 8, step: float = 0.2):
    """A synthetic staircase for the cut: us_by_rows[r - 1], flat within each
    block of step_rows rows with a jump of up to `step` (relative, uniform) at
    every block boundary and small seeded noise; for CPU tests of the cut."""
    g = rng(seed, stream, max_rows, step_rows)
    us = np.empty(max_rows, np.float64)
    level = base
    for r in range(1, max_rows + 1):
        if r > 1 and (r - 1) % step_rows == 0:
            level *= 1.0 + g.uniform(0.0, step)
        us[r - 1] = level * (1.0 + g.uniform(-0.01, 0.01))
    return us
