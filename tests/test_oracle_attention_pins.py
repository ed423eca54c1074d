"""Pins of the tree-verify attention oracle (CPU): a hand-worked case, closed
forms, the same attention through torch's scaled_dot_product_attention
(float64, an explicit mask built here), and invariants. Each is chosen so that
a plausible mistake in the oracle (a dropped or extra position, a mask that is
transposed or leaks between siblings, a wrong query-to-key/value head map, a
misapplied scale) fails at least one of them."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import attention as att

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_attention_hand.txt")


def bits(x):
    """fp64 values that are exact in bf16 -> bf16 bit patterns."""
    f = np.asarray(x, np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def rand_bits(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 is a valid input


def test_hand_worked_example():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    want = np.array([[float(Fraction(x)) for x in r[1:]] for r in rows])
    k = bits([[[0, 5], [1, 5], [2, 5]]])
    v = bits([[[1, 0], [0, 1], [1, 1]]])
    q = bits([[[1, 0]], [[1, 0]]])
    o, a, e = att.tree_attention(q, k, v, [-1, 0], ctx_len=1, scale=math.log(2.0))
    assert np.allclose(o[:, 0, :], want, rtol=0, atol=1e-15)
    assert np.allclose(a, o)
    assert np.allclose(e[:, 0], [math.log(2.0), 2 * math.log(2.0)])


def test_equal_keys_give_the_mean_of_the_visible_values():
    # every key equal: uniform weights over exactly the visible positions
    rng = np.random.default_rng(1)
    T, D = 9, 8
    parent = [-1, 0, 0, 1, 3]  # rows 3 and 4 descend through row 1; row 2 is a sibling of row 1
    M = len(parent)
    k = np.tile(bits(np.full(D, 0.5)), (1, T + M, 1))
    v = rand_bits(rng, (1, T + M, D))
    q = rand_bits(rng, (M, 1, D))
    o, _, _ = att.tree_attention(q, k, v, parent, T, scale=0.3)
    vf = att.bf16_to_f64(v)[0]
    paths = {0: [0], 1: [0, 1], 2: [0, 2], 3: [0, 1, 3], 4: [0, 1, 3, 4]}  # written out by hand
    for i in range(M):
        pos = list(range(T)) + [T + j for j in paths[i]]
        assert np.allclose(o[i, 0], vf[pos].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_a_root_without_context_returns_its_own_value():
    rng = np.random.default_rng(2)
    v = rand_bits(rng, (2, 1, 16))
    q = rand_bits(rng, (1, 4, 16))
    k = rand_bits(rng, (2, 1, 16))
    o, a, _ = att.tree_attention(q, k, v, [-1], 0, scale=0.25)
    vf = att.bf16_to_f64(v)
    for h in range(4):
        assert np.array_equal(o[0, h], vf[h // 2, 0])
        assert np.array_equal(a[0, h], np.abs(vf[h // 2, 0]))


def test_one_dominant_key():
    rng = np.random.default_rng(3)
    T, D = 40, 16
    q = bits(np.ones((1, 1, D)))
    k = rand_bits(rng, (1, T + 1, D), 0.01)
    k[0, 17] = bits(np.full(D, 8.0))  # score 128 * scale above the rest
    v = rand_bits(rng, (1, T + 1, D))
    o, _, _ = att.tree_attention(q, k, v, [-1], T, scale=0.5)
    assert np.allclose(o[0, 0], att.bf16_to_f64(v)[0, 17], rtol=0, atol=1e-20)


def _sdpa(q_bits, k_bits, v_bits, allowed, scale, group):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F

    q = torch.from_numpy(att.bf16_to_f64(q_bits)).permute(1, 0, 2)  # [Hq][M][D]
    k = torch.from_numpy(att.bf16_to_f64(k_bits)).repeat_interleave(group, dim=0)  # [Hq][P][D]
    v = torch.from_numpy(att.bf16_to_f64(v_bits)).repeat_interleave(group, dim=0)
    mask = torch.from_numpy(allowed)[None]  # True = attend
    o = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask[None], scale=scale)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("shape", ["chain", "star", "random"])
def test_matches_library_attention_with_an_explicit_mask(shape):
    rng = np.random.default_rng({"chain": 4, "star": 5, "random": 6}[shape])
    T, M, D, hkv, group = 23, 7, 32, 2, 3
    if shape == "chain":
        parent = [-1] + list(range(M - 1))
    elif shape == "star":
        parent = [-1] + [0] * (M - 1)
    else:
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, M)]
    # the mask built from scratch: row i may see context and its ancestors
    allowed = np.zeros((M, T + M), bool)
    allowed[:, :T] = True
    for i in range(M):
        anc = {i}
        j = i
        while parent[j] >= 0:
            j = parent[j]
            anc.add(j)
        for j in anc:
            allowed[i, T + j] = True
    if shape == "chain":
        assert np.array_equal(allowed[:, T:], np.tril(np.ones((M, M), bool)))  # causal
    if shape == "star":
        assert np.array_equal(allowed[:, T:], np.eye(M, dtype=bool) | (np.arange(M)[None, :] == 0))
    q = rand_bits(rng, (M, hkv * group, D))
    k = rand_bits(rng, (hkv, T + M, D))
    v = rand_bits(rng, (hkv, T + M, D))
    scale = 1.0 / math.sqrt(D)
    o, a, e = att.tree_attention(q, k, v, parent, T, scale)
    ref = _sdpa(q, k, v, allowed, scale, group)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-14)
    assert np.all(a >= np.abs(o) - 1e-15) and np.all(e > 0)


def test_context_order_and_sibling_independence():
    rng = np.random.default_rng(7)
    T, D = 30, 16
    parent = [-1, 0, 0, 0]  # three siblings under the root
    M = len(parent)
    q = rand_bits(rng, (M, 2, D))
    k = rand_bits(rng, (1, T + M, D))
    v = rand_bits(rng, (1, T + M, D))
    o, _, _ = att.tree_attention(q, k, v, parent, T, 0.2)
    # permuting the context positions changes nothing
    perm = np.concatenate([rng.permutation(T), np.arange(T, T + M)])
    o2, _, _ = att.tree_attention(q, k[:, perm], v[:, perm], parent, T, 0.2)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-15)
    # a sibling's row equals a tree of the root and that node alone
    for i in (1, 2, 3):
        sel = np.concatenate([np.arange(T), [T, T + i]])
        o1, _, _ = att.tree_attention(q[[0, i]], k[:, sel], v[:, sel], [-1, 0], T, 0.2)
        assert np.allclose(o[i], o1[1], rtol=1e-12, atol=1e-15)


def test_tolerance_rejects_a_dropped_position():
    # the check is tight enough to see one missing context position at T = 64
    rng = np.random.default_rng(8)
    T, D = 64, 128
    q = rand_bits(rng, (1, 1, D))
    k = rand_bits(rng, (1, T + 1, D))
    v = rand_bits(rng, (1, T + 1, D))
    o, a, e = att.tree_attention(q, k, v, [-1], T, 1 / math.sqrt(D))
    assert att.within_tolerance(o.astype(np.float32), o, a, e).all()
    keep = np.concatenate([np.arange(1, T), [T]])
    o_drop, _, _ = att.tree_attention(q, k[:, keep], v[:, keep], [-1], T - 1, 1 / math.sqrt(D))
    assert not att.within_tolerance(o_drop, o, a, e).all()
