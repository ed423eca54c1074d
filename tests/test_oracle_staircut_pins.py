"""Pins of the StairCut cut-rule oracle (oracle/staircut.py) to things other
than itself, and the library's cut against the oracle (host code, CPU).

* The hand-worked example of tests/golden/: the pages' own staircase (release
  post: 75.5 / 74.4 / 83.1 / 87.8 ms at 8 / 16 / 24 / 32 rows) with a 31-node
  chain of guesses accepted with probability 0.8 each (closed form
  1 + 4 (1 - 0.8^n)); the cut keeps 15 nodes.
* Brute force on small trees: every subtree of every size, its expected
  committed tokens counted by walking the acceptance outcomes (the model's
  token matches at most one child; the walk stops at the first miss), not by
  the oracle's sum of path probabilities; the oracle's cut must reach the
  brute-force optimum at every size, and its choice of size must be the
  brute-force argmax of tokens per millisecond.
* Closed forms: all-zero acceptance commits exactly one token; certain
  acceptance commits n + 1.
"""

import itertools
import os

import numpy as np
import pytest

import nvfp4_skinny_gemm_amd as nv
import synth
from oracle import staircut as oc

from conftest import read_golden

GOLDEN = "staircut_chain_p08.txt"


def golden():
    g = read_golden(GOLDEN)
    return g


def pages_staircase():
    rows = {}
    path = os.path.join(os.path.dirname(__file__), "golden", GOLDEN)
    for line in open(path):
        if line.startswith("rows_ms"):
            _, r, ms = line.split()
            rows[int(r)] = float(ms) * 1000.0
    us = np.zeros(32)
    for r, v in rows.items():
        us[r - 1] = v
    return us


def golden_values(key):
    path = os.path.join(os.path.dirname(__file__), "golden", GOLDEN)
    out = {}
    for line in open(path):
        if line.startswith(key + " "):
            _, n, v = line.split()
            out[int(n)] = float(v)
    return out


def walk_expected(parent, p, kept):
    """Expected committed tokens of a kept node set by walking the outcomes:
    from a node, the model's next token is kept child c with probability p[c]
    (siblings exclusive), anything else with the rest; the walk stops at the
    first token outside the kept children. Committed = 1 + nodes walked."""
    kept = set(kept)
    children = {}
    for v, u in enumerate(parent):
        children.setdefault(int(u), []).append(v)

    def tail(u):  # expected further accepted nodes below an accepted u
        return sum(p[c] * (1.0 + tail(c)) for c in children.get(u, []) if c in kept)

    return 1.0 + tail(-1)


def subtrees(parent, size):
    """Every node set of `size` nodes that contains each member's parent."""
    n = len(parent)
    for combo in itertools.combinations(range(n), size):
        s = set(combo)
        if all(parent[v] < 0 or parent[v] in s for v in s):
            yield combo


def test_worked_example_on_the_pages_staircase():
    us = pages_staircase()
    parent, p = synth.draft_tree(31, shape="chain")
    p[:] = 0.8
    n, kept, e, rate = oc.cut(us, parent, p)
    exp, rates = golden_values("expected"), golden_values("rate")
    choice = int(read_golden(GOLDEN)["choice"][0])
    assert n == choice == 15 and kept == list(range(15))
    for size in (7, 15, 23, 31):
        n2, _, e2, r2 = oc.cut(us, parent, p, sizes=(size,))
        assert n2 == size
        assert e2 == pytest.approx(exp[size], rel=1e-14)
        assert r2 == pytest.approx(rates[size], rel=1e-14)


@pytest.mark.parametrize("seed", range(12))
def test_cut_reaches_the_bruteforce_optimum(seed):
    n = 7
    shape = ("random", "wide", "chain")[seed % 3]
    parent, p = synth.draft_tree(n, seed=seed, shape=shape)
    for size in range(1, n + 1):
        best = max(walk_expected(parent, p, s) for s in subtrees(parent, size))
        k, kept, e, _ = oc.cut(np.full(n + 1, 100.0), parent, p, sizes=(size,))
        assert k == size
        assert all(parent[v] < 0 or parent[v] in kept for v in kept), "cut is not a subtree"
        assert e == pytest.approx(best, rel=1e-12, abs=1e-15)
        assert walk_expected(parent, p, kept) == pytest.approx(e, rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("seed", range(12))
def test_choice_is_the_bruteforce_argmax(seed):
    n = 7
    parent, p = synth.draft_tree(n, seed=100 + seed)
    us = synth.staircase_us(16, seed=seed, step_rows=3, step=0.6)
    sizes = (1, 3, 5, 7)
    rates = {}
    for size in sizes:
        best = max(walk_expected(parent, p, s) for s in subtrees(parent, size))
        rates[size] = best / (us[size] * 1e-3)
    want = min(sizes, key=lambda s: (-rates[s], s))
    k, _, _, r = oc.cut(us, parent, p, sizes=sizes)
    assert k == want
    assert r == pytest.approx(rates[want], rel=1e-12)


def test_closed_forms():
    parent, p = synth.draft_tree(31, shape="random", seed=5)
    us = synth.staircase_us(32, seed=1)
    zero = np.zeros_like(p)
    n, _, e, rate = oc.cut(us, parent, zero)
    assert e == 1.0
    cheapest = min((7, 15, 23, 31), key=lambda s: (us[s], s))
    assert n == cheapest and rate == 1.0 / (us[n] * 1e-3)
    chain, _ = synth.draft_tree(31, shape="chain")
    one = np.ones(31)
    for size in (7, 15, 23, 31):
        assert oc.cut(us, chain, one, sizes=(size,))[2] == size + 1.0
    # a tree smaller than the candidates is kept whole
    par5, p5 = synth.draft_tree(5, seed=3)
    n, kept, _, _ = oc.cut(us, par5, p5)
    assert n == 5 and kept == list(range(5))


@pytest.mark.parametrize("seed", range(20))
def test_library_cut_matches_oracle(seed):
    shape = ("random", "wide", "chain")[seed % 3]
    n_nodes = (31, 20, 31, 5, 31)[seed % 5]
    parent, p = synth.draft_tree(n_nodes, seed=seed, shape=shape)
    us = synth.staircase_us(64, seed=seed, step_rows=(8, 16, 4)[seed % 3])
    n, keep, e, rate = nv.staircut(us, parent, p)
    n2, kept2, e2, rate2 = oc.cut(us, parent, p)
    assert n == n2
    assert sorted(np.nonzero(keep)[0].tolist()) == kept2
    assert e == pytest.approx(e2, rel=1e-15) and rate == pytest.approx(rate2, rel=1e-15)


def test_library_cut_on_the_pages_staircase():
    us = pages_staircase()
    parent, p = synth.draft_tree(31, shape="chain")
    p[:] = 0.8
    n, keep, e, rate = nv.staircut(us, parent, p)
    assert n == 15 and keep.tolist() == [1] * 15 + [0] * 16
    assert e == pytest.approx(golden_values("expected")[15], rel=1e-14)


def test_library_cut_argument_errors():
    us = synth.staircase_us(32)
    parent, p = synth.draft_tree(31)
    with pytest.raises(nv.Nvfp4vError) as ei:
        nv.staircut(us, np.array([0], np.int32), np.array([0.5]))  # a node cannot be its own parent
    assert ei.value.status == nv.E_SHAPE
    bad = p.copy()
    bad[3] = 1.5
    with pytest.raises(nv.Nvfp4vError) as ei:
        nv.staircut(us, parent, bad)
    assert ei.value.status == nv.E_INVALID_ARG
    with pytest.raises(nv.Nvfp4vError) as ei:  # two children of the root summing above 1
        nv.staircut(us, np.array([-1, -1], np.int32), np.array([0.7, 0.6]))
    assert ei.value.status == nv.E_INVALID_ARG
    with pytest.raises(nv.Nvfp4vError) as ei:  # 31 nodes need 32 rows
        nv.staircut(us[:20], parent, p)
    assert ei.value.status == nv.E_M_RANGE
    holes = us.copy()
    holes[15] = 0.0
    with pytest.raises(nv.Nvfp4vError) as ei:
        nv.staircut(holes, parent, p)
    assert ei.value.status == nv.E_INVALID_ARG
