"""Oracle of StairCut's cut rule (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
CPU-baseline leg may import this module; the product (the HIP library and its
binding) never does, and the two share no code.

What the pages say (StairCut research page, "What it says"; release post,
third paragraph): every round the router builds a candidate draft tree of up to
31 guessed tokens, prices the verify pass on the measured staircase of its cost
per row count, and cuts the tree to the node count with the most expected
committed tokens per millisecond, snapping to 7, 15, 23 or 31 nodes. A guess
the model agrees with is a free token, and at the first wrong guess the model
puts in its own token (TandemLLM manual, "What TandemLLM is", 1.2 "Two
levers"). The pages give no formula; the plainest reading, written out here:

* node v carries p(v): the chance that the model's token at v's position is
  v's token, given that v's parent was accepted. Siblings are different tokens
  at one position, so at most one of them is accepted;
* v is accepted exactly when every node on its root path is, with probability
  P(v) = the product of p along that path;
* the accepted nodes form one path, so a round that keeps the node set K
  commits 1 + (number of accepted nodes in K) tokens, whose mean is
  E(K) = 1 + sum of P(v) over v in K;
* a cut to n nodes keeps the n nodes of largest P (earlier node first on ties):
  P never grows along a path, so those n nodes include every ancestor of each
  of them, and no other n-node subtree has a larger sum;
* the verify pass checks those n nodes plus the root's token, n + 1 rows,
  priced at the staircase's time for n + 1 rows; a tree smaller than a
  candidate size is kept whole;
* the candidate with the largest E / time wins; equal rates keep the smaller
  tree.
"""

from __future__ import annotations

DEFAULT_SIZES = (7, 15, 23, 31)


def path_probabilities(parent, p_accept):
    """P(v) for every node (parents come before their children; -1 = root)."""
    probs = []
    for v in range(len(parent)):
        up = 1.0 if parent[v] < 0 else probs[parent[v]]
        probs.append(float(p_accept[v]) * up)
    return probs


def ranked_nodes(parent, p_accept):
    """Nodes by decreasing path probability, the earlier node first on ties."""
    probs = path_probabilities(parent, p_accept)
    return sorted(range(len(parent)), key=lambda v: (-probs[v], v)), probs


def cut(us_by_rows, parent, p_accept, sizes=DEFAULT_SIZES):
    """The cut: returns (n_keep, kept nodes (sorted), expected committed tokens,
    tokens per millisecond). us_by_rows[r - 1] is the verify time in
    microseconds at r rows."""
    order, probs = ranked_nodes(parent, p_accept)
    best = None
    for size in sizes:
        n = min(int(size), len(parent))
        kept = order[:n]
        expected = 1.0
        for v in kept:  # largest first
            expected += probs[v]
        millis = float(us_by_rows[n]) * 1e-3  # n + 1 rows
        rate = expected / millis
        if best is None or rate > best[3] or (rate == best[3] and n < best[0]):
            best = (n, sorted(kept), expected, rate)
    return best
