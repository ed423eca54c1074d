// StairCut's cut rule: given a candidate draft tree with a per-node acceptance
// probability and the measured price of a verify pass per row count (the
// staircase this library measures), keep the node count, among a few
// tile-aligned sizes, that commits the most expected tokens per millisecond
// (StairCut research page, "What it says": every round is priced on the
// measured staircase and keeps the tree size that pays the most expected
// tokens per millisecond; release post: the candidate tree is cut to the node
// count with the most expected committed tokens per millisecond at the
// measured price, snapping to 7, 15, 23 or 31 nodes).
//
// Reading of the pages (which give no formula):
//  * Node v of the tree carries p(v), the probability that the model's own
//    token at v's position is v's token given that v's parent was accepted.
//    Siblings are different tokens at one position, so at most one of them is
//    the model's: the probabilities of a node's children sum to at most 1.
//  * The model accepts the longest path of agreeing guesses and then writes
//    its own token (TandemLLM manual, "What TandemLLM is", 1.2 "Two levers":
//    at the first wrong guess the model puts in its own token). A round with a
//    kept set K therefore commits 1 + |accepted path| tokens, and
//    E = 1 + sum over v in K of P(v), P(v) = product of p along the root path
//    of v (v is accepted exactly when its whole path is).
//  * A cut to n nodes keeps the n nodes of highest P. P never increases along
//    a path, so those nodes form a subtree that contains the root, and no
//    other n-node subtree has a larger sum.
//  * The verify pass checks the kept nodes plus the root's token: n + 1 rows,
//    priced at the staircase's time for n + 1 rows. Trees smaller than a
//    candidate size are kept whole (that candidate becomes the tree's size).
//  * Equal rates keep the smaller tree.
// Host code only: it runs on the CPU between rounds, on numbers the GPU
// measured.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/nvfp4v.h"

namespace {

const int32_t kDefaultSizes[4] = {7, 15, 23, 31};

}  // namespace

extern "C" int nvfp4v_staircut(const double *us_by_rows, int max_rows, const int32_t *parent,
                               const double *p_accept, int n_nodes, const int32_t *sizes, int n_sizes,
                               int32_t *n_keep, uint8_t *keep, double *expected_tokens,
                               double *tokens_per_ms) {
  if (!us_by_rows || !parent || !p_accept || !n_keep || !keep) return NVFP4V_E_INVALID_ARG;
  if (n_nodes < 1 || n_nodes > NVFP4V_STAIRCUT_MAX_NODES || max_rows < 1) return NVFP4V_E_SHAPE;
  if (!sizes) {
    sizes = kDefaultSizes;
    n_sizes = 4;
  }
  if (n_sizes < 1 || n_sizes > 64) return NVFP4V_E_SHAPE;
  for (int i = 0; i < n_sizes; ++i)
    if (sizes[i] < 1) return NVFP4V_E_SHAPE;
  // The tree: parents precede their children; -1 is the root (the last
  // committed token). The children's probabilities of every node sum to <= 1.
  std::vector<double> child_sum((size_t)n_nodes + 1, 0.0);  // [0] is the root
  for (int v = 0; v < n_nodes; ++v) {
    const int32_t u = parent[v];
    const double p = p_accept[v];
    if (u < -1 || u >= v) return NVFP4V_E_SHAPE;
    if (!(p >= 0.0 && p <= 1.0)) return NVFP4V_E_INVALID_ARG;
    child_sum[(size_t)(u + 1)] += p;
  }
  for (double s : child_sum)
    if (s > 1.0 + 1e-9) return NVFP4V_E_INVALID_ARG;

  // Path probabilities, in node order (a parent's is known before its child's).
  std::vector<double> P((size_t)n_nodes);
  for (int v = 0; v < n_nodes; ++v) P[(size_t)v] = parent[v] < 0 ? p_accept[v] : P[(size_t)parent[v]] * p_accept[v];
  // Nodes by decreasing P, earlier node first on ties (a parent precedes a
  // child of equal P), so every prefix of the order is a subtree.
  std::vector<int32_t> order((size_t)n_nodes);
  for (int v = 0; v < n_nodes; ++v) order[(size_t)v] = v;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return P[(size_t)a] > P[(size_t)b]; });
  // Expected tokens of each prefix: 1 + the sum of its P, added in that order.
  std::vector<double> E((size_t)n_nodes + 1);
  E[0] = 1.0;
  for (int i = 0; i < n_nodes; ++i) E[(size_t)i + 1] = E[(size_t)i] + P[(size_t)order[(size_t)i]];

  int best_n = -1;
  double best_rate = -1.0;
  for (int i = 0; i < n_sizes; ++i) {
    const int n = std::min<int>(sizes[i], n_nodes);
    if (n + 1 > max_rows) return NVFP4V_E_M_RANGE;
    const double us = us_by_rows[n];  // price of n + 1 rows (index rows - 1)
    if (!(us > 0.0) || !std::isfinite(us)) return NVFP4V_E_INVALID_ARG;
    const double rate = E[(size_t)n] / (us * 1e-3);
    if (rate > best_rate || (rate == best_rate && n < best_n)) {
      best_rate = rate;
      best_n = n;
    }
  }
  std::memset(keep, 0, (size_t)n_nodes);
  for (int i = 0; i < best_n; ++i) keep[(size_t)order[(size_t)i]] = 1;
  *n_keep = best_n;
  if (expected_tokens) *expected_tokens = E[(size_t)best_n];
  if (tokens_per_ms) *tokens_per_ms = best_rate;
  return NVFP4V_OK;
}
