// Candidate trees on the host: path lists (dense and greedy sparse),
// validation, node arrays, ancestor bitmask, retrieve table and positions;
// and the library's error reporting.  Plain C++ with no HIP dependency, so the
// same source also builds with the address and undefined-behaviour
// sanitizers for the CPU tests.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <new>
#include <queue>
#include <string>

#include "tree.h"

namespace medusa {

static thread_local std::string g_last_error;

medusa_status fail(medusa_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

void clear_error() { g_last_error.clear(); }

void tree_delete_host(medusa_tree *t) { delete t; }

}  // namespace medusa

using medusa::fail;

extern "C" const char *medusa_last_error(void) { return medusa::g_last_error.c_str(); }
extern "C" int medusa_abi_version(void) { return MEDUSA_ABI_VERSION; }

using Path = std::vector<int32_t>;

// (length, lexicographic) order of rank paths
static bool path_less(const Path &a, const Path &b) {
  if (a.size() != b.size()) return a.size() < b.size();
  return a < b;
}

extern "C" medusa_status medusa_dense_paths(int K, int k, int cap, int32_t *ranks,
                                            int32_t *path_len, int *n_paths) {
  if (K < 1 || k < 1) return fail(MEDUSA_ERR_ARG, "dense_paths: K=%d k=%d must be >= 1", K, k);
  double total = 0, p = 1;
  for (int d = 1; d <= K; ++d) {
    p *= k;
    total += p;
  }
  if (total > MEDUSA_MAX_TREE - 1)
    return fail(MEDUSA_ERR_UNSUPPORTED, "dense_paths: %.0f paths exceed the tree limit %d", total,
                MEDUSA_MAX_TREE - 1);
  const int n = static_cast<int>(total);
  if (n_paths) *n_paths = n;
  if (!ranks && !path_len) return MEDUSA_OK;  // size query
  if (!ranks || !path_len) return fail(MEDUSA_ERR_ARG, "dense_paths: NULL output");
  if (cap < n) return fail(MEDUSA_ERR_ARG, "dense_paths: capacity %d < %d paths", cap, n);
  int out = 0;
  for (int d = 1; d <= K; ++d) {
    std::vector<int32_t> digits(d, 0);
    while (true) {
      for (int i = 0; i < K; ++i) ranks[out * K + i] = i < d ? digits[i] : 0;
      path_len[out++] = d;
      int pos = d - 1;  // odometer, last digit fastest: lexicographic order
      while (pos >= 0 && ++digits[pos] == k) digits[pos--] = 0;
      if (pos < 0) break;
    }
  }
  return MEDUSA_OK;
}

extern "C" medusa_status medusa_greedy_paths(const double *acc, int K, int rank_cap, int n_paths,
                                             int32_t *ranks, int32_t *path_len) {
  if (!acc || !ranks || !path_len) return fail(MEDUSA_ERR_ARG, "greedy_paths: NULL pointer");
  if (K < 1 || rank_cap < 1 || n_paths < 0)
    return fail(MEDUSA_ERR_ARG, "greedy_paths: K=%d rank_cap=%d n_paths=%d", K, rank_cap, n_paths);
  if (n_paths > MEDUSA_MAX_TREE - 1)
    return fail(MEDUSA_ERR_UNSUPPORTED, "greedy_paths: %d paths exceed the tree limit", n_paths);
  for (int i = 0; i < K * rank_cap; ++i)
    if (!(acc[i] > 0.0 && acc[i] <= 1.0))
      return fail(MEDUSA_ERR_ARG, "greedy_paths: accuracy %d = %g outside (0, 1]", i, acc[i]);
  struct Cand {
    double score;
    Path path;
  };
  // best first: larger gain; gains within 1e-12 (relative) are equal and then
  // the shorter, then the lexicographically smaller path wins
  auto worse = [](const Cand &a, const Cand &b) {
    const double tol = 1e-12 * std::max(a.score, b.score);
    if (std::fabs(a.score - b.score) > tol) return a.score < b.score;
    return path_less(b.path, a.path);
  };
  std::priority_queue<Cand, std::vector<Cand>, decltype(worse)> frontier(worse);
  for (int i = 0; i < rank_cap; ++i) frontier.push({acc[i], Path{i}});
  for (int n = 0; n < n_paths; ++n) {
    if (frontier.empty()) return fail(MEDUSA_ERR_TREE, "greedy_paths: only %d paths exist", n);
    Cand c = frontier.top();
    frontier.pop();
    for (int d = 0; d < K; ++d) ranks[n * K + d] = d < (int)c.path.size() ? c.path[d] : 0;
    path_len[n] = static_cast<int32_t>(c.path.size());
    const int d = static_cast<int>(c.path.size());
    if (d < K)
      for (int i = 0; i < rank_cap; ++i) {
        Path p = c.path;
        p.push_back(i);
        frontier.push({c.score * acc[d * rank_cap + i], std::move(p)});
      }
  }
  return MEDUSA_OK;
}

extern "C" medusa_status medusa_build_tree(const int32_t *ranks, const int32_t *path_len,
                                           int n_paths, int K, int k, medusa_tree **out) {
  if (!out) return fail(MEDUSA_ERR_ARG, "build_tree: out is NULL");
  *out = nullptr;
  if (n_paths < 0 || (n_paths > 0 && (!ranks || !path_len)))
    return fail(MEDUSA_ERR_ARG, "build_tree: bad path arrays");
  if (K < 1 || k < 1) return fail(MEDUSA_ERR_ARG, "build_tree: K=%d k=%d must be >= 1", K, k);
  if (k > MEDUSA_MAX_TOPK) return fail(MEDUSA_ERR_UNSUPPORTED, "build_tree: k=%d > %d", k, MEDUSA_MAX_TOPK);
  if (n_paths + 1 > MEDUSA_MAX_TREE)
    return fail(MEDUSA_ERR_UNSUPPORTED, "build_tree: T=%d > %d", n_paths + 1, MEDUSA_MAX_TREE);
  std::vector<Path> paths;
  paths.reserve(n_paths);
  for (int p = 0; p < n_paths; ++p) {
    const int len = path_len[p];
    if (len < 1 || len > K) return fail(MEDUSA_ERR_TREE, "path %d: length %d outside [1, %d]", p, len, K);
    Path v(ranks + static_cast<size_t>(p) * K, ranks + static_cast<size_t>(p) * K + len);
    for (int32_t r : v)
      if (r < 0 || r >= k) return fail(MEDUSA_ERR_TREE, "path %d: rank %d outside [0, %d)", p, r, k);
    paths.push_back(std::move(v));
  }
  std::sort(paths.begin(), paths.end(), path_less);
  for (size_t i = 1; i < paths.size(); ++i)
    if (paths[i] == paths[i - 1]) return fail(MEDUSA_ERR_TREE, "duplicate path");
  std::map<Path, int> index;
  index[Path{}] = 0;
  for (size_t i = 0; i < paths.size(); ++i) index[paths[i]] = static_cast<int>(i) + 1;

  medusa_tree *t = new (std::nothrow) medusa_tree();
  if (!t) return fail(MEDUSA_ERR_ARG, "build_tree: out of host memory");
  t->K = K;
  t->k = k;
  t->T = n_paths + 1;
  t->W = (t->T + 63) / 64;
  t->parent.assign(t->T, -1);
  t->depth.assign(t->T, 0);
  t->rank.assign(t->T, -1);
  for (int j = 1; j < t->T; ++j) {
    const Path &p = paths[j - 1];
    Path pre(p.begin(), p.end() - 1);
    auto it = index.find(pre);
    if (it == index.end()) {
      delete t;
      return fail(MEDUSA_ERR_TREE, "a path of length %zu lacks its prefix", p.size());
    }
    t->parent[j] = it->second;
    t->depth[j] = static_cast<int32_t>(p.size());
    t->rank[j] = p.back();
  }
  // ancestor bitmask: walk each node's parent chain
  t->mask.assign(static_cast<size_t>(t->T) * t->W, 0);
  for (int j = 0; j < t->T; ++j)
    for (int i = j; i != -1; i = t->parent[i]) t->mask[static_cast<size_t>(j) * t->W + i / 64] |= 1ull << (i % 64);
  t->tile_need.assign((t->T + 15) / 16, 0u);
  for (int j = 0; j < t->T; ++j)
    for (int w = 0; w < t->W; ++w)
      if (t->mask[static_cast<size_t>(j) * t->W + w]) t->tile_need[j / 16] |= 1u << w;
  std::vector<char> has_child(t->T, 0);
  for (int j = 1; j < t->T; ++j) has_child[t->parent[j]] = 1;
  t->slot.assign(t->T, -1);
  for (int j = 0; j < t->T; ++j)
    if (has_child[j]) {
      t->slot[j] = static_cast<int32_t>(t->internal.size());
      t->internal.push_back(j);
    }
  t->n_internal = static_cast<int>(t->internal.size());
  t->cstart.assign(t->T + 1, 0);
  for (int j = 1; j < t->T; ++j) ++t->cstart[t->parent[j] + 1];
  for (int j = 0; j < t->T; ++j) t->cstart[j + 1] += t->cstart[j];
  t->clist.assign(t->T - 1, 0);
  {
    std::vector<int32_t> next(t->cstart.begin(), t->cstart.end() - 1);
    for (int j = 1; j < t->T; ++j) t->clist[next[t->parent[j]]++] = j;
  }
  t->depth_max = *std::max_element(t->depth.begin(), t->depth.end());
  t->dstart.assign(t->depth_max + 2, t->T);  // nodes are sorted by depth
  for (int j = t->T - 1; j >= 0; --j) t->dstart[t->depth[j]] = j;
  const int R = t->depth_max + 1;
  for (int j = 0; j < t->T; ++j)
    if (!has_child[j]) {
      std::vector<int32_t> row(R, -1);
      std::vector<int32_t> chain;
      for (int i = j; i != -1; i = t->parent[i]) chain.push_back(i);
      std::reverse(chain.begin(), chain.end());
      std::copy(chain.begin(), chain.end(), row.begin());
      t->retrieve.insert(t->retrieve.end(), row.begin(), row.end());
      ++t->n_leaves;
    }
  *out = t;
  return MEDUSA_OK;
}

extern "C" medusa_status medusa_tree_mask(const medusa_tree *t, int *T, int *W, int *depth_max,
                                          int *n_leaves, uint64_t *mask, int32_t *parent,
                                          int32_t *depth, int32_t *rank, int32_t *retrieve) {
  if (!t) return fail(MEDUSA_ERR_ARG, "tree_mask: tree is NULL");
  if (T) *T = t->T;
  if (W) *W = t->W;
  if (depth_max) *depth_max = t->depth_max;
  if (n_leaves) *n_leaves = t->n_leaves;
  if (mask) std::copy(t->mask.begin(), t->mask.end(), mask);
  if (parent) std::copy(t->parent.begin(), t->parent.end(), parent);
  if (depth) std::copy(t->depth.begin(), t->depth.end(), depth);
  if (rank) std::copy(t->rank.begin(), t->rank.end(), rank);
  if (retrieve) std::copy(t->retrieve.begin(), t->retrieve.end(), retrieve);
  return MEDUSA_OK;
}

extern "C" medusa_status medusa_tree_positions(const medusa_tree *t, int L, int32_t *pos) {
  if (!t || !pos) return fail(MEDUSA_ERR_ARG, "tree_positions: NULL pointer");
  if (L < 0) return fail(MEDUSA_ERR_ARG, "tree_positions: L=%d < 0", L);
  for (int j = 0; j < t->T; ++j) pos[j] = L + t->depth[j];
  return MEDUSA_OK;
}

