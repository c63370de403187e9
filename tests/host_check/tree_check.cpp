// Drives the library's host-side tree code (tree.cpp, built here with the
// address and undefined-behaviour sanitizers) from text commands on stdin,
// one per line, and prints what the calls return, one line per command:
//
//   tree K k P  len r0 .. r(len-1)  [P paths]  -> status and every node array
//   dense K k                                  -> status and the path list
//   greedy K cap n  a(0,0) .. a(K-1,cap-1)     -> status and the path list
//   errors                                     -> statuses of calls with NULL /
//                                                 out-of-range arguments
//
// The tests compare the printed arrays with the oracle's and the statuses
// with the documented error classes.  Test infrastructure only.
#include <stdio.h>

#include <string>
#include <vector>

#include "medusa.h"
#include "tree.h"

namespace {

template <typename T>
void print_array(const char *name, const std::vector<T> &v) {
  printf(" %s=", name);
  for (size_t i = 0; i < v.size(); ++i) printf(i ? ",%lld" : "%lld", static_cast<long long>(v[i]));
}

void print_paths(medusa_status s, int K, int n, const std::vector<int32_t> &ranks, const std::vector<int32_t> &len) {
  printf("status=%d n=%d paths=", static_cast<int>(s), n);
  if (s == MEDUSA_OK)
    for (int p = 0; p < n; ++p) {
      printf(p ? ";" : "");
      for (int d = 0; d < len[p]; ++d) printf(d ? ".%d" : "%d", ranks[static_cast<size_t>(p) * K + d]);
    }
  printf("\n");
}

void cmd_tree() {
  int K = 0, k = 0, P = 0;
  if (scanf("%d %d %d", &K, &k, &P) != 3 || K < 1 || P < 0 || P > 100000) {
    printf("bad command\n");
    return;
  }
  std::vector<int32_t> ranks(static_cast<size_t>(P) * K, 0), len(P, 0);
  for (int p = 0; p < P; ++p) {
    int l = 0;
    if (scanf("%d", &l) != 1) return;
    len[p] = l;
    for (int d = 0; d < l; ++d) {
      int r = 0;
      if (scanf("%d", &r) != 1) return;
      if (d < K) ranks[static_cast<size_t>(p) * K + d] = r;  // longer paths are cut here; len says the truth
    }
  }
  medusa_tree *t = nullptr;
  const medusa_status s = medusa_build_tree(P ? ranks.data() : nullptr, P ? len.data() : nullptr, P, K, k, &t);
  printf("status=%d", static_cast<int>(s));
  if (s == MEDUSA_OK) {
    int T = 0, W = 0, D = 0, nl = 0;
    medusa_tree_mask(t, &T, &W, &D, &nl, nullptr, nullptr, nullptr, nullptr, nullptr);
    std::vector<uint64_t> mask(static_cast<size_t>(T) * W);
    std::vector<int32_t> parent(T), depth(T), rank(T), retrieve(static_cast<size_t>(nl) * (D + 1)), pos(T);
    medusa_tree_mask(t, &T, &W, &D, &nl, mask.data(), parent.data(), depth.data(), rank.data(), retrieve.data());
    medusa_tree_positions(t, 100, pos.data());
    printf(" T=%d W=%d D=%d leaves=%d", T, W, D, nl);
    printf(" mask=");
    for (size_t i = 0; i < mask.size(); ++i) printf(i ? ",%llx" : "%llx", static_cast<unsigned long long>(mask[i]));
    print_array("parent", parent);
    print_array("depth", depth);
    print_array("rank", rank);
    print_array("retrieve", retrieve);
    print_array("pos100", pos);
    medusa::tree_delete_host(t);
  }
  printf("\n");
}

void cmd_dense() {
  int K = 0, k = 0;
  if (scanf("%d %d", &K, &k) != 2) return;
  int n = 0;
  medusa_status s = medusa_dense_paths(K, k, 0, nullptr, nullptr, &n);
  std::vector<int32_t> ranks, len;
  if (s == MEDUSA_OK) {
    ranks.assign(static_cast<size_t>(n) * K, 0);
    len.assign(n, 0);
    s = medusa_dense_paths(K, k, n, ranks.data(), len.data(), &n);
  }
  print_paths(s, K, n, ranks, len);
}

void cmd_greedy() {
  int K = 0, cap = 0, n = 0;
  if (scanf("%d %d %d", &K, &cap, &n) != 3 || K < 1 || cap < 1 || K * cap > 100000 || n < 0 || n > 100000) return;
  std::vector<double> acc(static_cast<size_t>(K) * cap);
  for (double &a : acc)
    if (scanf("%lf", &a) != 1) return;
  std::vector<int32_t> ranks(static_cast<size_t>(n) * K + 1, 0), len(n + 1, 0);
  const medusa_status s = medusa_greedy_paths(acc.data(), K, cap, n, ranks.data(), len.data());
  print_paths(s, K, n, ranks, len);
}

void cmd_errors() {
  const int32_t r1[2] = {0, 0}, l1[1] = {1};
  medusa_tree *t = nullptr;
  int n = 0, T = 0;
  int32_t pos[4];
  double acc[2] = {0.5, 0.25};
  int32_t rk[8], ln[8];
  const int codes[] = {
      medusa_build_tree(r1, l1, 1, 2, 2, nullptr),            // out NULL
      medusa_build_tree(nullptr, l1, 1, 2, 2, &t),            // ranks NULL
      medusa_build_tree(r1, l1, -1, 2, 2, &t),                // negative count
      medusa_build_tree(r1, l1, 1, 0, 2, &t),                 // K = 0
      medusa_build_tree(r1, l1, 1, 2, 65, &t),                // k above the limit
      medusa_tree_mask(nullptr, &T, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
      medusa_tree_positions(nullptr, 0, pos),
      medusa_dense_paths(0, 2, 0, nullptr, nullptr, &n),      // K = 0
      medusa_dense_paths(5, 5, 0, nullptr, nullptr, &n),      // 3905 paths: above the tree limit
      medusa_dense_paths(2, 2, 3, rk, ln, &n),                // capacity 3 < 6
      medusa_dense_paths(2, 2, 6, rk, nullptr, &n),           // one output NULL
      medusa_greedy_paths(nullptr, 1, 2, 1, rk, ln),          // acc NULL
      medusa_greedy_paths(acc, 1, 2, 3, rk, ln),              // only 2 paths exist
      medusa_greedy_paths(acc, 1, 2, 1024, rk, ln),           // above the tree limit
  };
  printf("status=0 codes=");
  for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i) printf(i ? ",%d" : "%d", codes[i]);
  printf("\n");
}

}  // namespace

int main() {
  char cmd[32];
  while (scanf("%31s", cmd) == 1) {
    const std::string c(cmd);
    if (c == "tree")
      cmd_tree();
    else if (c == "dense")
      cmd_dense();
    else if (c == "greedy")
      cmd_greedy();
    else if (c == "errors")
      cmd_errors();
    else {
      printf("unknown command %s\n", cmd);
      return 2;
    }
    fflush(stdout);
  }
  return 0;
}
