// Host-only part of the library: the candidate tree's arrays and error
// reporting.  No HIP header is needed here, so tree.cpp also builds as plain
// C++ (the sanitizer build the CPU tests drive).
#pragma once

#include <stdint.h>

#include <vector>

#include "medusa.h"

// Candidate tree: host arrays plus one device copy (see medusa_tree_upload).
struct medusa_tree {
  int K = 0, k = 0, T = 0, W = 0, depth_max = 0, n_leaves = 0, n_internal = 0;
  std::vector<int32_t> parent, depth, rank, retrieve;
  std::vector<int32_t> internal;  // nodes with children, ascending
  std::vector<int32_t> slot;      // node -> index in `internal`, -1 for leaves
  std::vector<int32_t> dstart;    // [depth_max + 2]: nodes of depth d are dstart[d] .. dstart[d+1]-1
  // children of node u, ascending (rank order): clist[cstart[u] .. cstart[u+1])
  std::vector<int32_t> cstart;    // [T + 1]
  std::vector<int32_t> clist;     // [T - 1]
  std::vector<uint64_t> mask;     // [T][W]
  // per group of 16 consecutive nodes: bit w set iff some node of the group
  // has an ancestor (or is itself) among nodes 64w .. 64w+63
  std::vector<uint32_t> tile_need;  // [ceil(T/16)]
  // device copy (valid after upload; owned by the HIP side of the library)
  void *d_base = nullptr;
  int device = -1;
  const uint64_t *d_mask = nullptr;
  const int32_t *d_parent = nullptr, *d_depth = nullptr, *d_rank = nullptr;
  const int32_t *d_internal = nullptr, *d_slot = nullptr, *d_dstart = nullptr;
  const uint32_t *d_tile_need = nullptr;
  const int32_t *d_cstart = nullptr, *d_clist = nullptr;
};

namespace medusa {

// Record the thread-local error text of a non-OK status and return it.
medusa_status fail(medusa_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
// Release the host arrays of a tree (its device copy must be gone already).
void tree_delete_host(medusa_tree *t);

}  // namespace medusa
