// KV-cache commit after acceptance: the accepted path root..best of every
// sequence is appended to its prefix cache, in depth order, so the next step
// attends to the accepted tokens as ordinary prefix keys; the sequence length
// advances by the rows written and the next root becomes the greedy token
// after the accepted prefix.
//
// One block per sequence.  Thread 0 walks best's parent chain (at most
// depth_max steps) into LDS, then the block copies the path's K and V rows
// for every head in 16-byte chunks; the length is updated after the copy, so
// no other block ever reads a half-updated length.
#include "common.h"

using namespace medusa;

namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void kv_commit_kernel(
    int T, int nh, int row_chunks, int L_cap, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ depth, const u32x4_t *__restrict__ kt, const u32x4_t *__restrict__ vt,
    const int32_t *__restrict__ best_node, int32_t *__restrict__ seq_len, u32x4_t *__restrict__ kc,
    u32x4_t *__restrict__ vc, const int32_t *__restrict__ next_tok, int32_t *__restrict__ root_tok) {
  __shared__ int path[MEDUSA_MAX_TREE];
  __shared__ int n_rows, L0;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) {
    const int best = best_node[b];
    const int len = seq_len[b];
    int n = 0;
    if (best >= 0 && best < T && len >= 0 && len <= L_cap) {
      // path[d] = the ancestor of best at depth d (best itself at its depth)
      const int d_best = depth[best];
      for (int j = best, d = d_best; d >= 0; j = parent[j], --d) path[d] = j;
      n = d_best + 1;
      if (n > L_cap - len) n = L_cap - len;   // rows that do not fit are dropped
    }
    n_rows = n;
    L0 = len;
  }
  __syncthreads();
  const int n = n_rows, base = L0;
  const int per_row = nh * row_chunks;
  for (int i = threadIdx.x; i < n * per_row; i += kThreads) {
    const int r = i / per_row, h = (i / row_chunks) % nh, c = i % row_chunks;
    const size_t src = (((size_t)b * T + path[r]) * nh + h) * row_chunks + c;
    const size_t dst = (((size_t)b * nh + h) * L_cap + base + r) * row_chunks + c;
    kc[dst] = kt[src];
    vc[dst] = vt[src];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    seq_len[b] = base + n;
    if (next_tok && root_tok) root_tok[b] = next_tok[b];
  }
}

}  // namespace

extern "C" medusa_status medusa_kv_commit(medusa_stream_t stream, medusa_dtype dt, const medusa_tree *t, int B,
                                          int nh, int dh, int L_cap, const void *k_tree, const void *v_tree,
                                          const int32_t *best_node, int32_t *seq_len, void *k_cache,
                                          void *v_cache, const int32_t *next_tok, int32_t *root_tok) {
  TraceRange tr("medusa_kv_commit");
  medusa_status s = check_tree_on_device(t);
  if (s != MEDUSA_OK) return s;
  if (dt != MEDUSA_F32 && dt != MEDUSA_BF16) return fail(MEDUSA_ERR_ARG, "medusa_kv_commit: unknown dtype");
  if (B < 1 || nh < 1 || dh < 1 || L_cap < 1)
    return fail(MEDUSA_ERR_ARG, "medusa_kv_commit: B=%d nh=%d dh=%d L_cap=%d", B, nh, dh, L_cap);
  const int esize = dt == MEDUSA_BF16 ? 2 : 4;
  if ((dh * esize) % 16 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "medusa_kv_commit: dh*elem %% 16 != 0 (dh=%d)", dh);
  if (!k_tree || !v_tree || !best_node || !seq_len || !k_cache || !v_cache)
    return fail(MEDUSA_ERR_ARG, "medusa_kv_commit: NULL pointer");
  if ((next_tok == nullptr) != (root_tok == nullptr))
    return fail(MEDUSA_ERR_ARG, "medusa_kv_commit: next_tok and root_tok go together");
  if (!aligned16(k_tree) || !aligned16(v_tree) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(MEDUSA_ERR_ARG, "medusa_kv_commit: K/V pointers must be 16-byte aligned");
  MEDUSA_LAUNCH("medusa_kv_commit", kv_commit_kernel, dim3(B), dim3(kThreads), 0, as_stream(stream), t->T, nh, dh * esize / 16,
                     L_cap, t->d_parent, t->d_depth, static_cast<const u32x4_t *>(k_tree),
                     static_cast<const u32x4_t *>(v_tree), best_node, seq_len, static_cast<u32x4_t *>(k_cache),
                     static_cast<u32x4_t *>(v_cache), next_tok, root_tok);
  return check_launch("medusa_kv_commit");
}
