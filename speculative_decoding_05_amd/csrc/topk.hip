// Per-row top-k over the vocabulary, and the tree-token gather.
//
// Each element becomes a distinct 64-bit key: the order-preserving image of
// the float (with -0.0 folded onto +0.0) in the high word and the bitwise
// complement of the index in the low word, so that "larger key" means
// "larger value, then smaller index" and every row has exactly one answer.
//
// One block of 1024 threads holds a chunk of up to 32768 elements of a row in
// registers.  The block's 64 groups of 16 lanes each find their largest key;
// the k-th largest of those 64 group maxima, theta, is a lower bound of the
// chunk's k-th largest key (k distinct keys are >= theta), so every answer is
// >= theta.  The keys >= theta (typically a few dozen) are appended to LDS and
// each is ranked exactly by counting the larger candidates; rank r < k goes to
// output slot r.  Should the candidate set overflow LDS, the block falls back
// to k rounds of block-wide max extraction.  Rows longer than one chunk write
// per-chunk candidates that a second kernel merges by the same extraction.
#include "common.h"

using namespace medusa;

namespace {

constexpr int kThreads = 256;               // merge kernel
constexpr int kPerThread = 8;
constexpr int kMergeMax = kThreads * kPerThread;  // candidates the merge can hold

__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  const uint32_t mono = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(mono) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int off) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), off);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), off);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// k rounds: each round finds the block-wide largest remaining key, removes it
// from its (unique) owner and appends it to out[] (written by thread 0).
template <int NT, int E>
__device__ void block_extract(uint64_t (&keys)[E], int k, uint64_t *out, uint64_t (*s_wave)[NT / 64]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int round = 0; round < k; ++round) {
    uint64_t best = 0;
    int bi = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (keys[e] > best) {
        best = keys[e];
        bi = e;
      }
    uint64_t w = best;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint64_t o = shfl_xor_u64(w, off);
      w = o > w ? o : w;
    }
    uint64_t *buf = s_wave[round & 1];  // alternate buffers: one barrier per round
    if (lane == 0) buf[wave] = w;
    __syncthreads();
    uint64_t g = buf[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) g = buf[i] > g ? buf[i] : g;
    if (g != 0 && best == g) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (e == bi) keys[e] = 0;
    }
    if (threadIdx.x == 0) out[round] = g;
  }
}

// Optional tree-token scatter: the block that finishes row (head, b) writes the
// tokens of every node at depth head+1 (its rank-th candidate), and the head-0
// block also writes the root token.  Each node is written by exactly one block.
struct TokenScatter {
  int32_t *tree_tok;  // [B][T] or nullptr
  const int32_t *rank, *dstart, *root;
  int B, T, depth_max;
};

__device__ __forceinline__ void scatter_tokens(const TokenScatter &ts, int row, const uint64_t *s_out) {
  if (!ts.tree_tok) return;
  const int head = row / ts.B, b = row % ts.B;
  if (head + 1 > ts.depth_max) return;
  const int j0 = ts.dstart[head + 1], j1 = ts.dstart[head + 2];
  for (int j = j0 + (int)threadIdx.x; j < j1; j += blockDim.x)
    ts.tree_tok[(size_t)b * ts.T + j] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(s_out[ts.rank[j]]));
  if (head == 0 && threadIdx.x == 0) ts.tree_tok[(size_t)b * ts.T] = ts.root[b];
}

constexpr int kFThreads = 1024;
constexpr int kFE = 32;
constexpr int kFChunk = kFThreads * kFE;  // 32768 elements per block
constexpr int kCandMax = 1024;

__global__ __launch_bounds__(kFThreads) void topk_chunk(const float *__restrict__ logits, int V, int k,
                                                        int nchunks, int32_t *__restrict__ idx,
                                                        float *__restrict__ val,
                                                        uint64_t *__restrict__ part, TokenScatter ts) {
  __shared__ uint64_t s_gmax[kFThreads / 16];
  __shared__ uint64_t s_cand[kCandMax];
  __shared__ uint64_t s_out[MEDUSA_MAX_TOPK];
  __shared__ uint64_t s_wave[2][kFThreads / 64];
  __shared__ uint64_t s_theta;
  __shared__ int s_cnt;
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x, row = blockIdx.y;
  const float *z = logits + (size_t)row * V;
  const int base = chunk * kFChunk;
  // values stay in registers as floats; keys are rebuilt from (value, index).
  // Element e of this thread is index base + (e/4)*4096 + 4*tid + e%4, read
  // as float4 when the row allows it.
  float v[kFE];
  const bool vec = (V % 4) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0;
#pragma unroll
  for (int g = 0; g < kFE / 4; ++g) {
    const int i0 = base + g * 4 * kFThreads + 4 * tid;
    if (vec && i0 + 3 < V) {
      const float4 f = *reinterpret_cast<const float4 *>(z + i0);
      v[4 * g] = f.x;
      v[4 * g + 1] = f.y;
      v[4 * g + 2] = f.z;
      v[4 * g + 3] = f.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * g + j] = i0 + j < V ? z[i0 + j] : 0.f;
    }
  }
  auto index_of = [&](int e) { return base + (e >> 2) * 4 * kFThreads + 4 * tid + (e & 3); };
  auto key_of = [&](int e) -> uint64_t {
    const int i = index_of(e);
    return i < V ? make_key(v[e], static_cast<uint32_t>(i)) : 0ull;
  };
  uint64_t m = 0;
#pragma unroll
  for (int e = 0; e < kFE; ++e) {
    const uint64_t key = key_of(e);
    m = key > m ? key : m;
  }
  m = row_max_u64(m);  // DPP steps within each 16-lane group
  if ((tid & 15) == 0) s_gmax[tid >> 4] = m;
  if (tid < MEDUSA_MAX_TOPK) s_out[tid] = 0ull;
  if (tid == 0) {
    s_theta = 1ull;  // fewer than k non-empty groups: every valid key is a candidate
    s_cnt = 0;
  }
  __syncthreads();
  if (tid < kFThreads / 16) {
    const uint64_t v = s_gmax[tid];
    int rank = 0;
    for (int j = 0; j < kFThreads / 16; ++j) rank += s_gmax[j] > v ? 1 : 0;
    if (v != 0ull && rank == k - 1) s_theta = v;
  }
  __syncthreads();
  const uint64_t theta = s_theta;
#pragma unroll
  for (int e = 0; e < kFE; ++e) {
    const uint64_t key = key_of(e);
    if (key >= theta) {
      const int p = atomicAdd(&s_cnt, 1);
      if (p < kCandMax) s_cand[p] = key;
    }
  }
  __syncthreads();
  const int C = s_cnt;
  if (C <= kCandMax) {
    for (int i = tid; i < C; i += kFThreads) {
      const uint64_t key = s_cand[i];
      int rank = 0;
      for (int j = 0; j < C; ++j) rank += s_cand[j] > key ? 1 : 0;
      if (rank < k) s_out[rank] = key;
    }
  } else {
    // overflow (rare: e.g. massive ties): k rounds of block-wide max; the
    // values are re-read from memory so the fast path keeps its registers
    const int wave = tid >> 6, lane = tid & 63;
    uint32_t taken = 0u;
    for (int round = 0; round < k; ++round) {
      uint64_t best = 0;
      int bi = 0;
#pragma unroll 1
      for (int e = 0; e < kFE; ++e) {
        const int i = index_of(e);
        const uint64_t key = ((taken >> e) & 1u) || i >= V ? 0ull : make_key(z[i], static_cast<uint32_t>(i));
        if (key > best) {
          best = key;
          bi = e;
        }
      }
      uint64_t w = best;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = shfl_xor_u64(w, off);
        w = o > w ? o : w;
      }
      uint64_t *buf = s_wave[round & 1];
      if (lane == 0) buf[wave] = w;
      __syncthreads();
      uint64_t g = buf[0];
#pragma unroll
      for (int i = 1; i < kFThreads / 64; ++i) g = buf[i] > g ? buf[i] : g;
      if (g != 0ull && best == g) taken |= 1u << bi;
      if (tid == 0) s_out[round] = g;
    }
  }
  __syncthreads();
  for (int j = tid; j < k; j += kFThreads) {
    const uint64_t key = s_out[j];
    if (nchunks == 1) {
      const uint32_t id = 0xFFFFFFFFu - static_cast<uint32_t>(key);
      idx[(size_t)row * k + j] = static_cast<int32_t>(id);
      if (val) val[(size_t)row * k + j] = z[id];
    } else {
      part[((size_t)row * nchunks + chunk) * k + j] = key;
    }
  }
  if (nchunks == 1) scatter_tokens(ts, row, s_out);
}

__global__ __launch_bounds__(kThreads) void topk_stage2(const float *__restrict__ logits, int V,
                                                        int k, int nchunks,
                                                        const uint64_t *__restrict__ part,
                                                        int32_t *__restrict__ idx,
                                                        float *__restrict__ val, TokenScatter ts) {
  __shared__ uint64_t s_wave[2][kThreads / 64];
  __shared__ uint64_t s_out[MEDUSA_MAX_TOPK];
  const int row = blockIdx.x;
  const int n = nchunks * k;
  const uint64_t *p = part + (size_t)row * n;
  uint64_t keys[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = e * kThreads + threadIdx.x;
    keys[e] = i < n ? p[i] : 0ull;
  }
  block_extract<kThreads, kPerThread>(keys, k, s_out, s_wave);
  __syncthreads();
  for (int j = threadIdx.x; j < k; j += kThreads) {
    const uint32_t id = 0xFFFFFFFFu - static_cast<uint32_t>(s_out[j]);
    idx[(size_t)row * k + j] = static_cast<int32_t>(id);
    if (val) val[(size_t)row * k + j] = logits[(size_t)row * V + id];
  }
  scatter_tokens(ts, row, s_out);
}

__global__ void tree_tokens_kernel(int B, int T, int k, const int32_t *__restrict__ depth,
                                   const int32_t *__restrict__ rank, const int32_t *__restrict__ root,
                                   const int32_t *__restrict__ topk_idx, int32_t *__restrict__ tok) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * T) return;
  const int b = i / T, j = i % T;
  tok[i] = j == 0 ? root[b] : topk_idx[((size_t)(depth[j] - 1) * B + b) * k + rank[j]];
}

inline int chunks_for(int V) { return (V + kFChunk - 1) / kFChunk; }

}  // namespace

extern "C" size_t medusa_topk_workspace(int R, int V, int k) {
  if (R < 1 || V < 1 || k < 1) return 0;
  const int nchunks = chunks_for(V);
  return nchunks > 1 ? (size_t)R * nchunks * k * sizeof(uint64_t) : 0;
}

static medusa_status topk_launch(const char *who, hipStream_t st, int R, int V, int k, const float *logits,
                                 int32_t *idx, float *val, void *ws, size_t ws_bytes, const TokenScatter &ts) {
  if (R < 1 || V < 1) return fail(MEDUSA_ERR_ARG, "%s: R=%d V=%d", who, R, V);
  if (k < 1 || k > V) return fail(MEDUSA_ERR_ARG, "%s: k=%d outside [1, V=%d]", who, k, V);
  if (k > MEDUSA_MAX_TOPK) return fail(MEDUSA_ERR_UNSUPPORTED, "%s: k=%d > %d", who, k, MEDUSA_MAX_TOPK);
  if (!logits || !idx) return fail(MEDUSA_ERR_ARG, "%s: NULL pointer", who);
  const int nchunks = chunks_for(V);
  if ((long)nchunks * k > kMergeMax)
    return fail(MEDUSA_ERR_UNSUPPORTED, "%s: V=%d with k=%d exceeds the merge capacity", who, V, k);
  const size_t need = medusa_topk_workspace(R, V, k);
  if (ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu", who, ws_bytes, need);
  if (need > 0 && !ws) return fail(MEDUSA_ERR_ARG, "%s: NULL workspace", who);
  if (R > 65535) return fail(MEDUSA_ERR_UNSUPPORTED, "%s: R=%d > 65535", who, R);
  uint64_t *part = static_cast<uint64_t *>(ws);
  hipLaunchKernelGGL(topk_chunk, dim3(nchunks, R), dim3(kFThreads), 0, st, logits, V, k, nchunks, idx, val, part, ts);
  medusa_status s = check_launch(who);
  if (s != MEDUSA_OK || nchunks == 1) return s;
  hipLaunchKernelGGL(topk_stage2, dim3(R), dim3(kThreads), 0, st, logits, V, k, nchunks, part, idx, val, ts);
  return check_launch(who);
}

extern "C" medusa_status medusa_topk(medusa_stream_t stream, int R, int V, int k, const float *logits,
                                     int32_t *idx, float *val, void *ws, size_t ws_bytes) {
  const TokenScatter none = {nullptr, nullptr, nullptr, nullptr, 1, 1, 0};
  return topk_launch("medusa_topk", as_stream(stream), R, V, k, logits, idx, val, ws, ws_bytes, none);
}

extern "C" medusa_status medusa_topk_tree_tokens(medusa_stream_t stream, const medusa_tree *t, int B, int K,
                                                 int V, int k, const float *logits, const int32_t *root_tok,
                                                 int32_t *topk_idx, int32_t *tree_tok, void *ws,
                                                 size_t ws_bytes) {
  medusa_status s = check_tree_on_device(t);
  if (s != MEDUSA_OK) return s;
  if (B < 1 || K < 1) return fail(MEDUSA_ERR_ARG, "medusa_topk_tree_tokens: B=%d K=%d", B, K);
  if (!root_tok || !tree_tok) return fail(MEDUSA_ERR_ARG, "medusa_topk_tree_tokens: NULL pointer");
  if (K < t->depth_max || k < t->k)
    return fail(MEDUSA_ERR_SHAPE, "medusa_topk_tree_tokens: top-k block [K=%d][k=%d] smaller than the tree's [%d][%d]",
                K, k, t->depth_max, t->k);
  const TokenScatter ts = {tree_tok, t->d_rank, t->d_dstart, root_tok, B, t->T, t->depth_max};
  return topk_launch("medusa_topk_tree_tokens", as_stream(stream), K * B, V, k, logits, topk_idx, nullptr, ws,
                     ws_bytes, ts);
}

extern "C" medusa_status medusa_tree_tokens(medusa_stream_t stream, const medusa_tree *t, int B,
                                            int K, int k, const int32_t *root_tok,
                                            const int32_t *topk_idx, int32_t *tree_tok) {
  medusa_status s = check_tree_on_device(t);
  if (s != MEDUSA_OK) return s;
  if (B < 1) return fail(MEDUSA_ERR_ARG, "medusa_tree_tokens: B=%d", B);
  if (!root_tok || !topk_idx || !tree_tok) return fail(MEDUSA_ERR_ARG, "medusa_tree_tokens: NULL pointer");
  if (K < t->depth_max || k < t->k)
    return fail(MEDUSA_ERR_SHAPE, "medusa_tree_tokens: top-k block [K=%d][k=%d] smaller than the tree's [%d][%d]",
                K, k, t->depth_max, t->k);
  const int n = B * t->T;
  hipLaunchKernelGGL(tree_tokens_kernel, dim3((n + 255) / 256), dim3(256), 0, as_stream(stream), B,
                     t->T, k, t->d_depth, t->d_rank, root_tok, topk_idx, tree_tok);
  return check_launch("medusa_tree_tokens");
}
