// Per-row top-k over the vocabulary, and the tree-token gather.
//
// Each element becomes a distinct 64-bit key: the order-preserving image of
// the float (with -0.0 folded onto +0.0) in the high word and the bitwise
// complement of the index in the low word, so that "larger key" means
// "larger value, then smaller index" and every row has exactly one answer.
//
// A row is cut into slices of NT*PT elements, one NT-thread block each.  In a
// slice the 64 groups of NT/64 lanes each find their largest 32-bit value
// image; theta, the largest group maximum that at least k group maxima
// reach, is a lower bound of the slice's k-th largest value (k distinct
// elements reach it).  The keys whose image is >= theta (typically a few
// dozen) are appended to LDS and each is ranked exactly by counting the
// larger candidates; rank r < k goes to slot r.  Should the candidate set
// overflow LDS, the block falls back to k rounds of block-wide max
// extraction.  A row of one slice is finished there; otherwise every slice
// writes its sorted k keys to the workspace and a second kernel merges each
// row's lists (a key's rank is the number of larger keys over all lists,
// found by scanning each list down to its first smaller key).
#include "common.h"

using namespace medusa;

namespace {

constexpr int kCandMax = 1024;   // candidates a slice can rank
constexpr int kMergeMax = 4096;  // slices * k the merge can hold
constexpr int kMergeThreads = 256;

__device__ __forceinline__ uint64_t make_key(uint32_t image, uint32_t idx) {
  return (static_cast<uint64_t>(image) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t key) {
  return 0xFFFFFFFFu - static_cast<uint32_t>(key);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int off) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), off);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), off);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// max over aligned groups of G lanes (G = 4 or 16), result in every lane
template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  uint32_t o = dpp<kDppXor1>(v);
  v = o > v ? o : v;
  o = dpp<kDppXor2>(v);
  v = o > v ? o : v;
  if (G == 16) {
    o = dpp<kDppHalfMirror>(v);
    v = o > v ? o : v;
    o = dpp<kDppMirror>(v);
    v = o > v ? o : v;
  }
  return v;
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
  // the root first: a root-only tree (depth_max = 0) has no node to scatter
  if (head == 0 && threadIdx.x == 0) ts.tree_tok[(size_t)b * ts.T] = ts.root[b];
  if (head + 1 > ts.depth_max) return;
  const int j0 = ts.dstart[head + 1], j1 = ts.dstart[head + 2];
  for (int j = j0 + (int)threadIdx.x; j < j1; j += blockDim.x)
    ts.tree_tok[(size_t)b * ts.T + j] = static_cast<int32_t>(key_index(s_out[ts.rank[j]]));
}

// idx/val/scatter of a finished row from its sorted keys
__device__ __forceinline__ void emit_row(const float *z, int row, int k, const uint64_t *s_out, int32_t *idx,
                                         float *val, const TokenScatter &ts) {
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    const uint32_t id = key_index(s_out[j]);
    idx[(size_t)row * k + j] = static_cast<int32_t>(id);
    if (val) val[(size_t)row * k + j] = z[id];
  }
  scatter_tokens(ts, row, s_out);
}

template <int NT, int PT>
__global__ __launch_bounds__(NT) void topk_slices(const float *__restrict__ logits, int V, int k, int nslices,
                                                  int32_t *__restrict__ idx, float *__restrict__ val,
                                                  uint64_t *__restrict__ part, TokenScatter ts) {
  constexpr int G = NT / 64;  // lanes per group; 64 groups
  __shared__ uint32_t s_gmax[64];
  __shared__ uint64_t s_cand[kCandMax];
  __shared__ uint64_t s_out[MEDUSA_MAX_TOPK];
  __shared__ uint64_t s_wave[2][NT / 64];
  __shared__ uint32_t s_theta;
  __shared__ int s_cnt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slice = blockIdx.x, row = blockIdx.y;
  const float *z = logits + (size_t)row * V;
  const int base = slice * NT * PT;
  // element e of this thread is index base + (e/4)*4*NT + 4*tid + e%4; every
  // load is issued unconditionally (clamped into the row), indices >= V are
  // masked afterwards
  auto index_of = [&](int e) { return base + (e >> 2) * 4 * NT + 4 * tid + (e & 3); };
  uint32_t img[PT];
  if ((V % 4) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0) {
#pragma unroll
    for (int g = 0; g < PT / 4; ++g) {
      const int i0 = min(index_of(4 * g), V - 4);
      const float4 f = *reinterpret_cast<const float4 *>(z + i0);
      img[4 * g] = order_image(f.x);
      img[4 * g + 1] = order_image(f.y);
      img[4 * g + 2] = order_image(f.z);
      img[4 * g + 3] = order_image(f.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < PT; ++e) img[e] = order_image(z[min(index_of(e), V - 1)]);
  }
  // images of indices >= V become 0, at or below every valid image
  uint32_t m = 0u;
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    if (index_of(e) >= V) img[e] = 0u;
    m = img[e] > m ? img[e] : m;
  }
  m = group_max<G>(m);
  if ((tid & (G - 1)) == 0) s_gmax[tid / G] = m;
  if (tid < MEDUSA_MAX_TOPK) s_out[tid] = 0ull;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  if (wave == 0) {
    // theta = largest group maximum reached by at least k group maxima (a
    // group maximum of 0 is at most every valid image, so theta = 0 admits
    // every valid element)
    const uint32_t g = s_gmax[lane];
    int reach = 0;
#pragma unroll 8
    for (int j = 0; j < 64; ++j) reach += s_gmax[j] >= g ? 1 : 0;
    const uint32_t t = wave_max_u32(reach >= k ? g : 0u);
    if (lane == 0) s_theta = t;
  }
  __syncthreads();
  const uint32_t theta = s_theta;
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    const int i = index_of(e);
    if (i < V && img[e] >= theta) {
      const int p = atomicAdd(&s_cnt, 1);
      if (p < kCandMax) s_cand[p] = make_key(img[e], static_cast<uint32_t>(i));
    }
  }
  __syncthreads();
  const int C = s_cnt;
  if (C <= kCandMax) {
    for (int i = tid; i < C; i += NT) {
      const uint64_t key = s_cand[i];
      int rank = 0;
      for (int j = 0; j < C; ++j) rank += s_cand[j] > key ? 1 : 0;
      if (rank < k) s_out[rank] = key;
    }
  } else {
    // overflow (rare: e.g. massive ties): k rounds of block-wide max; the
    // values are re-read from memory so that the common path keeps its
    // registers (keys hoisted out of this loop would spill)
    uint32_t taken = 0u;
    for (int round = 0; round < k; ++round) {
      uint64_t best = 0ull;
      int bi = 0;
#pragma unroll 1
      for (int e = 0; e < PT; ++e) {
        const int i = index_of(e);
        const uint64_t key =
            ((taken >> e) & 1u) || i >= V ? 0ull : make_key(order_image(z[i]), static_cast<uint32_t>(i));
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
      uint64_t *buf = s_wave[round & 1];  // alternate buffers: one barrier per round
      if (lane == 0) buf[wave] = w;
      __syncthreads();
      uint64_t g = buf[0];
#pragma unroll
      for (int i = 1; i < NT / 64; ++i) g = buf[i] > g ? buf[i] : g;
      if (g != 0ull && best == g) taken |= 1u << bi;
      if (tid == 0) s_out[round] = g;
    }
  }
  __syncthreads();
  if (nslices == 1) {
    emit_row(z, row, k, s_out, idx, val, ts);
  } else {
    // this slice's sorted list (zeros pad a slice of fewer than k elements)
    for (int j = tid; j < k; j += NT) part[((size_t)row * nslices + slice) * k + j] = s_out[j];
  }
}

// One block per row: merge the slices' sorted lists.
__global__ __launch_bounds__(kMergeThreads) void topk_merge(const float *__restrict__ logits, int V, int k,
                                                            int nslices, const uint64_t *__restrict__ part,
                                                            int32_t *__restrict__ idx, float *__restrict__ val,
                                                            TokenScatter ts) {
  __shared__ uint64_t s_all[kMergeMax];
  __shared__ uint64_t s_out[MEDUSA_MAX_TOPK];
  const int row = blockIdx.x, n = nslices * k;
  const uint64_t *rp = part + (size_t)row * n;
  for (int c = threadIdx.x; c < n; c += kMergeThreads) s_all[c] = rp[c];
  __syncthreads();
  for (int c = threadIdx.x; c < n; c += kMergeThreads) {
    const uint64_t x = s_all[c];
    if (x == 0ull) continue;
    int rank = 0;
    for (int s = 0; s < nslices && rank < k; ++s) {
      const uint64_t *lst = s_all + s * k;
      for (int j = 0; j < k && lst[j] > x; ++j) ++rank;
    }
    if (rank < k) s_out[rank] = x;
  }
  __syncthreads();
  emit_row(logits + (size_t)row * V, row, k, s_out, idx, val, ts);
}

// Top-k from tile maxima.  With the logits come the images of each 16-value
// tile's largest element (written by the vocabulary projection's blocks, which
// hold a tile's 16 values together).  A row's tile images are dealt to the
// threads in order, and the 64 sets {lane l of every wave} each take their
// largest: theta, the largest set maximum that at least k set maxima reach, is
// reached by k distinct tiles and so by k distinct elements, hence is at most
// the row's k-th largest value.  The row's top k therefore lie in the tiles
// whose image reaches theta: the block loads those tiles' values only (a
// 32000-value row: 8 KB of images and typically a dozen 64-byte tiles, not
// 128 KB) and ranks the candidate keys exactly as above.  Should the tiles or
// the candidates overflow LDS (massive ties), k rounds each take the largest
// key below the previous round's over the whole row.
constexpr int kTileCand = 256;  // candidate tiles a row can load

template <int PT>
__global__ __launch_bounds__(1024) void topk_tiles(const float *__restrict__ logits,
                                                   const uint32_t *__restrict__ timg, int V, int k,
                                                   int32_t *__restrict__ idx, TokenScatter ts) {
  constexpr int NT = 1024;
  __shared__ uint32_t s_lmax[NT / 64][64];
  __shared__ int s_tile[kTileCand];
  __shared__ uint64_t s_cand[kCandMax];
  __shared__ uint64_t s_out[MEDUSA_MAX_TOPK];
  __shared__ uint64_t s_wave[2][NT / 64];
  __shared__ uint32_t s_theta;
  __shared__ int s_ntile, s_cnt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row = blockIdx.x;
  const int nt = (V + 15) >> 4;
  const float *z = logits + (size_t)row * V;
  // tile e*NT + tid; reads past the row's nt images return 0, at or below
  // every valid image
  const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t *>(timg + (size_t)row * nt), (short)0, nt * 4, kBufferWord3);
  uint32_t img[PT];
#pragma unroll
  for (int e = 0; e < PT; ++e) img[e] = __builtin_amdgcn_raw_buffer_load_b32(tr, (e * NT + tid) * 4, 0, 0);
  uint32_t m = 0u;
#pragma unroll
  for (int e = 0; e < PT; ++e) m = img[e] > m ? img[e] : m;
  s_lmax[wave][lane] = m;
  if (tid < MEDUSA_MAX_TOPK) s_out[tid] = 0ull;
  if (tid == 0) {
    s_ntile = 0;
    s_cnt = 0;
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t g = 0u;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) g = s_lmax[w][lane] > g ? s_lmax[w][lane] : g;
    int reach = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) reach += readlane(g, j) >= g ? 1 : 0;
    const uint32_t t = wave_max_u32(reach >= k ? g : 0u);
    if (lane == 0) s_theta = t;
  }
  __syncthreads();
  const uint32_t theta = s_theta;
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    const int t = e * NT + tid;
    if (t < nt && img[e] >= theta) {
      const int p = atomicAdd(&s_ntile, 1);
      if (p < kTileCand) s_tile[p] = t;
    }
  }
  __syncthreads();
  const int ntile = s_ntile;
  const bool tiles_fit = ntile <= kTileCand;
  if (tiles_fit) {
    // 64 tiles per pass, 16 lanes per tile; reads past the row return 0
    const __amdgpu_buffer_rsrc_t zr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(z), (short)0, V * 4, kBufferWord3);
    for (int s0 = 0; s0 < ntile; s0 += NT / 16) {
      const int slot = s0 + (tid >> 4);
      const bool in_list = slot < ntile;
      const int i = s_tile[in_list ? slot : 0] * 16 + (tid & 15);
      const bool valid = in_list && i < V;
      const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(zr, (valid ? i : V) * 4, 0, 0));
      const uint32_t im = order_image(x);
      if (valid && im >= theta) {
        const int p = atomicAdd(&s_cnt, 1);
        if (p < kCandMax) s_cand[p] = make_key(im, static_cast<uint32_t>(i));
      }
    }
  }
  __syncthreads();
  const int C = s_cnt;
  if (tiles_fit && C <= kCandMax) {
    for (int i = tid; i < C; i += NT) {
      const uint64_t key = s_cand[i];
      int rank = 0;
      for (int j = 0; j < C; ++j) rank += s_cand[j] > key ? 1 : 0;
      if (rank < k) s_out[rank] = key;
    }
  } else {
    // keys are distinct, so "largest below the previous" needs no marks
    uint64_t prev = ~0ull;
    for (int round = 0; round < k; ++round) {
      uint64_t best = 0ull;
      for (int i = tid; i < V; i += NT) {
        const uint64_t key = make_key(order_image(z[i]), static_cast<uint32_t>(i));
        if (key < prev && key > best) best = key;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = shfl_xor_u64(best, off);
        best = o > best ? o : best;
      }
      uint64_t *buf = s_wave[round & 1];  // alternate buffers: one barrier per round
      if (lane == 0) buf[wave] = best;
      __syncthreads();
      uint64_t g = buf[0];
#pragma unroll
      for (int w = 1; w < NT / 64; ++w) g = buf[w] > g ? buf[w] : g;
      prev = g;
      if (tid == 0) s_out[round] = g;
    }
  }
  __syncthreads();
  emit_row(z, row, k, s_out, idx, nullptr, ts);
}

__global__ void tree_tokens_kernel(int B, int T, int k, const int32_t *__restrict__ depth,
                                   const int32_t *__restrict__ rank, const int32_t *__restrict__ root,
                                   const int32_t *__restrict__ topk_idx, int32_t *__restrict__ tok) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * T) return;
  const int b = i / T, j = i % T;
  tok[i] = j == 0 ? root[b] : topk_idx[((size_t)(depth[j] - 1) * B + b) * k + rank[j]];
}

// Slice shape: 1024 threads x 32 elements = 32768, a whole 32000-token row in
// one block with no merge.  (Slices of 256 x 16 with a merge kernel measured
// slower at 4 and 64 rows of 32000: the second launch costs more than the
// wider block.)
constexpr int kNT = 1024, kPT = 32;
constexpr int kSlice = kNT * kPT;
inline int slices_for(int V) { return (V + kSlice - 1) / kSlice; }

}  // namespace

// Workspace of rows of several slices: their sorted lists [R][slices][k] of
// 64-bit keys.
extern "C" size_t medusa_topk_workspace(int R, int V, int k) {
  if (R < 1 || V < 1 || k < 1) return 0;
  const int ns = slices_for(V);
  return ns > 1 ? (size_t)R * ns * k * sizeof(uint64_t) : 0;
}

static medusa_status topk_launch(const char *who, hipStream_t st, int R, int V, int k, const float *logits,
                                 int32_t *idx, float *val, void *ws, size_t ws_bytes, const TokenScatter &ts,
                                 int n_root = 0) {
  if (R < 1 || V < 1) return fail(MEDUSA_ERR_ARG, "%s: R=%d V=%d", who, R, V);
  if (k < 1 || k > V) return fail(MEDUSA_ERR_ARG, "%s: k=%d outside [1, V=%d]", who, k, V);
  if (k > MEDUSA_MAX_TOPK) return fail(MEDUSA_ERR_UNSUPPORTED, "%s: k=%d > %d", who, k, MEDUSA_MAX_TOPK);
  if (!logits || !idx) return fail(MEDUSA_ERR_ARG, "%s: NULL pointer", who);
  const int ns = slices_for(V);
  if ((long)ns * k > kMergeMax)
    return fail(MEDUSA_ERR_UNSUPPORTED, "%s: V=%d with k=%d exceeds the merge capacity", who, V, k);
  const size_t need = medusa_topk_workspace(R, V, k);
  if (ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu", who, ws_bytes, need);
  if (need > 0 && !ws) return fail(MEDUSA_ERR_ARG, "%s: NULL workspace", who);
  if (need > 0 && (reinterpret_cast<uintptr_t>(ws) & 7u))
    return fail(MEDUSA_ERR_ARG, "%s: workspace must be 8-byte aligned", who);
  if (R > 65535) return fail(MEDUSA_ERR_UNSUPPORTED, "%s: R=%d > 65535", who, R);
  if (validate_enabled()) {  // NaN logits; root tokens outside [0, V)
    ValidateSpec v;
    v.a = logits;
    v.na = (size_t)R * V;
    v.tok = ts.root;
    v.nt = ts.root ? (size_t)n_root : 0;
    v.V = V;
    medusa_status vs = validate_inputs(st, who, v);
    if (vs != MEDUSA_OK) return vs;
  }
  uint64_t *part = static_cast<uint64_t *>(ws);
  MEDUSA_LAUNCH("medusa_topk", (topk_slices<kNT, kPT>), dim3(ns, R), dim3(kNT), 0, st, logits, V, k, ns, idx, val, part, ts);
  medusa_status s = check_launch(who);
  if (s != MEDUSA_OK || ns == 1) return s;
  MEDUSA_LAUNCH("medusa_topk", topk_merge, dim3(R), dim3(kMergeThreads), 0, st, logits, V, k, ns, part, idx, val, ts);
  return check_launch(who);
}

extern "C" medusa_status medusa_topk(medusa_stream_t stream, int R, int V, int k, const float *logits,
                                     int32_t *idx, float *val, void *ws, size_t ws_bytes) {
  TraceRange tr("medusa_topk");
  const TokenScatter none = {nullptr, nullptr, nullptr, nullptr, 1, 1, 0};
  return topk_launch("medusa_topk", as_stream(stream), R, V, k, logits, idx, val, ws, ws_bytes, none);
}

extern "C" medusa_status medusa_topk_tree_tokens(medusa_stream_t stream, const medusa_tree *t, int B, int K,
                                                 int V, int k, const float *logits, const int32_t *root_tok,
                                                 int32_t *topk_idx, int32_t *tree_tok, void *ws,
                                                 size_t ws_bytes) {
  TraceRange tr("medusa_topk_tree_tokens");
  medusa_status s = check_tree_on_device(t);
  if (s != MEDUSA_OK) return s;
  if (B < 1 || K < 1) return fail(MEDUSA_ERR_ARG, "medusa_topk_tree_tokens: B=%d K=%d", B, K);
  if (!root_tok || !tree_tok) return fail(MEDUSA_ERR_ARG, "medusa_topk_tree_tokens: NULL pointer");
  if (K < t->depth_max || k < t->k)
    return fail(MEDUSA_ERR_SHAPE, "medusa_topk_tree_tokens: top-k block [K=%d][k=%d] smaller than the tree's [%d][%d]",
                K, k, t->depth_max, t->k);
  const TokenScatter ts = {tree_tok, t->d_rank, t->d_dstart, root_tok, B, t->T, t->depth_max};
  return topk_launch("medusa_topk_tree_tokens", as_stream(stream), K * B, V, k, logits, topk_idx, nullptr, ws,
                     ws_bytes, ts, B);
}

extern "C" medusa_status medusa_topk_tree_tokens_tmax(medusa_stream_t stream, const medusa_tree *t, int B,
                                                      int K, int V, int k, const float *logits,
                                                      const uint32_t *tile_max, const int32_t *root_tok,
                                                      int32_t *topk_idx, int32_t *tree_tok) {
  const char *who = "medusa_topk_tree_tokens_tmax";
  TraceRange tr(who);
  medusa_status s = check_tree_on_device(t);
  if (s != MEDUSA_OK) return s;
  if (B < 1 || K < 1 || V < 1) return fail(MEDUSA_ERR_ARG, "%s: B=%d K=%d V=%d", who, B, K, V);
  if (!logits || !tile_max || !root_tok || !topk_idx || !tree_tok) return fail(MEDUSA_ERR_ARG, "%s: NULL pointer", who);
  if (reinterpret_cast<uintptr_t>(tile_max) & 3u) return fail(MEDUSA_ERR_ARG, "%s: tile_max must be 4-byte aligned", who);
  if (K < t->depth_max || k < t->k)
    return fail(MEDUSA_ERR_SHAPE, "%s: top-k block [K=%d][k=%d] smaller than the tree's [%d][%d]", who, K, k,
                t->depth_max, t->k);
  if (k < 1 || k > V) return fail(MEDUSA_ERR_ARG, "%s: k=%d outside [1, V=%d]", who, k, V);
  if (k > MEDUSA_MAX_TOPK) return fail(MEDUSA_ERR_UNSUPPORTED, "%s: k=%d > %d", who, k, MEDUSA_MAX_TOPK);
  const long R = (long)K * B;
  if (R > 65535) return fail(MEDUSA_ERR_UNSUPPORTED, "%s: K*B=%ld > 65535", who, R);
  const int nt = (V + 15) / 16;
  if (nt > kNT * 32) return fail(MEDUSA_ERR_UNSUPPORTED, "%s: V=%d > %d", who, V, kNT * 32 * 16);
  const hipStream_t st = as_stream(stream);
  if (validate_enabled()) {  // NaN logits; root tokens outside [0, V)
    ValidateSpec v;
    v.a = logits;
    v.na = (size_t)R * V;
    v.tok = root_tok;
    v.nt = (size_t)B;
    v.V = V;
    medusa_status vs = validate_inputs(st, who, v);
    if (vs != MEDUSA_OK) return vs;
  }
  const TokenScatter ts = {tree_tok, t->d_rank, t->d_dstart, root_tok, B, t->T, t->depth_max};
  if (nt <= kNT * 2)
    MEDUSA_LAUNCH("medusa_topk", topk_tiles<2>, dim3((unsigned)R), dim3(kNT), 0, st, logits, tile_max, V, k, topk_idx, ts);
  else if (nt <= kNT * 8)
    MEDUSA_LAUNCH("medusa_topk", topk_tiles<8>, dim3((unsigned)R), dim3(kNT), 0, st, logits, tile_max, V, k, topk_idx, ts);
  else
    MEDUSA_LAUNCH("medusa_topk", topk_tiles<32>, dim3((unsigned)R), dim3(kNT), 0, st, logits, tile_max, V, k, topk_idx, ts);
  return check_launch(who);
}

extern "C" medusa_status medusa_tree_tokens(medusa_stream_t stream, const medusa_tree *t, int B,
                                            int K, int k, const int32_t *root_tok,
                                            const int32_t *topk_idx, int32_t *tree_tok) {
  TraceRange tr("medusa_tree_tokens");
  medusa_status s = check_tree_on_device(t);
  if (s != MEDUSA_OK) return s;
  if (B < 1) return fail(MEDUSA_ERR_ARG, "medusa_tree_tokens: B=%d", B);
  if (!root_tok || !topk_idx || !tree_tok) return fail(MEDUSA_ERR_ARG, "medusa_tree_tokens: NULL pointer");
  if (K < t->depth_max || k < t->k)
    return fail(MEDUSA_ERR_SHAPE, "medusa_tree_tokens: top-k block [K=%d][k=%d] smaller than the tree's [%d][%d]",
                K, k, t->depth_max, t->k);
  const int n = B * t->T;
  MEDUSA_LAUNCH("medusa_topk", tree_tokens_kernel, dim3((n + 255) / 256), dim3(256), 0, as_stream(stream), B,
                     t->T, k, t->d_depth, t->d_rank, root_tok, topk_idx, tree_tok);
  return check_launch("medusa_tree_tokens");
}
