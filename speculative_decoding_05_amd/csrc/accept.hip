// Typical acceptance over the candidate tree.
//
// Row pass (one block per 4096-wide chunk of a verification row of a node
// that has children): the chunk is held in registers; a block max/argmax
// (lowest index on ties) is followed by S = sum e^(y-m) and
// E = sum e^(y-m) (y-m) with y = z / temperature, from which
// H = ln S - E/S.  Partials (m, S, E, argmax) per chunk go to the workspace.
// Scan (one block per sequence): merge the chunk partials of every internal
// row into its threshold min(eps, delta e^-H); decide every candidate against
// its parent's row; a node is accepted iff every node on its path (the root
// excepted) is, which is one AND over the node's ancestor bitmask; pick the
// deepest accepted node (smallest index on ties), write its path, and take the
// next greedy token from its row.
#include <math.h>

#include "common.h"

using namespace medusa;

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kVec = 4;                         // float4 per thread
constexpr int kChunk = kThreads * kVec * 4;     // 4096 floats
constexpr float kLog2e = 1.4426950408889634f;

struct Part {  // 32 bytes
  float m, S, E, amax_val;
  int amax_idx, pad0, pad1, pad2;
};

__device__ __forceinline__ void arg_better(float &bv, int &bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// block-wide argmax (value desc, index asc); result valid in every thread
__device__ void block_argmax(float &bv, int &bi, float *s_v, int *s_i) {
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    arg_better(bv, bi, ov, oi);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) {
    s_v[wave] = bv;
    s_i[wave] = bi;
  }
  __syncthreads();
  bv = s_v[0];
  bi = s_i[0];
  for (int w = 1; w < kThreads / 64; ++w) arg_better(bv, bi, s_v[w], s_i[w]);
}

__device__ float block_sum(float v, float *s) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) s[wave] = v;
  __syncthreads();
  float r = 0.f;
  for (int w = 0; w < kThreads / 64; ++w) r += s[w];
  return r;
}

__global__ __launch_bounds__(kThreads) void accept_rowpass(const float *__restrict__ logits, int T,
                                                           int V, int n_internal,
                                                           const int32_t *__restrict__ internal,
                                                           int nchunks, float inv_tau, int greedy,
                                                           Part *__restrict__ part) {
  __shared__ float s_v[kThreads / 64];
  __shared__ int s_i[kThreads / 64];
  const int chunk = blockIdx.x, slot = blockIdx.y, b = blockIdx.z;
  const int row = internal[slot];
  const float *z = logits + ((size_t)b * T + row) * V;
  const int base = chunk * kChunk;
  const bool vec_ok = (V % 4) == 0;
  float val[kVec][4];
  float bv = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int i0 = base + (u * kThreads + threadIdx.x) * 4;
    if (vec_ok && i0 + 3 < V) {
      const f32x4_t f = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(z + i0));
#pragma unroll
      for (int j = 0; j < 4; ++j) val[u][j] = f[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) val[u][j] = i0 + j < V ? z[i0 + j] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i0 + j < V) arg_better(bv, bi, val[u][j], i0 + j);
  }
  block_argmax(bv, bi, s_v, s_i);
  float S = 0.f, E = 0.f;
  const float m = bv * inv_tau;  // max of y = z / tau (tau > 0 keeps the order)
  if (!greedy && m != -INFINITY) {
#pragma unroll
    for (int u = 0; u < kVec; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float d = val[u][j] * inv_tau - m;  // -inf for padding
        const float e = exp2f(d * kLog2e);
        S += e;
        E += e == 0.f ? 0.f : e * d;
      }
    S = block_sum(S, s_v);
    E = block_sum(E, s_v);
  }
  if (threadIdx.x == 0) {
    Part p;
    p.m = m;
    p.S = S;
    p.E = E;
    p.amax_val = bv;
    p.amax_idx = bi;
    p.pad0 = p.pad1 = p.pad2 = 0;
    part[((size_t)b * n_internal + slot) * nchunks + chunk] = p;
  }
}

__global__ __launch_bounds__(kThreads) void accept_scan(
    const float *__restrict__ logits, const int32_t *__restrict__ tree_tok, int T, int W, int V,
    int depth_max, int n_internal, int nchunks, const int32_t *__restrict__ internal,
    const int32_t *__restrict__ slot_of, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ depth, const uint64_t *__restrict__ mask, float eps, float delta,
    float inv_tau, int greedy, const Part *__restrict__ part, int32_t *__restrict__ accept_len,
    int32_t *__restrict__ best_node, int32_t *__restrict__ next_tok,
    int32_t *__restrict__ accepted_tok, float *__restrict__ cand_p, float *__restrict__ row_thr) {
  __shared__ float s_m[MEDUSA_MAX_TREE], s_S[MEDUSA_MAX_TREE], s_thr[MEDUSA_MAX_TREE];
  __shared__ int s_amax[MEDUSA_MAX_TREE];
  __shared__ unsigned int s_dec[MEDUSA_MAX_TREE / 32];
  __shared__ unsigned int s_key[kThreads / 64];
  __shared__ float s_v[kThreads / 64];
  __shared__ int s_i[kThreads / 64];
  const int b = blockIdx.x;
  for (int w = threadIdx.x; w < MEDUSA_MAX_TREE / 32; w += kThreads) s_dec[w] = 0u;

  // 1. per internal row: merge chunk partials, threshold
  for (int sl = threadIdx.x; sl < n_internal; sl += kThreads) {
    const Part *p = part + ((size_t)b * n_internal + sl) * nchunks;
    float M = -INFINITY, av = -INFINITY;
    int ai = 0x7fffffff;
    for (int c = 0; c < nchunks; ++c) {
      M = fmaxf(M, p[c].m);
      arg_better(av, ai, p[c].amax_val, p[c].amax_idx);
    }
    float S = 0.f, E = 0.f;
    if (!greedy) {
      for (int c = 0; c < nchunks; ++c) {
        if (p[c].S == 0.f) continue;
        const float dm = p[c].m - M;
        const float w = exp2f(dm * kLog2e);
        S += w * p[c].S;
        E += w * (p[c].E + dm * p[c].S);
      }
    }
    const float H = greedy ? 0.f : logf(S) - E / S;
    s_m[sl] = M;
    s_S[sl] = S;
    s_thr[sl] = fminf(eps, delta * expf(-H));
    s_amax[sl] = ai;
  }
  __syncthreads();

  // 2. decisions: candidate c against its parent's row
  for (int c = threadIdx.x; c < T; c += kThreads) {
    const int sc = slot_of[c];
    if (row_thr) row_thr[(size_t)b * T + c] = sc >= 0 ? s_thr[sc] : NAN;
    if (c == 0) {
      if (cand_p) cand_p[(size_t)b * T] = NAN;
      continue;
    }
    const int n = parent[c];
    const int sl = slot_of[n];
    const int tok = tree_tok[(size_t)b * T + c];
    float p;
    bool dec;
    if (greedy) {
      dec = tok == s_amax[sl];
      p = dec ? 1.f : 0.f;
    } else if (tok < 0 || tok >= V) {  // out-of-range id: never accepted
      p = 0.f;
      dec = false;
    } else {
      const float zc = logits[((size_t)b * T + n) * V + tok];
      p = exp2f((zc * inv_tau - s_m[sl]) * kLog2e) / s_S[sl];
      dec = p > s_thr[sl];
    }
    if (cand_p) cand_p[(size_t)b * T + c] = p;
    if (dec) atomicOr(&s_dec[c >> 5], 1u << (c & 31));
  }
  __syncthreads();

  // 3. accepted iff all ancestors but the root decided yes; deepest, then smallest index
  unsigned int key = 0u;
  for (int c = threadIdx.x; c < T; c += kThreads) {
    bool acc = true;
    for (int w = 0; w < W; ++w) {
      uint64_t anc = mask[(size_t)c * W + w];
      if (w == 0) anc &= ~1ull;
      const int i0 = w * 64;
      const uint64_t dec = (uint64_t)s_dec[i0 >> 5] | ((uint64_t)s_dec[(i0 >> 5) + 1] << 32);
      if (anc & ~dec) acc = false;
    }
    if (acc) {
      const unsigned int k = ((unsigned)depth[c] << 16) | (0xFFFFu - (unsigned)c);
      key = k > key ? k : key;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned int o = __shfl_xor(key, off);
    key = o > key ? o : key;
  }
  if ((threadIdx.x & 63) == 0) s_key[threadIdx.x >> 6] = key;
  __syncthreads();
  key = s_key[0];
  for (int w = 1; w < kThreads / 64; ++w) key = s_key[w] > key ? s_key[w] : key;
  const int alen = (int)(key >> 16);
  const int best = (int)(0xFFFFu - (key & 0xFFFFu));

  if (threadIdx.x == 0) {
    accept_len[b] = alen;
    best_node[b] = best;
    int32_t *at = accepted_tok + (size_t)b * (depth_max + 1);
    for (int d = alen + 1; d <= depth_max; ++d) at[d] = -1;
    int d = alen;
    for (int j = best; j != -1; j = parent[j]) at[d--] = tree_tok[(size_t)b * T + j];
  }
  // 4. next greedy token: argmax of the winner's row
  const int sb = slot_of[best];
  if (sb >= 0) {
    if (threadIdx.x == 0) next_tok[b] = s_amax[sb];
  } else {
    const float *z = logits + ((size_t)b * T + best) * V;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = threadIdx.x; i < V; i += kThreads) arg_better(bv, bi, z[i], i);
    block_argmax(bv, bi, s_v, s_i);
    if (threadIdx.x == 0) next_tok[b] = bi;
  }
}

inline int chunks_for(int V) { return (V + kChunk - 1) / kChunk; }

}  // namespace

extern "C" size_t typical_accept_workspace(const medusa_tree *t, int B, int V) {
  if (!t || B < 1 || V < 1) return 0;
  return (size_t)B * (t->n_internal > 0 ? t->n_internal : 1) * chunks_for(V) * sizeof(Part);
}

extern "C" medusa_status typical_accept(medusa_stream_t stream, const medusa_tree *t, int B, int V,
                                        const float *logits, const int32_t *tree_tok, float eps,
                                        float delta, float temperature, int32_t *accept_len,
                                        int32_t *best_node, int32_t *next_tok, int32_t *accepted_tok,
                                        float *cand_p, float *row_thr, void *ws, size_t ws_bytes) {
  medusa_status s = check_tree_on_device(t);
  if (s != MEDUSA_OK) return s;
  if (B < 1 || V < 1) return fail(MEDUSA_ERR_ARG, "typical_accept: B=%d V=%d", B, V);
  if (!(eps >= 0.f) || !(delta >= 0.f) || !(temperature >= 0.f) || !isfinite(temperature))
    return fail(MEDUSA_ERR_ARG, "typical_accept: eps, delta, temperature must be >= 0 (and finite temperature)");
  if (!logits || !tree_tok || !accept_len || !best_node || !next_tok || !accepted_tok || !ws)
    return fail(MEDUSA_ERR_ARG, "typical_accept: NULL pointer");
  if (!aligned16(logits) || !aligned16(ws)) return fail(MEDUSA_ERR_ARG, "typical_accept: logits and ws must be 16-byte aligned");
  if (B > 65535) return fail(MEDUSA_ERR_UNSUPPORTED, "typical_accept: B=%d > 65535", B);
  const size_t need = typical_accept_workspace(t, B, V);
  if (ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "typical_accept: workspace %zu < %zu", ws_bytes, need);
  hipStream_t st = as_stream(stream);
  const int nchunks = chunks_for(V);
  const int greedy = temperature == 0.f;
  const float inv_tau = greedy ? 1.f : 1.f / temperature;
  Part *part = static_cast<Part *>(ws);
  if (t->n_internal > 0) {
    hipLaunchKernelGGL(accept_rowpass, dim3(nchunks, t->n_internal, B), dim3(kThreads), 0, st, logits,
                       t->T, V, t->n_internal, t->d_internal, nchunks, inv_tau, greedy, part);
    s = check_launch("typical_accept row pass");
    if (s != MEDUSA_OK) return s;
  }
  hipLaunchKernelGGL(accept_scan, dim3(B), dim3(kThreads), 0, st, logits, tree_tok, t->T, t->W, V,
                     t->depth_max, t->n_internal, nchunks, t->d_internal, t->d_slot, t->d_parent,
                     t->d_depth, t->d_mask, eps, delta, inv_tau, greedy, part, accept_len, best_node,
                     next_tok, accepted_tok, cand_p, row_thr);
  return check_launch("typical_accept scan");
}
