// Rejection-sampling acceptance over the candidate tree (the comparison
// point of typical acceptance).  One block of 1024 threads per sequence walks
// the tree from the root: at the current node u it forms the verification
// distribution p (softmax of u's row at the temperature) and the drafting
// head's distribution q (softmax of head depth(u)'s row for this sequence),
// tries u's children in rank order -- child x is kept iff its uniform is
// below min(1, p(x)/q(x)), and a rejected child replaces p by the
// renormalised residual max(0, p - q) -- and moves to the first kept child.
// When no child is kept, or u is a leaf, the next token is drawn by inverse
// CDF from the current p.
//
// The residual after j rejections is never stored: every pass recomputes it
// per element from p(v), q(v) and the j normalisers, so the block only streams
// the two rows (L2-resident after the first pass).  Temperature 0 uses
// one-hot distributions at the argmax (lowest index): greedy verification.
#include <math.h>

#include "common.h"

using namespace medusa;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxResid = MEDUSA_MAX_TREE;   // rejections at one node <= its children

struct BlockScratch {
  float f[kWaves];
  uint64_t k[kWaves];
};

__device__ __forceinline__ float wave_sum(float v) {
  v += dppf<kDppXor1>(v);
  v += dppf<kDppXor2>(v);
  v += dppf<kDppHalfMirror>(v);
  v += dppf<kDppMirror>(v);
  return readlanef(v, 0) + readlanef(v, 16) + readlanef(v, 32) + readlanef(v, 48);
}
__device__ __forceinline__ float wave_maxf(float v) {
  v = fmaxf(v, dppf<kDppXor1>(v));
  v = fmaxf(v, dppf<kDppXor2>(v));
  v = fmaxf(v, dppf<kDppHalfMirror>(v));
  v = fmaxf(v, dppf<kDppMirror>(v));
  return fmaxf(fmaxf(readlanef(v, 0), readlanef(v, 16)), fmaxf(readlanef(v, 32), readlanef(v, 48)));
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = row_max_u64(v);
  uint64_t r = 0;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint64_t x = ((uint64_t)readlane((uint32_t)(v >> 32), row * 16) << 32) | readlane((uint32_t)v, row * 16);
    r = x > r ? x : r;
  }
  return r;
}

// block-wide reductions; every thread gets the result
__device__ float block_sum(float v, BlockScratch &s) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.f[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r += s.f[w];
  return r;
}
__device__ float block_max(float v, BlockScratch &s) {
  v = wave_maxf(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.f[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r = fmaxf(r, s.f[w]);
  return r;
}
__device__ uint64_t block_max_u64(uint64_t v, BlockScratch &s) {
  v = wave_max_u64(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.k[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t r = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r = s.k[w] > r ? s.k[w] : r;
  return r;
}

// argmax key: larger value first, then smaller index
__device__ __forceinline__ uint64_t argmax_key(float x, int i) {
  uint32_t u = __builtin_bit_cast(uint32_t, x == 0.f ? 0.f : x);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)i);
}

// A distribution over the vocabulary: softmax(row / tau), or one-hot at amax
struct Dist {
  const float *row;
  float m = 0.f, S = 1.f, inv_tau = 0.f;
  int amax = 0;  // >= 0: one-hot
  __device__ float operator()(int v) const {
    if (amax >= 0) return v == amax ? 1.f : 0.f;
    return __expf((row[v] * inv_tau - m)) / S;
  }
};

__device__ Dist make_dist(const float *row, int V, float tau, BlockScratch &s) {
  Dist d;
  d.row = row;
  if (tau == 0.f) {
    uint64_t best = 0;
    for (int v = threadIdx.x; v < V; v += kThreads) {
      const uint64_t key = argmax_key(row[v], v);
      best = key > best ? key : best;
    }
    best = block_max_u64(best, s);
    d.amax = (int)(~(uint32_t)best);
    d.m = 0.f;
    d.S = 1.f;
    d.inv_tau = 0.f;
    return d;
  }
  d.amax = -1;
  d.inv_tau = 1.f / tau;
  float m = -INFINITY;
  for (int v = threadIdx.x; v < V; v += kThreads) m = fmaxf(m, row[v] * d.inv_tau);
  d.m = block_max(m, s);
  float S = 0.f;
  for (int v = threadIdx.x; v < V; v += kThreads) S += __expf(row[v] * d.inv_tau - d.m);
  d.S = block_sum(S, s);
  return d;
}

// p after the rejections recorded in Z[0..nz): p_{j+1} = max(0, p_j - q) / Z[j]
__device__ __forceinline__ float residual(float p, float q, const float *Z, int nz) {
  for (int j = 0; j < nz; ++j) p = fmaxf(p - q, 0.f) / Z[j];
  return p;
}

// Inverse-CDF draw: the smallest v with f(0) + ... + f(v) > u * sum(f), or the
// last v with f(v) > 0 if rounding leaves none.  Thread t owns the contiguous
// range [t*C, (t+1)*C); a block scan of the 1024 range sums finds the range
// that holds the target.  Every thread gets the token.
template <typename F>
__device__ int inverse_cdf(const F &f, int V, float u, float *s_part, int *s_tok, BlockScratch &scr) {
  const int tid = threadIdx.x;
  const int C = (V + kThreads - 1) / kThreads;
  const int v0 = min(V, tid * C), v1 = min(V, v0 + C);
  float own = 0.f;
  for (int v = v0; v < v1; ++v) own += f(v);
  __syncthreads();
  s_part[tid] = own;
  if (tid == 0) *s_tok = -1;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {   // inclusive scan (Hillis-Steele)
    const float add = tid >= off ? s_part[tid - off] : 0.f;
    __syncthreads();
    s_part[tid] += add;
    __syncthreads();
  }
  // thread t's range of the running sum is [s_part[t-1], s_part[t]): the
  // ranges are disjoint, so at most one thread claims the target
  const float target = u * s_part[kThreads - 1];
  const float lo = tid > 0 ? s_part[tid - 1] : 0.f, hi = s_part[tid];
  if (hi > lo && target >= lo && target < hi) {
    float acc = lo;
    int tok = -1;
    for (int v = v0; v < v1 && tok < 0; ++v) {
      const float pv = f(v);
      acc += pv;
      if (pv > 0.f && acc > target) tok = v;
    }
    for (int v = v1 - 1; v >= v0 && tok < 0; --v)
      if (f(v) > 0.f) tok = v;
    *s_tok = tok;
  }
  __syncthreads();
  int tok = *s_tok;
  if (tok < 0) {
    int last = -1;
    for (int v = tid; v < V; v += kThreads)
      if (f(v) > 0.f) last = v;
    tok = (int)block_max_u64((uint64_t)(uint32_t)(last + 1), scr) - 1;
  }
  return tok;
}

__global__ __launch_bounds__(kThreads) void rejection_accept_kernel(
    int T, int V, int depth_max, const int32_t *__restrict__ parent, const int32_t *__restrict__ depth,
    const int32_t *__restrict__ dstart, const float *__restrict__ logits, const float *__restrict__ head_logits,
    int B, const int32_t *__restrict__ tree_tok, float tau, const float *__restrict__ u_node,
    const float *__restrict__ u_bonus, int32_t *__restrict__ accept_len, int32_t *__restrict__ best_node,
    int32_t *__restrict__ next_tok, int32_t *__restrict__ accepted_tok, float *__restrict__ keep_prob) {
  __shared__ BlockScratch scr;
  __shared__ int cld[MEDUSA_MAX_TREE];
  __shared__ float Z[kMaxResid];
  __shared__ int path[MEDUSA_MAX_TREE];
  __shared__ float s_part[kThreads];
  __shared__ int s_ncld, s_kept, s_tok;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  if (keep_prob)
    for (int c = tid; c < T; c += kThreads) keep_prob[(size_t)b * T + c] = __builtin_nanf("");
  for (int i = tid; i <= depth_max; i += kThreads) accepted_tok[(size_t)b * (depth_max + 1) + i] = -1;

  int u = 0, plen = 1, nz = 0;
  if (tid == 0) path[0] = 0;
  Dist p, q;
  q.row = nullptr;
  bool resid = false;   // the final draw is from the residual of u's rejected children
  while (true) {
    p = make_dist(logits + ((size_t)b * T + u) * V, V, tau, scr);
    const int d = depth[u];
    if (tid == 0) {
      int n = 0;
      if (d < depth_max)
        for (int c = dstart[d + 1]; c < dstart[d + 2]; ++c)
          if (parent[c] == u) cld[n++] = c;
      s_ncld = n;
    }
    __syncthreads();
    const int ncld = s_ncld;
    nz = 0;
    if (ncld == 0) break;                                   // leaf: draw from p
    q = make_dist(head_logits + ((size_t)d * B + b) * V, V, tau, scr);
    int kept = -1;
    for (int i = 0; i < ncld; ++i) {
      const int c = cld[i];
      if (tid == 0) {
        const int x = tree_tok[(size_t)b * T + c];
        float a = 0.f;                                      // out-of-range tokens are never kept
        if (x >= 0 && x < V) {
          const float qx = q(x), px = residual(p(x), qx, Z, nz);
          a = qx == 0.f ? (px > 0.f ? 1.f : 0.f) : fminf(1.f, px / qx);
        }
        if (keep_prob) keep_prob[(size_t)b * T + c] = a;
        s_kept = u_node[(size_t)b * T + c] < a ? c : -1;
      }
      __syncthreads();
      kept = s_kept;
      if (kept >= 0) break;
      // normaliser of the residual max(0, p_nz - q) after this rejection
      float part = 0.f;
      for (int v = tid; v < V; v += kThreads) {
        const float qv = q(v);
        part += fmaxf(residual(p(v), qv, Z, nz) - qv, 0.f);
      }
      const float Zn = block_sum(part, scr);
      if (Zn > 0.f) {   // p <= q everywhere cannot reject: p stays
        if (tid == 0) Z[nz] = Zn;
        ++nz;
      }
      __syncthreads();
    }
    if (kept < 0) {                                          // all rejected
      resid = nz > 0;
      break;
    }
    u = kept;
    if (tid == 0) path[plen] = u;
    ++plen;
  }
  int tok;
  if (resid) {
    tok = inverse_cdf([&](int v) { const float qv = q(v); return residual(p(v), qv, Z, nz); }, V, u_bonus[b],
                      s_part, &s_tok, scr);
  } else {
    tok = inverse_cdf([&](int v) { return p(v); }, V, u_bonus[b], s_part, &s_tok, scr);
  }
  __syncthreads();
  if (tid == 0) {
    next_tok[b] = tok;
    accept_len[b] = depth[u];
    best_node[b] = u;
  }
  for (int i = tid; i < plen; i += kThreads)
    accepted_tok[(size_t)b * (depth_max + 1) + i] = tree_tok[(size_t)b * T + path[i]];
}

// The same walk with the distributions held on chip, for V <= 1024 * C: p in
// registers (thread t owns v = t + 1024 j, j < C, the order in which the
// streaming kernel above sums, so p, q, every normaliser and every keep
// probability come out bit for bit the same), q in LDS.  A rejection costs
// one block sum (the residual is updated in place, never recomputed from the
// rows), and the final draw scans p from LDS.
template <int C>
__global__ __launch_bounds__(kThreads) void rejection_accept_regs(
    int T, int V, int depth_max, const int32_t *__restrict__ parent, const int32_t *__restrict__ depth,
    const int32_t *__restrict__ dstart, const float *__restrict__ logits, const float *__restrict__ head_logits,
    int B, const int32_t *__restrict__ tree_tok, float tau, const float *__restrict__ u_node,
    const float *__restrict__ u_bonus, int32_t *__restrict__ accept_len, int32_t *__restrict__ best_node,
    int32_t *__restrict__ next_tok, int32_t *__restrict__ accepted_tok, float *__restrict__ keep_prob) {
  __shared__ BlockScratch scr;
  __shared__ int cld[MEDUSA_MAX_TREE];
  __shared__ int path[MEDUSA_MAX_TREE];
  __shared__ float s_part[kThreads];
  __shared__ float s_dist[kThreads * C];
  __shared__ int s_ncld, s_kept, s_tok;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  if (keep_prob)
    for (int c = tid; c < T; c += kThreads) keep_prob[(size_t)b * T + c] = __builtin_nanf("");
  for (int i = tid; i <= depth_max; i += kThreads) accepted_tok[(size_t)b * (depth_max + 1) + i] = -1;

  // this thread's values of p over the vocabulary (0 past V)
  auto load_dist = [&](float (&d)[C], const float *row) {
    if (tau == 0.f) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int v = tid + kThreads * j;
        if (v < V) {
          const uint64_t key = argmax_key(row[v], v);
          best = key > best ? key : best;
        }
      }
      const int amax = (int)(~(uint32_t)block_max_u64(best, scr));
#pragma unroll
      for (int j = 0; j < C; ++j) d[j] = tid + kThreads * j == amax ? 1.f : 0.f;
      return;
    }
    const float inv_tau = 1.f / tau;
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < C; ++j) {   // the scaled logits first, in place
      const int v = tid + kThreads * j;
      d[j] = v < V ? row[v] * inv_tau : -INFINITY;
      m = fmaxf(m, d[j]);
    }
    m = block_max(m, scr);
    float S = 0.f;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      d[j] = tid + kThreads * j < V ? __expf(d[j] - m) : 0.f;
      S += d[j];
    }
    S = block_sum(S, scr);
#pragma unroll
    for (int j = 0; j < C; ++j) d[j] = d[j] / S;
  };

  // q into s_dist (0 past V), by rolled loops: the same values as load_dist
  auto load_q = [&](const float *row) {
    if (tau == 0.f) {
      uint64_t best = 0;
      for (int v = tid; v < V; v += kThreads) {
        const uint64_t key = argmax_key(row[v], v);
        best = key > best ? key : best;
      }
      const int amax = (int)(~(uint32_t)block_max_u64(best, scr));
      for (int v = tid; v < kThreads * C; v += kThreads) s_dist[v] = v == amax ? 1.f : 0.f;
    } else {
      const float inv_tau = 1.f / tau;
      float m = -INFINITY;
      for (int v = tid; v < V; v += kThreads) m = fmaxf(m, row[v] * inv_tau);
      m = block_max(m, scr);
      float S = 0.f;
      for (int v = tid; v < V; v += kThreads) S += __expf(row[v] * inv_tau - m);
      S = block_sum(S, scr);
      for (int v = tid; v < kThreads * C; v += kThreads) s_dist[v] = v < V ? __expf(row[v] * inv_tau - m) / S : 0.f;
    }
    __syncthreads();
  };

  float pv[C];
  int u = 0, plen = 1;
  if (tid == 0) path[0] = 0;
  while (true) {
    load_dist(pv, logits + ((size_t)b * T + u) * V);
    const int d = depth[u];
    if (tid == 0) {
      int n = 0;
      if (d < depth_max)
        for (int c = dstart[d + 1]; c < dstart[d + 2]; ++c)
          if (parent[c] == u) cld[n++] = c;
      s_ncld = n;
    }
    __syncthreads();
    const int ncld = s_ncld;
    if (ncld == 0) break;                                   // leaf: draw from p
    load_q(head_logits + ((size_t)d * B + b) * V);
    int kept = -1;
    for (int i = 0; i < ncld; ++i) {
      const int c = cld[i];
      const int x = tree_tok[(size_t)b * T + c];
      const bool in_range = x >= 0 && x < V;
      // the keep probability, by the thread that holds token x (thread 0 for
      // an out-of-range token, which is never kept)
      if (in_range ? tid == x % kThreads : tid == 0) {
        float a = 0.f;
        if (in_range) {
          const int jx = x / kThreads;
          float px = 0.f;
#pragma unroll
          for (int j = 0; j < C; ++j)
            if (j == jx) px = pv[j];
          const float qx = s_dist[x];
          a = qx == 0.f ? (px > 0.f ? 1.f : 0.f) : fminf(1.f, px / qx);
        }
        if (keep_prob) keep_prob[(size_t)b * T + c] = a;
        s_kept = u_node[(size_t)b * T + c] < a ? c : -1;
      }
      __syncthreads();
      kept = s_kept;
      if (kept >= 0) break;
      // p <- max(0, p - q) / its sum (p <= q everywhere cannot reject: p stays)
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < C; ++j) part += fmaxf(pv[j] - s_dist[tid + kThreads * j], 0.f);
      const float Zn = block_sum(part, scr);
      if (Zn > 0.f) {
#pragma unroll
        for (int j = 0; j < C; ++j) pv[j] = fmaxf(pv[j] - s_dist[tid + kThreads * j], 0.f) / Zn;
      }
      __syncthreads();
    }
    if (kept < 0) break;                                     // all rejected: draw from the residual
    u = kept;
    if (tid == 0) path[plen] = u;
    ++plen;
  }
  __syncthreads();   // every thread is done with q
#pragma unroll
  for (int j = 0; j < C; ++j) s_dist[tid + kThreads * j] = pv[j];
  __syncthreads();
  const int tok = inverse_cdf([&](int v) { return s_dist[v]; }, V, u_bonus[b], s_part, &s_tok, scr);
  __syncthreads();
  if (tid == 0) {
    next_tok[b] = tok;
    accept_len[b] = depth[u];
    best_node[b] = u;
  }
  for (int i = tid; i < plen; i += kThreads)
    accepted_tok[(size_t)b * (depth_max + 1) + i] = tree_tok[(size_t)b * T + path[i]];
}

}  // namespace

extern "C" medusa_status rejection_accept(medusa_stream_t stream, const medusa_tree *t, int B, int V, int K,
                                          const float *logits, const float *head_logits, const int32_t *tree_tok,
                                          float temperature, const float *u_node, const float *u_bonus,
                                          int32_t *accept_len, int32_t *best_node, int32_t *next_tok,
                                          int32_t *accepted_tok, float *keep_prob) {
  TraceRange tr("rejection_accept");
  medusa_status s = check_tree_on_device(t);
  if (s != MEDUSA_OK) return s;
  if (B < 1 || V < 1) return fail(MEDUSA_ERR_ARG, "rejection_accept: B=%d V=%d", B, V);
  if (K < t->depth_max)
    return fail(MEDUSA_ERR_SHAPE, "rejection_accept: %d heads for a tree of depth %d", K, t->depth_max);
  if (!(temperature >= 0.f) || !isfinite(temperature))
    return fail(MEDUSA_ERR_ARG, "rejection_accept: temperature must be >= 0");
  if (!logits || !head_logits || !tree_tok || !u_node || !u_bonus || !accept_len || !best_node || !next_tok ||
      !accepted_tok)
    return fail(MEDUSA_ERR_ARG, "rejection_accept: NULL pointer");
  if (validate_enabled()) {  // NaN / +inf logits of either distribution; tree tokens outside [0, V)
    ValidateSpec v;
    v.a = logits;
    v.na = (size_t)B * t->T * V;
    v.b = head_logits;
    v.nb = (size_t)K * B * V;
    v.posinf_bad = true;
    v.tok = tree_tok;
    v.nt = (size_t)B * t->T;
    v.V = V;
    s = validate_inputs(as_stream(stream), "rejection_accept", v);
    if (s != MEDUSA_OK) return s;
  }
  // vocabularies up to 32768: both distributions in registers; beyond, the
  // streaming kernel
  auto kern = V <= kThreads * 4 ? rejection_accept_regs<4>
            : V <= kThreads * 8 ? rejection_accept_regs<8>
            : V <= kThreads * 16 ? rejection_accept_regs<16>
            : V <= kThreads * 32 ? rejection_accept_regs<32>
                                 : rejection_accept_kernel;
  MEDUSA_LAUNCH("rejection_accept", kern, dim3(B), dim3(kThreads), 0, as_stream(stream), t->T, V,
                     t->depth_max, t->d_parent, t->d_depth, t->d_dstart, logits, head_logits, B, tree_tok,
                     temperature, u_node, u_bonus, accept_len, best_node, next_tok, accepted_tok, keep_prob);
  return check_launch("rejection_accept");
}
