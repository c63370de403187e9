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
constexpr int kBufferWord3 = 0x00020000;     // buffer resource word 3 on gfx9: 32-bit elements

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

// x, opaque to the optimiser: values derived from it inside a loop are
// recomputed there (one instruction each) rather than hoisted out of the loop
// and held in registers across it.  Register-only; no memory is touched.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Block reductions with one barrier each: the wave results go to one of two
// scratch halves, used in turn.  A thread writes half h again only two calls
// later, after the barrier of the call in between, which every thread reaches
// only once it has read half h.  Every thread makes the same calls.
struct PingPong {
  float f[2][kWaves];
  uint64_t k[2][kWaves];
};
struct Reducer {
  PingPong &s;
  int ph = 0;
  __device__ float sum(float v) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) s.f[ph][threadIdx.x >> 6] = v;
    __syncthreads();
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) r += s.f[ph][w];
    ph ^= 1;
    return r;
  }
  __device__ float max(float v) {
    v = wave_maxf(v);
    if ((threadIdx.x & 63) == 0) s.f[ph][threadIdx.x >> 6] = v;
    __syncthreads();
    float r = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) r = fmaxf(r, s.f[ph][w]);
    ph ^= 1;
    return r;
  }
  __device__ uint64_t max_u64(uint64_t v) {
    v = wave_max_u64(v);
    if ((threadIdx.x & 63) == 0) s.k[ph][threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t r = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) r = s.k[ph][w] > r ? s.k[ph][w] : r;
    ph ^= 1;
    return r;
  }
};

// The same walk with the distributions held on chip, for V <= 1024 * C.
// Thread t holds p(v) for v = t + 1024 j, j < C, in registers; q sits in LDS.
// Each node's two rows are read once, every load of a row in flight at once
// (buffer loads, which return 0 past the row's end).  The sequence's tokens
// and uniforms and the child offsets are copied to LDS at the start, so a
// node costs one global lookup (its child list) besides its rows.  p at each
// child's token is gathered into LDS by the thread holding it; every thread
// then evaluates each keep probability itself (the residual normalisers so
// far applied to that value), so a decision needs no broadcast, and a
// rejection costs one block sum, the residual max(0, p - q) / Z replacing p in
// place.  The final draw stores p in LDS padded by one word per C, so thread
// t reads its contiguous range [t C, t C + C) without bank conflicts, and
// scans the range sums with wave shuffles and one pass over the wave totals.
template <int C>
__global__ __launch_bounds__(kThreads) void rejection_accept_regs(
    int T, int V, int depth_max, const int32_t *__restrict__ depth, const int32_t *__restrict__ cstart,
    const int32_t *__restrict__ clist, const float *__restrict__ logits, const float *__restrict__ head_logits,
    int B, const int32_t *__restrict__ tree_tok, float tau, const float *__restrict__ u_node,
    const float *__restrict__ u_bonus, int32_t *__restrict__ accept_len, int32_t *__restrict__ best_node,
    int32_t *__restrict__ next_tok, int32_t *__restrict__ accepted_tok, float *__restrict__ keep_prob) {
  constexpr int kPad = kThreads * C + kThreads;   // element v at v + v / C
  __shared__ PingPong pp;
  __shared__ int s_cstart[MEDUSA_MAX_TREE + 1];
  __shared__ int s_tok_all[MEDUSA_MAX_TREE];
  __shared__ float s_u_all[MEDUSA_MAX_TREE];
  __shared__ int cld[MEDUSA_MAX_TREE];
  __shared__ float cpx[MEDUSA_MAX_TREE];   // p at each child's token before any rejection
  __shared__ float rZ[kMaxResid];          // 1 / normaliser of each residual so far
  __shared__ float s_dist[kPad];
  __shared__ float s_wt[kWaves];
  __shared__ int s_tok;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  Reducer red{pp};
  auto at = [](int v) { return v + v / C; };
  constexpr int kStride = kThreads + kThreads / C;   // at(v + 1024) - at(v)
  const int tat = at(tid);
  for (int c = tid; c < T; c += kThreads) {
    s_tok_all[c] = tree_tok[(size_t)b * T + c];
    s_u_all[c] = u_node[(size_t)b * T + c];
    if (keep_prob) keep_prob[(size_t)b * T + c] = __builtin_nanf("");
  }
  for (int c = tid; c <= T; c += kThreads) s_cstart[c] = cstart[c];
  for (int i = tid; i <= depth_max; i += kThreads)
    accepted_tok[(size_t)b * (depth_max + 1) + i] = i == 0 ? tree_tok[(size_t)b * T] : -1;
  __syncthreads();

  // this thread's values of softmax(row / tau) (one-hot at the argmax for
  // tau = 0), 0 past V
  auto load_dist = [&](float (&d)[C], const float *row) {
    // a buffer resource over the row: reads past its V words return 0
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row), (short)0, V * 4, kBufferWord3);
    auto ld = [&](int v) {
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, v * 4, 0, 0));
    };
    const int t = opaque(tid);
    if (tau == 0.f) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int v = t + kThreads * j;
        const uint64_t key = argmax_key(ld(v), v);
        best = v < V && key > best ? key : best;
      }
      const int amax = (int)(~(uint32_t)red.max_u64(best));
#pragma unroll
      for (int j = 0; j < C; ++j) d[j] = t + kThreads * j == amax ? 1.f : 0.f;
      return;
    }
    const float inv_tau = 1.f / tau;
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int v = t + kThreads * j;
      const float x = ld(v);
      d[j] = v < V ? x * inv_tau : -INFINITY;
      m = fmaxf(m, d[j]);
    }
    m = red.max(m);
    float S = 0.f;
#pragma unroll
    for (int j = 0; j < C; ++j) {   // past V: exp(-inf) = 0
      d[j] = __expf(d[j] - m);
      S += d[j];
    }
    const float rS = 1.f / red.sum(S);
#pragma unroll
    for (int j = 0; j < C; ++j) d[j] *= rS;
  };

  float pv[C];
  int u = 0, plen = 1;
  while (true) {
    const int d = depth[u];
    const int c0 = s_cstart[u], ncld = s_cstart[u + 1] - c0;
    for (int i = tid; i < ncld; i += kThreads) cld[i] = clist[c0 + i];
    // q (when u has children) through the registers into LDS, then p; one
    // copy of the loads, so the second row's cannot be hoisted over the first
    // row's reductions and double the registers in use
#pragma unroll 1
    for (int r = ncld > 0 ? 0 : 1; r < 2; ++r) {
      load_dist(pv, r == 0 ? head_logits + ((size_t)d * B + b) * V : logits + ((size_t)b * T + u) * V);
      if (r == 0) {
        const int o = opaque(tat);
#pragma unroll
        for (int j = 0; j < C; ++j) s_dist[o + kStride * j] = pv[j];
      }
    }
    // the reductions' barriers have published cld and q
    if (ncld == 0) break;                              // leaf: draw from p
    for (int i = 0; i < ncld; ++i) {
      const int x = s_tok_all[cld[i]];
      if (x >= 0 && x < V && tid == x % kThreads) {
        const int jx = x / kThreads;
        float px = 0.f;
#pragma unroll
        for (int j = 0; j < C; ++j)
          if (j == jx) px = pv[j];
        cpx[i] = px;
      }
    }
    __syncthreads();
    int kept = -1, nz = 0;
    for (int i = 0; i < ncld; ++i) {
      const int c = cld[i];
      const int x = s_tok_all[c];
      float a = 0.f;                                   // out-of-range tokens are never kept
      if (x >= 0 && x < V) {
        const float qx = s_dist[at(x)];
        float px = cpx[i];
        for (int j = 0; j < nz; ++j) px = fmaxf(px - qx, 0.f) * rZ[j];
        a = qx == 0.f ? (px > 0.f ? 1.f : 0.f) : fminf(1.f, px / qx);
      }
      if (tid == 0 && keep_prob) keep_prob[(size_t)b * T + c] = a;
      if (s_u_all[c] < a) {
        kept = c;
        break;
      }
      // p <- max(0, p - q) / its sum (p <= q everywhere cannot reject: p stays)
      float part = 0.f;
      const int o = opaque(tat);
#pragma unroll
      for (int j = 0; j < C; ++j) part += fmaxf(pv[j] - s_dist[o + kStride * j], 0.f);
      const float Zn = red.sum(part);
      if (Zn > 0.f) {
        const float r = 1.f / Zn;
        const int o2 = opaque(tat);
#pragma unroll
        for (int j = 0; j < C; ++j) pv[j] = fmaxf(pv[j] - s_dist[o2 + kStride * j], 0.f) * r;
        rZ[nz] = r;   // by every thread, so each reads back its own write
        ++nz;
      }
    }
    __syncthreads();   // every thread is done with this node's q, cld and cpx
    if (kept < 0) break;                               // all rejected: draw from the residual
    if (tid == 0) accepted_tok[(size_t)b * (depth_max + 1) + plen] = s_tok_all[kept];
    u = kept;
    ++plen;
  }

  // inverse-CDF draw from p: the smallest v with p(0) + ... + p(v) > u * sum,
  // else (rounding) the last v with p(v) > 0
#pragma unroll
  for (int j = 0; j < C; ++j) s_dist[tat + kStride * j] = pv[j];
  if (tid == 0) s_tok = -1;
  __syncthreads();
  float own = 0.f;
#pragma unroll
  for (int i = 0; i < C; ++i) own += s_dist[tid * (C + 1) + i];
  float incl = own;   // inclusive scan over the wave's lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  float excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.f;
  if (lane == 63) s_wt[wave] = incl;
  __syncthreads();
  float base = 0.f, total = 0.f;
  for (int w = 0; w < kWaves; ++w) {   // the same running sum for every thread
    if (w == wave) base = total;
    total += s_wt[w];
  }
  // thread t's share of the running sum is [lo, hi); hi of one thread is lo
  // of the next bit for bit, so at most one thread claims the target
  const float lo = base + excl, hi = base + incl;
  const float target = u_bonus[b] * total;
  if (hi > lo && target >= lo && target < hi) {
    float acc = lo;
    int tok = -1;
    for (int i = 0; i < C && tok < 0; ++i) {
      const float x = s_dist[tid * (C + 1) + i];
      acc += x;
      if (x > 0.f && acc > target) tok = tid * C + i;
    }
    for (int i = C - 1; i >= 0 && tok < 0; --i)
      if (s_dist[tid * (C + 1) + i] > 0.f) tok = tid * C + i;
    s_tok = tok;
  }
  __syncthreads();
  int tok = s_tok;
  if (tok < 0) {
    int last = -1;
#pragma unroll
    for (int j = 0; j < C; ++j)
      if (pv[j] > 0.f) last = tid + kThreads * j;
    tok = (int)red.max_u64((uint64_t)(uint32_t)(last + 1)) - 1;
  }
  if (tid == 0) {
    next_tok[b] = tok;
    accept_len[b] = depth[u];
    best_node[b] = u;
  }
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
  if (V > kThreads * 32) {
    MEDUSA_LAUNCH("rejection_accept", rejection_accept_kernel, dim3(B), dim3(kThreads), 0, as_stream(stream), t->T,
                  V, t->depth_max, t->d_parent, t->d_depth, t->d_dstart, logits, head_logits, B, tree_tok,
                  temperature, u_node, u_bonus, accept_len, best_node, next_tok, accepted_tok, keep_prob);
  } else {
    auto kern = V <= kThreads * 4 ? rejection_accept_regs<4>
              : V <= kThreads * 8 ? rejection_accept_regs<8>
              : V <= kThreads * 16 ? rejection_accept_regs<16>
                                   : rejection_accept_regs<32>;
    MEDUSA_LAUNCH("rejection_accept", kern, dim3(B), dim3(kThreads), 0, as_stream(stream), t->T, V, t->depth_max,
                  t->d_depth, t->d_cstart, t->d_clist, logits, head_logits, B, tree_tok, temperature, u_node,
                  u_bonus, accept_len, best_node, next_tok, accepted_tok, keep_prob);
  }
  return check_launch("rejection_accept");
}
