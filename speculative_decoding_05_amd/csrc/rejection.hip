// Rejection-sampling acceptance over the candidate tree (the comparison
// point of typical acceptance).  One block of 1024 threads per sequence walks
// the tree from the root: at the current node u it forms the verification
// distribution p (softmax of u's row at the temperature) and the drafting
// head's distribution q (softmax of head depth(u)'s row for this sequence),
// tries u's children in rank order -- child x is kept iff its uniform is
// below min(1, p(x)/q(x)), and a rejected child replaces p by the
// renormalised residual max(0, p - q) -- and moves to the first kept child.
// When no child is kept, or u is a leaf, the next token is drawn by inverse
// CDF from the current p.  Temperature 0 uses one-hot distributions at the
// argmax (lowest index): greedy verification.
//
// Vocabularies up to 32768 hold p in registers and q in LDS
// (rejection_accept_regs); larger ones stream the two rows from L2
// (rejection_accept_stream).  Both read a row with buffer loads, all of a
// thread's loads in flight together, and stage the sequence's tokens,
// uniforms and the tree's child offsets in LDS, so the walk itself makes no
// dependent global loads beyond each node's child list and rows.
#include <math.h>

#include "common.h"

using namespace medusa;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxResid = MEDUSA_MAX_TREE;   // rejections at one node <= its children

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

// argmax key: larger value first, then smaller index
__device__ __forceinline__ uint64_t argmax_key(float x, int i) {
  uint32_t u = __builtin_bit_cast(uint32_t, x == 0.f ? 0.f : x);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)i);
}

// x, opaque to the optimiser: values derived from it inside a loop are
// recomputed there (one instruction each) rather than hoisted out of the loop
// and held in registers across it.  Register-only; no memory is touched.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A value every lane of the wave holds alike (read from LDS, or a block
// reduction's result), marked uniform for the compiler: branches on it stay
// scalar, and addresses built from it stay in scalar registers.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uni(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ uint64_t uni(uint64_t x) {
  return ((uint64_t)(uint32_t)uni((int)(x >> 32)) << 32) | (uint32_t)uni((int)(uint32_t)x);
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
    return uni(r);
  }
  __device__ float max(float v) {
    v = wave_maxf(v);
    if ((threadIdx.x & 63) == 0) s.f[ph][threadIdx.x >> 6] = v;
    __syncthreads();
    float r = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) r = fmaxf(r, s.f[ph][w]);
    ph ^= 1;
    return uni(r);
  }
  __device__ uint64_t max_u64(uint64_t v) {
    v = wave_max_u64(v);
    if ((threadIdx.x & 63) == 0) s.k[ph][threadIdx.x >> 6] = v;
    __syncthreads();
    uint64_t r = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) r = s.k[ph][w] > r ? s.k[ph][w] : r;
    ph ^= 1;
    return uni(r);
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
    const int c0 = uni(s_cstart[u]), ncld = uni(s_cstart[u + 1]) - c0;
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
      const int c = uni(cld[i]);
      const int x = uni(s_tok_all[c]);
      float a = 0.f;                                   // out-of-range tokens are never kept
      if (x >= 0 && x < V) {
        const float qx = s_dist[at(x)];
        float px = cpx[i];
        for (int j = 0; j < nz; ++j) px = fmaxf(px - qx, 0.f) * rZ[j];
        a = qx == 0.f ? (px > 0.f ? 1.f : 0.f) : fminf(1.f, px / qx);
      }
      if (tid == 0 && keep_prob) keep_prob[(size_t)b * T + c] = a;
      if (uni(s_u_all[c]) < uni(a)) {
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
  int tok = uni(s_tok);
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

// Vocabularies beyond what a block holds on chip: the same walk with the two
// rows of a node streamed (L2-resident after the first pass): one pass per
// distribution, 32 loads in flight per thread.  p and q at the children's tokens are
// gathered in parallel; the residual after j rejections is recomputed per
// element from p, q and the j normalisers, with the same arithmetic as the
// keep probabilities.  The final draw makes one pass over tiles of kTile
// values (each thread sums a contiguous run of kStreamU values of a tile
// staged in LDS; a wave scan and the wave totals give each tile's sum, one
// barrier per tile) and rescans the one tile that holds the target.
constexpr int kStreamU = 8;
constexpr int kTile = kThreads * kStreamU;
constexpr int kTilePad = kTile + kThreads;   // local index l at l + l / kStreamU
constexpr int kMaxTiles = 1024;              // V <= 8 Mi

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float *row, int V) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row), (short)0, V * 4, kBufferWord3);
}
__device__ __forceinline__ float ldb(__amdgpu_buffer_rsrc_t rs, int v) {   // 0 past the row
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, v * 4, 0, 0));
}

// softmax(row / tau) (amax < 0) or one-hot at amax
struct RowDist {
  __amdgpu_buffer_rsrc_t rs;
  float m, rS, inv_tau;
  int amax;
  __device__ float e(float x) const { return __expf(x * inv_tau - m); }
  __device__ float at(float x, int v) const { return amax >= 0 ? (v == amax ? 1.f : 0.f) : e(x) * rS; }
};

// f(v, x) for each v < V this thread visits (v = tid + 1024 i), x = row[v];
// N loads in flight per thread (N = 32: 128 KB per block, about what one
// round trip to L2 or HBM takes at a CU's share of the bandwidth)
template <int N, typename F>
__device__ __forceinline__ void stream1(__amdgpu_buffer_rsrc_t rs, int V, F f) {
  const int t = opaque((int)threadIdx.x);
  for (int v0 = t; v0 < V; v0 += kThreads * N) {
    float x[N];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = ldb(rs, v0 + kThreads * i);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (v0 + kThreads * i < V) f(v0 + kThreads * i, x[i]);
  }
}
template <int N, typename F>
__device__ __forceinline__ void stream2(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int V, F f) {
  const int t = opaque((int)threadIdx.x);
  for (int v0 = t; v0 < V; v0 += kThreads * N) {
    float x[N], y[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      x[i] = ldb(ra, v0 + kThreads * i);
      y[i] = ldb(rb, v0 + kThreads * i);
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (v0 + kThreads * i < V) f(v0 + kThreads * i, x[i], y[i]);
  }
}
constexpr int kOne = 32, kTwo = 16;   // loads in flight per thread: one row, two rows

// One pass over the row: each thread keeps a running max m of row/tau and
// the sum S of e^(y - m) over its values, rescaled when m grows; the block
// then merges the (m, S) pairs.
__device__ RowDist make_rowdist(const float *row, int V, float tau, Reducer &red) {
  RowDist d;
  d.rs = row_rsrc(row, V);
  d.amax = -1;
  d.m = 0.f;
  d.rS = 1.f;
  d.inv_tau = 0.f;
  if (tau == 0.f) {
    uint64_t best = 0;
    stream1<kOne>(d.rs, V, [&](int v, float x) {
      const uint64_t k = argmax_key(x, v);
      best = k > best ? k : best;
    });
    d.amax = (int)(~(uint32_t)red.max_u64(best));
    return d;
  }
  d.inv_tau = 1.f / tau;
  float m = -INFINITY, S = 0.f;
  stream1<kOne>(d.rs, V, [&](int, float x) {
    const float y = x * d.inv_tau;
    if (y > -INFINITY) {   // a -inf logit adds nothing
      const float mn = fmaxf(m, y);
      S = S * __expf(m - mn) + __expf(y - mn);
      m = mn;
    }
  });
  d.m = red.max(m);
  d.rS = 1.f / red.sum(m > -INFINITY ? S * __expf(m - d.m) : 0.f);
  return d;
}

// p after the rejections whose reciprocal normalisers are rZ[0..nz)
__device__ __forceinline__ float residual(float p, float q, const float *rZ, int nz) {
  for (int j = 0; j < nz; ++j) p = fmaxf(p - q, 0.f) * rZ[j];
  return p;
}

__global__ __launch_bounds__(kThreads) void rejection_accept_stream(
    int T, int V, int depth_max, const int32_t *__restrict__ depth, const int32_t *__restrict__ cstart,
    const int32_t *__restrict__ clist, const float *__restrict__ logits, const float *__restrict__ head_logits,
    int B, const int32_t *__restrict__ tree_tok, float tau, const float *__restrict__ u_node,
    const float *__restrict__ u_bonus, int32_t *__restrict__ accept_len, int32_t *__restrict__ best_node,
    int32_t *__restrict__ next_tok, int32_t *__restrict__ accepted_tok, float *__restrict__ keep_prob) {
  __shared__ PingPong pp;
  __shared__ int s_cstart[MEDUSA_MAX_TREE + 1];
  __shared__ int s_tok_all[MEDUSA_MAX_TREE];
  __shared__ float s_u_all[MEDUSA_MAX_TREE];
  __shared__ int cld[MEDUSA_MAX_TREE];
  __shared__ float cpx[MEDUSA_MAX_TREE], cqx[MEDUSA_MAX_TREE];   // p and q at each child's token
  __shared__ float rZ[kMaxResid];
  __shared__ float s_tile[2][kTilePad];
  __shared__ float s_wt[2][kWaves];
  __shared__ float s_base[kMaxTiles + 1];   // running sum of the final distribution before each tile
  __shared__ int s_tok, s_kstar;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  Reducer red{pp};
  for (int c = tid; c < T; c += kThreads) {
    s_tok_all[c] = tree_tok[(size_t)b * T + c];
    s_u_all[c] = u_node[(size_t)b * T + c];
    if (keep_prob) keep_prob[(size_t)b * T + c] = __builtin_nanf("");
  }
  for (int c = tid; c <= T; c += kThreads) s_cstart[c] = cstart[c];
  for (int i = tid; i <= depth_max; i += kThreads)
    accepted_tok[(size_t)b * (depth_max + 1) + i] = i == 0 ? tree_tok[(size_t)b * T] : -1;
  __syncthreads();

  RowDist P, Q;
  int u = 0, plen = 1, nz = 0;
  while (true) {
    const int d = depth[u];
    const int c0 = uni(s_cstart[u]), ncld = uni(s_cstart[u + 1]) - c0;
    for (int i = tid; i < ncld; i += kThreads) cld[i] = clist[c0 + i];
    P = make_rowdist(logits + ((size_t)b * T + u) * V, V, tau, red);   // its barriers publish cld
    Q = P;
    nz = 0;
    if (ncld == 0) break;                                               // leaf: draw from p
    Q = make_rowdist(head_logits + ((size_t)d * B + b) * V, V, tau, red);
    for (int i = tid; i < ncld; i += kThreads) {
      const int x = s_tok_all[cld[i]];
      const bool in = x >= 0 && x < V;
      cpx[i] = in ? P.at(ldb(P.rs, x), x) : 0.f;
      cqx[i] = in ? Q.at(ldb(Q.rs, x), x) : 0.f;
    }
    __syncthreads();
    int kept = -1;
    for (int i = 0; i < ncld; ++i) {
      const int c = uni(cld[i]);
      const int x = uni(s_tok_all[c]);
      float a = 0.f;                                                    // out-of-range tokens are never kept
      if (x >= 0 && x < V) {
        const float qx = cqx[i], px = residual(cpx[i], qx, rZ, nz);
        a = qx == 0.f ? (px > 0.f ? 1.f : 0.f) : fminf(1.f, px / qx);
      }
      if (tid == 0 && keep_prob) keep_prob[(size_t)b * T + c] = a;
      if (uni(s_u_all[c]) < uni(a)) {
        kept = c;
        break;
      }
      float part = 0.f;
      stream2<kTwo>(P.rs, Q.rs, V, [&](int v, float xp, float xq) {
        const float qv = Q.at(xq, v);
        part += fmaxf(residual(P.at(xp, v), qv, rZ, nz) - qv, 0.f);
      });
      const float Zn = red.sum(part);
      if (Zn > 0.f) {   // p <= q everywhere cannot reject: p stays
        rZ[nz] = 1.f / Zn;   // by every thread, so each reads back its own write
        ++nz;
      }
    }
    __syncthreads();   // every thread is done with this node's cld, cpx, cqx
    if (kept < 0) break;                                                // all rejected: the residual
    if (tid == 0) accepted_tok[(size_t)b * (depth_max + 1) + plen] = s_tok_all[kept];
    u = kept;
    ++plen;
  }

  // the final distribution, f(v) = residual of p after nz rejections (p itself when nz = 0)
  auto f = [&](int v, float xp, float xq) {
    const float p = P.at(xp, v);
    return nz > 0 ? residual(p, Q.at(xq, v), rZ, nz) : p;
  };
  const int ntiles = (V + kTile - 1) / kTile;
  // tile k's raw values (thread t: v = k kTile + 1024 i + t), then f of them
  // into s_tile[h]; split so that a tile's loads are in flight while the
  // tile before it is scanned
  float xr[kStreamU], yr[kStreamU];
  auto load_tile = [&](int k) {
    const int v0 = k * kTile + tid;
#pragma unroll
    for (int i = 0; i < kStreamU; ++i) {
      xr[i] = ldb(P.rs, v0 + kThreads * i);
      yr[i] = nz > 0 ? ldb(Q.rs, v0 + kThreads * i) : 0.f;
    }
  };
  auto put_tile = [&](int k, int h) {
    const int v0 = k * kTile + tid;
#pragma unroll
    for (int i = 0; i < kStreamU; ++i) {
      const int l = tid + kThreads * i, v = v0 + kThreads * i;
      s_tile[h][l + l / kStreamU] = v < V ? f(v, xr[i], yr[i]) : 0.f;
    }
  };
  // thread t's run [t U, t U + U) of the staged tile: its sum and the
  // inclusive scan of the sums over the wave; lane 63 posts the wave total
  auto scan = [&](int h, float &own, float &incl) {
    own = 0.f;
#pragma unroll
    for (int i = 0; i < kStreamU; ++i) own += s_tile[h][tid * (kStreamU + 1) + i];
    incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) s_wt[h][wave] = incl;
  };
  // a tile's sum: its wave totals added in wave order, the order in which
  // pass 2 forms each thread's running sum inside the tile, so the tile's last
  // upper bound there equals the next tile's base exactly
  auto tile_total = [&](int h) {
    float t = 0.f;
    for (int w = 0; w < kWaves; ++w) t += s_wt[h][w];
    return t;
  };
  // pass 1: every tile's sum, one barrier per tile (buffers used in turn)
  float run = 0.f;
  if (tid == 0) s_base[0] = 0.f;
  load_tile(0);
  put_tile(0, 0);
  if (ntiles > 1) load_tile(1);
  for (int k = 0; k < ntiles; ++k) {
    const int h = k & 1;
    __syncthreads();
    if (k > 0) {   // tile k-1's wave totals are complete
      run += tile_total(h ^ 1);
      if (tid == 0) s_base[k] = run;
    }
    float own, incl;
    scan(h, own, incl);
    if (k + 1 < ntiles) {
      put_tile(k + 1, h ^ 1);
      if (k + 2 < ntiles) load_tile(k + 2);
    }
  }
  __syncthreads();
  run += tile_total((ntiles - 1) & 1);
  if (tid == 0) {
    s_base[ntiles] = run;
    s_kstar = -1;
    s_tok = -1;
  }
  __syncthreads();
  const float total = run, target = u_bonus[b] * total;
  for (int k = tid; k < ntiles; k += kThreads)
    if (s_base[k + 1] > s_base[k] && target >= s_base[k] && target < s_base[k + 1]) s_kstar = k;
  __syncthreads();
  const int ks = uni(s_kstar);
  if (ks >= 0) {   // pass 2: rescan the tile that holds the target
    load_tile(ks);
    put_tile(ks, 0);
    __syncthreads();
    float own, incl;
    scan(0, own, incl);
    float excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.f;
    __syncthreads();
    float wb = 0.f;
    for (int w = 0; w < wave; ++w) wb += s_wt[0][w];
    // the same running sums as pass 1: hi of one thread is lo of the next, and
    // the tile's last hi is s_base[ks + 1]
    const float lo = s_base[ks] + (wb + excl), hi = s_base[ks] + (wb + incl);
    if (hi > lo && target >= lo && target < hi) {
      float acc = lo;
      int tok = -1;
      for (int i = 0; i < kStreamU && tok < 0; ++i) {
        const float x = s_tile[0][tid * (kStreamU + 1) + i];
        acc += x;
        if (x > 0.f && acc > target) tok = ks * kTile + tid * kStreamU + i;
      }
      for (int i = kStreamU - 1; i >= 0 && tok < 0; --i)
        if (s_tile[0][tid * (kStreamU + 1) + i] > 0.f) tok = ks * kTile + tid * kStreamU + i;
      s_tok = tok;
    }
    __syncthreads();
  }
  int tok = uni(s_tok);
  if (tok < 0) {   // rounding left the target past every run: the last v with f(v) > 0
    int last = -1;
    stream2<kTwo>(P.rs, Q.rs, V, [&](int v, float xp, float xq) {
      if (f(v, xp, xq) > 0.f) last = v;
    });
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
  if (V > kMaxTiles * kTile)
    return fail(MEDUSA_ERR_UNSUPPORTED, "rejection_accept: V=%d > %d", V, kMaxTiles * kTile);
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
  // vocabularies up to 32768: p in registers, q in LDS; beyond, the rows streamed
  auto kern = V <= kThreads * 4 ? rejection_accept_regs<4>
            : V <= kThreads * 8 ? rejection_accept_regs<8>
            : V <= kThreads * 16 ? rejection_accept_regs<16>
            : V <= kThreads * 32 ? rejection_accept_regs<32>
                                 : rejection_accept_stream;
  MEDUSA_LAUNCH("rejection_accept", kern, dim3(B), dim3(kThreads), 0, as_stream(stream), t->T, V, t->depth_max,
                t->d_depth, t->d_cstart, t->d_clist, logits, head_logits, B, tree_tok, temperature, u_node, u_bonus,
                accept_len, best_node, next_tok, accepted_tok, keep_prob);
  return check_launch("rejection_accept");
}
