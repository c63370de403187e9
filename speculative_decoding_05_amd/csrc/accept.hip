// Typical acceptance over the candidate tree.
//
// Row pass (one block per 4096-wide chunk of the verification row of a node
// that has children): every thread folds its 16 values into running
// statistics of y = z / temperature -- max m, S = sum e^(y-m),
// E = sum e^(y-m) (y-m) -- and the argmax of z (lowest index on ties); one
// block reduction merges the statistics (rescaling by e^(m_i - m)) with DPP
// row steps, readlane and LDS, and the chunk's (m, S, E, argmax) goes to the
// workspace.  Then H = ln S - E/S.
// Scan (one block per sequence): merge the chunk partials of every internal
// row into its threshold min(eps, delta e^-H); decide every candidate against
// its parent's row; a node is accepted iff every node on its path (the root
// excepted) is, which is one AND over the node's ancestor bitmask; pick the
// deepest accepted node (smallest index on ties), write its path, and take the
// next greedy token from its row.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "common.h"

using namespace medusa;

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;                  // row pass
constexpr int kVec = 4;                        // float4 per thread: 4096-wide chunks (measured
                                               // faster than 16384-wide ones at every shape)
constexpr int kScanThreads = 512;              // scan
constexpr int kBatch = 8;                      // independent loads issued together
constexpr int kLeafBatch = 16;                 // float4 loads per thread for a leaf row's argmax
constexpr int kLeafParts = 8;                  // scan blocks per sequence (at most)
constexpr float kLog2e = 1.4426950408889634f;

struct Part {  // 32 bytes
  float m, S, E, amax_val;
  int amax_idx, pad0, pad1, pad2;
};

// When the winner of sequence b is a leaf, the scan's blocks of b each take
// the argmax of a share of its row and fold it into `key` (larger value
// first, then smaller index); the last of them to count itself in `cnt`
// decodes the token.  The row pass of the same call zeroes both.
struct LeafSlot {  // 16 bytes
  unsigned long long key;
  unsigned int cnt, pad;
};

__device__ __forceinline__ unsigned long long argmax_order_key(float x, int i) {
  uint32_t u = __builtin_bit_cast(uint32_t, x == 0.f ? 0.f : x);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (uint32_t)(~(uint32_t)i);
}

// running statistics: max m of y, S = sum e^(y-m), E = sum e^(y-m)(y-m),
// argmax (av, ai) of z with the lowest index on ties
struct Stat {
  float m, S, E, av;
  int ai;
};

__device__ __forceinline__ void arg_better(float &bv, int &bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

__device__ __forceinline__ Stat empty_stat() { return {-INFINITY, 0.f, 0.f, -INFINITY, 0x7fffffff}; }

__device__ __forceinline__ Stat combine(const Stat &a, const Stat &b) {
  Stat r;
  r.m = fmaxf(a.m, b.m);
  r.S = 0.f;
  r.E = 0.f;
  if (a.S > 0.f) {
    const float d = a.m - r.m;
    const float w = exp2f(d * kLog2e);
    r.S += w * a.S;
    r.E += w * (a.E + d * a.S);
  }
  if (b.S > 0.f) {
    const float d = b.m - r.m;
    const float w = exp2f(d * kLog2e);
    r.S += w * b.S;
    r.E += w * (b.E + d * b.S);
  }
  r.av = a.av;
  r.ai = a.ai;
  arg_better(r.av, r.ai, b.av, b.ai);
  return r;
}

template <int CTRL>
__device__ __forceinline__ Stat dpp_stat(const Stat &s) {
  return {dppf<CTRL>(s.m), dppf<CTRL>(s.S), dppf<CTRL>(s.E), dppf<CTRL>(s.av),
          static_cast<int>(dpp<CTRL>(static_cast<uint32_t>(s.ai)))};
}

__device__ __forceinline__ Stat lane_stat(const Stat &s, int lane) {
  return {readlanef(s.m, lane), readlanef(s.S, lane), readlanef(s.E, lane), readlanef(s.av, lane),
          static_cast<int>(readlane(static_cast<uint32_t>(s.ai), lane))};
}

// block-wide merge; the result is valid in every thread
template <int NT>
__device__ Stat block_reduce(Stat s, Stat *sh) {
  s = combine(s, dpp_stat<kDppXor1>(s));
  s = combine(s, dpp_stat<kDppXor2>(s));
  s = combine(s, dpp_stat<kDppHalfMirror>(s));
  s = combine(s, dpp_stat<kDppMirror>(s));
  s = combine(combine(lane_stat(s, 0), lane_stat(s, 16)), combine(lane_stat(s, 32), lane_stat(s, 48)));
  __syncthreads();  // sh may still be read by a previous reduction
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  Stat r = sh[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) r = combine(r, sh[w]);
  return r;
}

template <int VEC>
__global__ __launch_bounds__(kThreads) void accept_rowpass(const float *__restrict__ logits, int T,
                                                           int V, int n_internal,
                                                           const int32_t *__restrict__ internal,
                                                           int nchunks, float inv_tau, int greedy,
                                                           Part *__restrict__ part, LeafSlot *__restrict__ leaf) {
  __shared__ Stat sh[kThreads / 64];
  const int chunk = blockIdx.x, slot = blockIdx.y, b = blockIdx.z;
  if (leaf && chunk == 0 && slot == 0 && threadIdx.x == 0) leaf[b] = LeafSlot{0ull, 0u, 0u};
  const int row = internal[slot];
  const float *z = logits + ((size_t)b * T + row) * V;
  const int base = chunk * kThreads * VEC * 4;
  // argmax as the values arrive: a thread visits its indices in increasing
  // order, so only a strictly larger value moves it (the first maximum stays)
  Stat st = empty_stat();
  float val[VEC][4];
  auto note = [&](int u) {
    const int i0 = base + (u * kThreads + threadIdx.x) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (val[u][j] > st.av || (u == 0 && j == 0)) {
        st.av = val[u][j];
        st.ai = i0 + j;
      }
  };
  if ((V % 4) == 0 && base + kThreads * VEC * 4 <= V) {   // a whole chunk: unconditional loads
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
      const f32x4_t f = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4_t *>(z + base + (u * kThreads + threadIdx.x) * 4));
#pragma unroll
      for (int j = 0; j < 4; ++j) val[u][j] = f[j];
      note(u);
    }
  } else {  // the row's tail chunk: element loads at clamped indices, -inf past the end
#pragma unroll
    for (int u = 0; u < VEC; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = base + (u * kThreads + threadIdx.x) * 4 + j;
        const float x = z[min(i, V - 1)];
        val[u][j] = i < V ? x : -INFINITY;
      }
      note(u);
    }
  }
  if (!greedy && st.av != -INFINITY) {
    st.m = st.av * inv_tau;  // max of y (tau > 0 keeps the order)
    // in base 2: d2 = (y - m) log2(e); e = 2^d2; E accumulates e*d2 and is
    // brought back to natural units once (padding and -inf give e = 0, and
    // the clamp keeps 0 * d2 finite)
    const float c = inv_tau * kLog2e, m2 = st.m * kLog2e;
    float S = 0.f, E2 = 0.f;
#pragma unroll
    for (int u = 0; u < VEC; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float d2 = fmaf(val[u][j], c, -m2);
        const float e = __builtin_amdgcn_exp2f(d2);
        S += e;
        E2 = fmaf(e, fmaxf(d2, -1e30f), E2);
      }
    st.S = S;
    st.E = E2 * (1.0f / kLog2e);
  }
  st = block_reduce<kThreads>(st, sh);
  if (threadIdx.x == 0) {
    Part p;
    p.m = st.m;
    p.S = st.S;
    p.E = st.E;
    p.amax_val = st.av;
    p.amax_idx = st.ai;
    p.pad0 = p.pad1 = p.pad2 = 0;
    part[((size_t)b * n_internal + slot) * nchunks + chunk] = p;
  }
}

__global__ __launch_bounds__(kScanThreads) void accept_scan(
    const float *__restrict__ logits, const int32_t *__restrict__ tree_tok, int T, int W, int V,
    int depth_max, int n_internal, int nchunks, const int32_t *__restrict__ slot_of,
    const int32_t *__restrict__ parent, const int32_t *__restrict__ depth,
    const uint64_t *__restrict__ mask, float eps, float delta, float inv_tau, int greedy,
    const Part *__restrict__ part, int32_t *__restrict__ accept_len, int32_t *__restrict__ best_node,
    int32_t *__restrict__ next_tok, int32_t *__restrict__ accepted_tok, float *__restrict__ cand_p,
    float *__restrict__ row_thr, int nparts, LeafSlot *__restrict__ leaf) {
  __shared__ float s_m[MEDUSA_MAX_TREE], s_S[MEDUSA_MAX_TREE], s_thr[MEDUSA_MAX_TREE];
  __shared__ int s_amax[MEDUSA_MAX_TREE];
  __shared__ unsigned int s_dec[MEDUSA_MAX_TREE / 32];
  __shared__ unsigned int s_key[kScanThreads / 64];
  __shared__ Stat sh[kScanThreads / 64];
  // nparts blocks per sequence: each takes the same decisions (from the same
  // inputs, so they agree on the winner); part 0 writes the outputs, and a
  // leaf winner's row is shared out among all of them for its argmax
  const int b = blockIdx.x / nparts, part_id = blockIdx.x % nparts;
  const bool writer = part_id == 0;
  const int tid = threadIdx.x;
  for (int w = tid; w < MEDUSA_MAX_TREE / 32; w += kScanThreads) s_dec[w] = 0u;

  // 0. issue every load the decisions need now, so that their latency overlaps
  // the partial merges: each thread owns candidates tid and tid + 512 (T <=
  // 1024); the candidate's logit under its parent, its token and the first
  // word of its ancestor mask
  constexpr int kPer = MEDUSA_MAX_TREE / kScanThreads;
  int c_tok[kPer], c_par[kPer], c_slot[kPer], c_pslot[kPer], c_depth[kPer];
  float c_z[kPer];
  uint64_t c_mask0[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = tid + i * kScanThreads;
    c_tok[i] = -1;
    c_par[i] = 0;
    c_slot[i] = c_pslot[i] = -1;
    c_depth[i] = 0;
    c_z[i] = 0.f;
    c_mask0[i] = 0ull;
    if (c < T) {
      c_mask0[i] = mask[(size_t)c * W];
      c_slot[i] = slot_of[c];
      c_depth[i] = depth[c];
      if (c > 0) {
        c_par[i] = parent[c];
        c_tok[i] = tree_tok[(size_t)b * T + c];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = tid + i * kScanThreads;
    if (c > 0 && c < T) {
      c_pslot[i] = slot_of[c_par[i]];
      if (!greedy && c_tok[i] >= 0 && c_tok[i] < V) c_z[i] = logits[((size_t)b * T + c_par[i]) * V + c_tok[i]];
    }
  }

  // 1. per internal row: merge the chunk partials, then the threshold
  for (int sl = tid; sl < n_internal; sl += kScanThreads) {
    const Part *p = part + ((size_t)b * n_internal + sl) * nchunks;
    Stat acc = empty_stat();
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      Part q[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (c0 + u < nchunks) q[u] = p[c0 + u];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (c0 + u < nchunks) acc = combine(acc, Stat{q[u].m, q[u].S, q[u].E, q[u].amax_val, q[u].amax_idx});
    }
    const float H = greedy ? 0.f : logf(acc.S) - acc.E / acc.S;
    s_m[sl] = acc.m;
    s_S[sl] = acc.S;
    s_thr[sl] = fminf(eps, delta * expf(-H));
    s_amax[sl] = acc.ai;
  }
  __syncthreads();

  // 2. decisions: candidate c against its parent's row
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = tid + i * kScanThreads;
    if (c >= T) continue;
    const int sc = c_slot[i];
    if (row_thr && writer) row_thr[(size_t)b * T + c] = sc >= 0 ? s_thr[sc] : NAN;
    if (c == 0) {
      if (cand_p && writer) cand_p[(size_t)b * T] = NAN;
      continue;
    }
    const int sl = c_pslot[i];
    const int tok = c_tok[i];
    float p;
    bool dec;
    if (greedy) {
      // one-hot p at the argmax: H = 0, so the threshold is min(eps, delta)
      // and the argmax token is kept iff 1 > that threshold
      p = tok == s_amax[sl] ? 1.f : 0.f;
      dec = p > s_thr[sl];
    } else if (tok < 0 || tok >= V) {  // out-of-range id: never accepted
      p = 0.f;
      dec = false;
    } else {
      p = exp2f((c_z[i] * inv_tau - s_m[sl]) * kLog2e) / s_S[sl];
      dec = p > s_thr[sl];
    }
    if (cand_p && writer) cand_p[(size_t)b * T + c] = p;
    if (dec) atomicOr(&s_dec[c >> 5], 1u << (c & 31));
  }
  __syncthreads();

  // 3. accepted iff all ancestors but the root decided yes; deepest, then smallest index
  unsigned int key = 0u;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = tid + i * kScanThreads;
    if (c >= T) continue;
    bool acc = true;
    for (int w = 0; w < W; ++w) {
      uint64_t anc = w == 0 ? c_mask0[i] : mask[(size_t)c * W + w];
      if (w == 0) anc &= ~1ull;
      const uint64_t dec = (uint64_t)s_dec[2 * w] | ((uint64_t)s_dec[2 * w + 1] << 32);
      if (anc & ~dec) acc = false;
    }
    if (acc) {
      const unsigned int k = ((unsigned)c_depth[i] << 16) | (0xFFFFu - (unsigned)c);
      key = k > key ? k : key;
    }
  }
  key = wave_max_u32(key);
  if ((tid & 63) == 0) s_key[tid >> 6] = key;
  __syncthreads();
  key = s_key[0];
  for (int w = 1; w < kScanThreads / 64; ++w) key = s_key[w] > key ? s_key[w] : key;
  const int alen = (int)(key >> 16);
  const int best = (int)(0xFFFFu - (key & 0xFFFFu));

  if (tid == 0 && writer) {
    accept_len[b] = alen;
    best_node[b] = best;
    int32_t *at = accepted_tok + (size_t)b * (depth_max + 1);
    for (int d = alen + 1; d <= depth_max; ++d) at[d] = -1;
    int d = alen;
    for (int j = best; j != -1; j = parent[j]) at[d--] = tree_tok[(size_t)b * T + j];
  }
  // 4. next greedy token: argmax of the winner's row (already known for rows with children)
  const int sb = slot_of[best];
  if (sb >= 0) {
    if (tid == 0 && writer) next_tok[b] = s_amax[sb];
    return;
  }
  // the leaf's row, this block's share: float4 index range [q0, q1) (element
  // range when V is not a multiple of 4)
  const float *z = logits + ((size_t)b * T + best) * V;
  Stat st = empty_stat();
  if ((V % 4) == 0) {
    // up to a 32768-wide share in one round of loads (16 float4 per thread,
    // issued unconditionally at clamped indices; indices past it are skipped)
    const int V4 = V / 4, per = (V4 + nparts - 1) / nparts;
    const int q0 = min(V4, part_id * per), q1 = min(V4, q0 + per);
    for (int base = q0 + tid; base < q1; base += kScanThreads * kLeafBatch) {
      f32x4_t v[kLeafBatch];
#pragma unroll
      for (int u = 0; u < kLeafBatch; ++u)
        v[u] = *reinterpret_cast<const f32x4_t *>(z + 4 * min(base + u * kScanThreads, q1 - 1));
#pragma unroll
      for (int u = 0; u < kLeafBatch; ++u)
        if (base + u * kScanThreads < q1) {
#pragma unroll
          for (int j = 0; j < 4; ++j) arg_better(st.av, st.ai, v[u][j], 4 * (base + u * kScanThreads) + j);
        }
    }
  } else {
    const int per = (V + nparts - 1) / nparts;
    const int e0 = min(V, part_id * per), e1 = min(V, e0 + per);
    for (int i = e0 + tid; i < e1; i += kScanThreads) arg_better(st.av, st.ai, z[i], i);
  }
  st = block_reduce<kScanThreads>(st, sh);
  if (tid != 0) return;
  if (nparts == 1) {
    next_tok[b] = st.ai;
    return;
  }
  // fold this share's argmax into the sequence's key; the count is an
  // acquire-release step, so the last block to count sees every block's fold
  __hip_atomic_fetch_max(&leaf[b].key, argmax_order_key(st.av, st.ai), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  const unsigned int seen = __hip_atomic_fetch_add(&leaf[b].cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  if (seen == (unsigned int)nparts - 1u) {
    const unsigned long long k = __hip_atomic_load(&leaf[b].key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    next_tok[b] = (int32_t)(~(uint32_t)k);
  }
}

inline int chunks_for(int V) { return (V + kThreads * kVec * 4 - 1) / (kThreads * kVec * 4); }

}  // namespace

// Scratch of typical_accept_noalloc: the row pass's chunk partials, then the
// scan's leaf slots (two to a partial), in device memory the library owns for
// the life of the process (one copy per GPU).  131072 partials of 32 bytes =
// 4 MiB: B * internal nodes * ceil(V / 4096) + ceil(B / 2) must not exceed
// that (the 341-node dense tree at batch 32 and V = 32000 needs 21776).  Host
// code never uses this name as an address: it looks the device address up
// once per device (scratch_on_device below).
constexpr size_t kScratchParts = 131072;
static __device__ __align__(256) Part scratch[kScratchParts];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
Part *g_scratch_ptr[kScratchDevices] = {};

// The current device's copy of `scratch` (hipGetSymbolAddress on the first
// call on each device, with that device current).
medusa_status scratch_on_device(const char *who, Part **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices)
    return fail(MEDUSA_ERR_HIP, "%s: no usable HIP device", who);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MEDUSA_ERR_HIP, "%s: device address of the scratch array: %s", who, hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<Part *>(p);
  }
  *out = g_scratch_ptr[dev];
  return MEDUSA_OK;
}

}  // namespace

// the row pass's chunk partials, then one LeafSlot per sequence
inline size_t partials_for(const medusa_tree *t, int B, int V) {
  return (size_t)B * (t->n_internal > 0 ? t->n_internal : 1) * chunks_for(V);
}
inline size_t workspace_bytes(const medusa_tree *t, int B, int V) {
  return partials_for(t, B, V) * sizeof(Part) + (size_t)B * sizeof(LeafSlot);
}

extern "C" size_t typical_accept_workspace(const medusa_tree *t, int B, int V) {
  if (!t || B < 1 || V < 1) return 0;
  return workspace_bytes(t, B, V);
}

namespace {

// The checks and launches shared by typical_accept and typical_accept_noalloc;
// `part` holds the row pass's chunk partials (B * n_internal * nchunks).
medusa_status typical_accept_impl(const char *who, medusa_stream_t stream, const medusa_tree *t, int B, int V,
                                  const float *logits, const int32_t *tree_tok, float eps, float delta,
                                  float temperature, int32_t *accept_len, int32_t *best_node, int32_t *next_tok,
                                  int32_t *accepted_tok, float *cand_p, float *row_thr, Part *part) {
  hipStream_t st = as_stream(stream);
  if (validate_enabled()) {  // NaN / +inf logits; tree tokens outside [0, V)
    ValidateSpec v;
    v.a = logits;
    v.na = (size_t)B * t->T * V;
    v.posinf_bad = true;
    v.tok = tree_tok;
    v.nt = (size_t)B * t->T;
    v.V = V;
    medusa_status s = validate_inputs(st, who, v);
    if (s != MEDUSA_OK) return s;
  }
  const int nchunks = chunks_for(V);
  const int greedy = temperature == 0.f;
  const float inv_tau = greedy ? 1.f : 1.f / temperature;
  // scan blocks per sequence: a leaf winner's row is read by all of them
  // (one CU pulls a 128 KB row in about 5 us; eight shares take about 1 us);
  // with no row pass (a root-only tree) nothing zeroes the leaf slots, and
  // one block reads the row
  const int nparts = t->n_internal > 0 ? std::max(1, std::min(kLeafParts, (V + 4095) / 4096)) : 1;
  LeafSlot *leaf = nparts > 1 ? reinterpret_cast<LeafSlot *>(part + partials_for(t, B, V)) : nullptr;
  if (t->n_internal > 0) {
    MEDUSA_LAUNCH(who, (accept_rowpass<kVec>), dim3(nchunks, t->n_internal, B), dim3(kThreads), 0, st,
                  logits, t->T, V, t->n_internal, t->d_internal, nchunks, inv_tau, greedy, part, leaf);
    medusa_status s = check_launch(who);
    if (s != MEDUSA_OK) return s;
  }
  MEDUSA_LAUNCH(who, accept_scan, dim3(B * nparts), dim3(kScanThreads), 0, st, logits, tree_tok, t->T, t->W, V,
                t->depth_max, t->n_internal, nchunks, t->d_slot, t->d_parent, t->d_depth, t->d_mask,
                eps, delta, inv_tau, greedy, part, accept_len, best_node, next_tok, accepted_tok,
                cand_p, row_thr, nparts, leaf);
  return check_launch(who);
}

// Arguments common to both entry points (everything but the workspace).
medusa_status typical_accept_args(const char *who, const medusa_tree *t, int B, int V, const float *logits,
                                  const int32_t *tree_tok, float eps, float delta, float temperature,
                                  const int32_t *accept_len, const int32_t *best_node, const int32_t *next_tok,
                                  const int32_t *accepted_tok) {
  medusa_status s = check_tree_on_device(t);
  if (s != MEDUSA_OK) return s;
  if (B < 1 || V < 1) return fail(MEDUSA_ERR_ARG, "%s: B=%d V=%d", who, B, V);
  if (!(eps >= 0.f) || !(delta >= 0.f) || !(temperature >= 0.f) || !isfinite(temperature))
    return fail(MEDUSA_ERR_ARG, "%s: eps, delta, temperature must be >= 0 (and finite temperature)", who);
  if (!logits || !tree_tok || !accept_len || !best_node || !next_tok || !accepted_tok)
    return fail(MEDUSA_ERR_ARG, "%s: NULL pointer", who);
  if (!aligned16(logits)) return fail(MEDUSA_ERR_ARG, "%s: logits must be 16-byte aligned", who);
  if (B > 65535) return fail(MEDUSA_ERR_UNSUPPORTED, "%s: B=%d > 65535", who, B);
  return MEDUSA_OK;
}

}  // namespace

extern "C" medusa_status typical_accept(medusa_stream_t stream, const medusa_tree *t, int B, int V,
                                        const float *logits, const int32_t *tree_tok, float eps,
                                        float delta, float temperature, int32_t *accept_len,
                                        int32_t *best_node, int32_t *next_tok, int32_t *accepted_tok,
                                        float *cand_p, float *row_thr, void *ws, size_t ws_bytes) {
  TraceRange tr("typical_accept");
  medusa_status s = typical_accept_args("typical_accept", t, B, V, logits, tree_tok, eps, delta, temperature,
                                        accept_len, best_node, next_tok, accepted_tok);
  if (s != MEDUSA_OK) return s;
  if (!ws) return fail(MEDUSA_ERR_ARG, "typical_accept: NULL workspace");
  if (!aligned16(ws)) return fail(MEDUSA_ERR_ARG, "typical_accept: ws must be 16-byte aligned");
  const size_t need = typical_accept_workspace(t, B, V);
  if (ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "typical_accept: workspace %zu < %zu", ws_bytes, need);
  return typical_accept_impl("typical_accept", stream, t, B, V, logits, tree_tok, eps, delta, temperature,
                             accept_len, best_node, next_tok, accepted_tok, cand_p, row_thr, static_cast<Part *>(ws));
}

extern "C" medusa_status typical_accept_noalloc(medusa_stream_t stream, const medusa_tree *t, int B, int V,
                                                const float *logits, const int32_t *tree_tok, float eps,
                                                float delta, float temperature, int32_t *accept_len,
                                                int32_t *best_node, int32_t *next_tok, int32_t *accepted_tok,
                                                float *cand_p, float *row_thr) {
  TraceRange tr("typical_accept_noalloc");
  const char *who = "typical_accept_noalloc";
  medusa_status s = typical_accept_args(who, t, B, V, logits, tree_tok, eps, delta, temperature, accept_len,
                                        best_node, next_tok, accepted_tok);
  if (s != MEDUSA_OK) return s;
  // partials, then the leaf slots (two to a Part)
  const size_t need = partials_for(t, B, V) + ((size_t)B + 1) / 2;
  if (need > kScratchParts)
    return fail(MEDUSA_ERR_UNSUPPORTED,
                "%s: B * internal nodes * ceil(V/4096) + B/2 = %zu partials exceed the %zu of the library's scratch",
                who, need, kScratchParts);
  Part *part = nullptr;
  s = scratch_on_device(who, &part);
  if (s != MEDUSA_OK) return s;
  // every partial and leaf slot the scan reads is written by the row pass of
  // the same call, so nothing needs clearing
  return typical_accept_impl(who, stream, t, B, V, logits, tree_tok, eps, delta, temperature, accept_len,
                             best_node, next_tok, accepted_tok, cand_p, row_thr, part);
}
