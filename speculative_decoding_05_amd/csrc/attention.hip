// Tree attention: every tree node attends to the prefix KV cache and to the
// tree tokens on its own branch.
//
// bf16 path (one block = one sequence b, one head h, 64 tree queries -- 128
// when the tree has more than 64 tokens -- and one slice of the prefix).  The block streams its keys in tiles of 64: each tile
// of K and V is read from HBM once with 16-byte coalesced loads (the next
// tile is prefetched into registers while the current one is consumed) and
// staged in LDS, where all 4 waves (16 queries each) use it.  Scores are
// computed transposed, S^T = K Q^T, on v_mfma_f32_16x16x32_bf16 so that every
// lane ends up owning one query and 16 keys of the tile: the online-softmax
// row statistics need only two cross-lane steps, and the probabilities are
// already in the B-operand layout of the O^T = V^T P^T product.  The V^T
// A-operand comes straight from the row-major V tile through the LDS
// transpose read (ds_read_b64_tr_b16): within each 16-lane group lane i
// receives element (i & 3) of the 8-byte value addressed by lane 4e + (i >> 2),
// so lanes that address keys k..k+3 at columns d..d+15 in groups of four
// deliver V[k+e][d+i] to lane i.  The tree keys come last, as extra tiles of
// the last slice, where the ancestor bitmask of each query is applied in
// registers; full prefix tiles skip masking.  With more than one slice per
// (b, h) the blocks write unnormalised partials (O, m, l) and a second kernel
// merges them with log-sum-exp weights.
//
// Three kernels, chosen per call: this one (bf16 trees of up to 64 tokens and
// of more than 384; trees of 65..128 tokens when the (b, head) pairs
// outnumber the CUs); tree_attn_wide_bf16 further down (bf16, dh = 128,
// trees of 129..384 tokens, or of 65..128 at up to one (b, head) pair per CU:
// one block covers the whole tree, so the prefix is read once per (b, head));
// and tree_attn_f32 (fp32, any tree).
#include <math.h>

#include "common.h"

using namespace medusa;

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 64;        // queries per block
constexpr int kKT = 64;        // keys per tile
constexpr int kPadK = 8;       // row padding (bf16) of the K tile: 16 rows of a b128 read hit distinct banks
constexpr int kPadV = 16;      // row padding (bf16) of the V tile: 8 rows of a transpose read hit distinct banks
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMinKeysPerSplit = 256;
constexpr int kSplitTargetBlocks = 128;
constexpr int kMergeUnroll = 8;       // slices the merge loads in one round

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// 4 bf16 of V^T from the row-major V tile through the LDS transpose read
__device__ __forceinline__ uint2 read_tr(const uint16_t *p) {
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p);  // generic -> LDS address space
  return __builtin_bit_cast(uint2, r);
}

struct Split {
  int nsplit, per_split;  // keys of the prefix per slice (multiple of kKT)
  bool three_per_cu;      // the 168-register build that runs three blocks per CU
};

// Prefix slices per (b, head): measured on MI355X, split partials plus the
// merge cost more than they gain once there are >= 128 (b, head, query-group)
// blocks, so the prefix is split only below that (down to 256 keys a slice).
// With 32 or fewer blocks before splitting (one sequence's heads) the split
// aims at one block per CU instead, down to 128 keys a slice (batch 1, 32
// heads, 1024 keys: 8 slices, kernel + merge 16.2 us against 17.4 with 4).
// Query tiles per wave: two once the tree has more than 64 tokens.
inline int qtiles_for(int T) { return T > kQB ? 2 : 1; }

// ns slices of whole key tiles covering L keys (fewer if the tiles run out)
inline Split split_into(int L, int ns) {
  if (ns < 1) ns = 1;
  int per = (L + ns - 1) / ns;
  per = (per + kKT - 1) / kKT * kKT;
  if (per == 0) per = kKT;
  ns = L > 0 ? (L + per - 1) / per : 1;
  return {ns, per, false};
}

inline Split choose_split(int B, int nh, int T, int L) {
  const int qb = kQB * qtiles_for(T);
  const long pairs = (long)B * nh * ((T + qb - 1) / qb);
  const long cus = device_compute_units();
  const bool few = pairs <= 32;
  int ns = (int)(((few ? cus : kSplitTargetBlocks) + pairs - 1) / pairs);
  // Between one and two (b, head) pairs per CU the CUs that get two set the
  // time.  With one query tile per wave the kernel also builds in 168
  // registers, which runs three blocks per CU: two slices then fill
  // 2 * pairs <= 768 block slots in one round, with half again the loads in
  // flight per CU (measured, 13B shape, 320 pairs, 4096 keys: 128.6 -> 119.3 us
  // with the merge; three slices at two blocks per CU before).  Elsewhere the
  // 168-register build is slower (batch 1: 16.2 -> 17.5 us).
  bool three = false;
  if (pairs > cus && pairs < 2 * cus) {
    three = qtiles_for(T) == 1;
    ns = three ? 2 : 3;
  }
  const int min_keys = few ? kMinKeysPerSplit / 2 : kMinKeysPerSplit;
  const int max_ns = L / min_keys > 1 ? L / min_keys : 1;
  if (ns > max_ns) ns = max_ns;
  if (ns > kMergeUnroll) ns = kMergeUnroll;
  Split sp = split_into(L, ns);
  sp.three_per_cu = three;
  return sp;
}

template <int DH>
struct TileRegs {
  static constexpr int kChunksPerRow = DH / 8;                     // 16-byte chunks
  static constexpr int kRowsPerPass = kThreads / kChunksPerRow;
  static constexpr int kPasses = kKT / kRowsPerPass;
  u32x4_t k[kPasses], v[kPasses];
};

// Load one tile of 64 keys (rows [r0, r0+64) of a segment) into registers;
// rows >= rend are zero.  Row i of the segment lives at base + i * row_stride.
template <int DH>
__device__ __forceinline__ void load_tile(TileRegs<DH> &t, const uint16_t *kbase,
                                          const uint16_t *vbase, long row_stride, int r0, int rend) {
  using TR = TileRegs<DH>;
  const int c = threadIdx.x % TR::kChunksPerRow;
#pragma unroll
  for (int p = 0; p < TR::kPasses; ++p) {
    const int row = r0 + p * TR::kRowsPerPass + threadIdx.x / TR::kChunksPerRow;
    if (row < rend) {
      const size_t off = (size_t)row * row_stride + c * 8;
      t.k[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(kbase + off));
      t.v[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(vbase + off));
    } else {
      t.k[p] = u32x4_t{0u, 0u, 0u, 0u};
      t.v[p] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
}

template <int DH>
__device__ __forceinline__ void store_tile(const TileRegs<DH> &t, uint16_t (*ks)[DH + kPadK],
                                           uint16_t (*vs)[DH + kPadV]) {
  using TR = TileRegs<DH>;
  const int c = threadIdx.x % TR::kChunksPerRow;
#pragma unroll
  for (int p = 0; p < TR::kPasses; ++p) {
    const int row = p * TR::kRowsPerPass + threadIdx.x / TR::kChunksPerRow;
    *reinterpret_cast<u32x4_t *>(&ks[row][c * 8]) = t.k[p];
    *reinterpret_cast<u32x4_t *>(&vs[row][c * 8]) = t.v[p];
  }
}

// One block: sequence b, head h, 64*QT tree queries (QT tiles of 16 per wave),
// one prefix slice.  With QT = 2 every K/V fragment read from LDS feeds two
// MFMAs and the two tiles' softmax and MFMA streams interleave.
// STAGES tiles are prefetched into registers ahead of the one being consumed.
template <int DH, int QT, int STAGES, int MINB>
__global__ __launch_bounds__(kThreads, MINB) void tree_attn_bf16(
    int B, int nh, int T, int W, int L, int Lstride, const int32_t *__restrict__ seq_len, float scale_log2,
    int qgroups, int nsplit, int per_split, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kt, const uint16_t *__restrict__ vt,
    const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc, const uint64_t *__restrict__ mask,
    const uint32_t *__restrict__ tile_need, uint16_t *__restrict__ out, float *__restrict__ ws_o,
    float2 *__restrict__ ws_ml) {
  constexpr int DS = DH / 32;  // 32-wide reduction steps over the head dim
  constexpr int DT = DH / 16;  // 16-wide output tiles over the head dim
  __shared__ __attribute__((aligned(16))) uint16_t ks[kKT][DH + kPadK];
  __shared__ __attribute__((aligned(16))) uint16_t vs[kKT][DH + kPadV];

  const int nblocks = gridDim.x;
  int lb = xcd_remap(blockIdx.x, nblocks);
  const int split = lb % nsplit;
  lb /= nsplit;
  const int qg = lb % qgroups;
  lb /= qgroups;
  const int h = lb % nh;
  const int b = lb / nh;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  int tq[QT];      // this lane's query (tree node) in each of its tiles
  bool qvalid[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    tq[qt] = qg * kQB * QT + (wave * QT + qt) * 16 + lr;
    qvalid[qt] = tq[qt] < T;
  }

  // Q^T as the B operand: lane holds q[tq][32s + 8lg .. +8]
  u32x4_t qreg[QT][DS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const uint16_t *qp = q + (((size_t)b * T + (qvalid[qt] ? tq[qt] : 0)) * nh + h) * DH + lg * 8;
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qreg[qt][s] = qvalid[qt] ? *reinterpret_cast<const u32x4_t *>(qp + s * 32) : u32x4_t{0u, 0u, 0u, 0u};
  }

  // key ranges: prefix slice [c0, c1) of this sequence's Lb cached keys, then
  // (last slice only) the tree tiles that hold an ancestor of some query of
  // the block, in order.  A wave skips the tree tiles none of its queries
  // needs, and all work of a tile when it has no valid query (it still takes
  // part in loading the tile).
  const int Lb = seq_len ? min(max(seq_len[b], 0), L) : L;
  const int c0 = split * per_split;
  const int c1 = min(Lb, c0 + per_split);
  const int ncache = c1 > c0 ? (c1 - c0 + kKT - 1) / kKT : 0;
  const bool last = split == nsplit - 1;
  // (with one query tile per wave the tree has at most 64 tokens: one tile,
  // needed by every wave, and nothing to skip)
  constexpr bool kSkip = QT > 1;
  const int ntree_all = (T + kKT - 1) / kKT;
  uint32_t need_block = ntree_all >= 32 ? ~0u : (1u << ntree_all) - 1u, need_wave = need_block;
  bool wave_live = true;
  if (kSkip) {
    need_block = need_wave = 0u;
    const int g0 = qg * 4 * QT, ngroups = (T + 15) / 16;
    for (int gq = g0; gq < g0 + 4 * QT && gq < ngroups; ++gq) {
      const uint32_t nb = tile_need[gq];
      need_block |= nb;
      if ((gq - g0) / QT == wave) need_wave |= nb;
    }
    wave_live = qg * kQB * QT + wave * QT * 16 < T;
  }
  const int ntree = last ? (kSkip ? __builtin_popcount(need_block) : ntree_all) : 0;
  const int ntiles = ncache + ntree;
  auto tree_tile = [&](int i) {  // i-th needed tree tile
    if (!kSkip) return i;
    uint32_t m = need_block;
    for (int j = 0; j < i; ++j) m &= m - 1;
    return __builtin_ctz(m);
  };

  const long cache_stride = DH;
  const long tree_stride = (long)nh * DH;
  const uint16_t *kc_bh = kc + ((size_t)b * nh + h) * Lstride * DH;
  const uint16_t *vc_bh = vc + ((size_t)b * nh + h) * Lstride * DH;
  const uint16_t *kt_bh = kt + ((size_t)b * T * nh + h) * DH;
  const uint16_t *vt_bh = vt + ((size_t)b * T * nh + h) * DH;

  f32x4_t oacc[QT][DT];
  float m_run[QT], l_lane[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int d = 0; d < DT; ++d) oacc[qt][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[qt] = -INFINITY;
    l_lane[qt] = 0.f;
  }

  // register stages: the next STAGES tiles are in flight while one is consumed
  TileRegs<DH> regs[STAGES];
  auto fetch = [&](TileRegs<DH> &r, int tile) {
    if (tile < ncache)
      load_tile<DH>(r, kc_bh, vc_bh, cache_stride, c0 + tile * kKT, c1);
    else
      load_tile<DH>(r, kt_bh, vt_bh, tree_stride, tree_tile(tile - ncache) * kKT, T);
  };
  auto consume = [&](int tile) {
    const bool is_tree = tile >= ncache;
    const int tt = is_tree ? tree_tile(tile - ncache) : 0;
    if (kSkip && (!wave_live || (is_tree && !((need_wave >> tt) & 1u)))) return;
    int kend;
    uint64_t mword[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) mword[qt] = ~0ull;
    if (is_tree) {
      kend = T - tt * kKT;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) mword[qt] = qvalid[qt] ? mask[(size_t)tq[qt] * W + tt] : 0ull;
    } else {
      kend = c1 - (c0 + tile * kKT);
    }
    const bool masked = is_tree || kend < kKT;

    // S^T for 4 sub-tiles of 16 keys: lane holds S[tq][key 16*st + 4*lg + v]
    f32x4_t sacc[QT][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) sacc[qt][st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t *>(&ks[st * 16 + lr][s * 32 + lg * 8]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) sacc[qt][st] = mfma(a, qreg[qt][s], sacc[qt][st]);
      }
    }

    // online softmax on raw scores; the scale is folded into one FMA before exp2
    u32x4_t pb[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (masked) {
            const int key = st * 16 + lg * 4 + v;
            const bool ok = key < kend && ((mword[qt] >> key) & 1ull);
            sacc[qt][st][v] = ok ? sacc[qt][st][v] : -INFINITY;
          }
          mx = fmaxf(mx, sacc[qt][st][v]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[qt], mx * scale_log2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_use);
      m_run[qt] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          sacc[qt][st][v] = __builtin_amdgcn_exp2f(fmaf(sacc[qt][st][v], scale_log2, -m_use));
          psum += sacc[qt][st][v];
        }
      l_lane[qt] = l_lane[qt] * alpha + psum;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int d = 0; d < DT; ++d) oacc[qt][d] *= alpha;
      }
      // P^T B operands: reduction slot 8*lg + e maps to key 32*hf + 4*lg + e
      // (e < 4) and 32*hf + 16 + 4*lg + (e - 4) (e >= 4)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        pb[qt][hf][0] = pack2(sacc[qt][2 * hf][0], sacc[qt][2 * hf][1]);
        pb[qt][hf][1] = pack2(sacc[qt][2 * hf][2], sacc[qt][2 * hf][3]);
        pb[qt][hf][2] = pack2(sacc[qt][2 * hf + 1][0], sacc[qt][2 * hf + 1][1]);
        pb[qt][hf][3] = pack2(sacc[qt][2 * hf + 1][2], sacc[qt][2 * hf + 1][3]);
      }
    }

    // O^T += V^T P^T; V^T fragments by transpose read: lane (lr, lg) names key
    // row base + lr/4 and columns 16*d + 4*(lr%4) .. +3
    const int trow = lg * 4 + (lr >> 2);
    const int tcol = (lr & 3) * 4;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        const uint2 lo = read_tr(&vs[hf * 32 + trow][d * 16 + tcol]);
        const uint2 hi = read_tr(&vs[hf * 32 + 16 + trow][d * 16 + tcol]);
        const u32x4_t a = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) oacc[qt][d] = mfma(a, pb[qt][hf], oacc[qt][d]);
      }
    }
  };
  // tile j waits in register stage j % STAGES; it is fetched STAGES tiles
  // before it is stored to LDS and consumed
#pragma unroll
  for (int r = 0; r < STAGES; ++r)
    if (r < ntiles) fetch(regs[r], r);
  for (int tile = 0; tile < ntiles; tile += STAGES) {
#pragma unroll
    for (int r = 0; r < STAGES; ++r) {
      const int tj = tile + r;
      if (tj < ntiles) {
        __syncthreads();  // previous tile fully consumed
        store_tile<DH>(regs[r], ks, vs);
        __syncthreads();
        if (tj + STAGES < ntiles) fetch(regs[r], tj + STAGES);
        consume(tj);
      }
    }
  }

#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float l_tot = l_lane[qt] + __shfl_xor(l_lane[qt], 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!qvalid[qt]) continue;
    // lane holds O[tq][16*d + 4*lg + v]
    if (nsplit == 1) {
      const float inv = 1.f / l_tot;
      uint16_t *op = out + (((size_t)b * T + tq[qt]) * nh + h) * DH + lg * 4;
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        uint2 w;
        w.x = pack2(oacc[qt][d][0] * inv, oacc[qt][d][1] * inv);
        w.y = pack2(oacc[qt][d][2] * inv, oacc[qt][d][3] * inv);
        *reinterpret_cast<uint2 *>(op + d * 16) = w;
      }
    } else {
      const size_t row = (((size_t)split * B + b) * nh + h) * T + tq[qt];
      float *op = ws_o + row * DH + lg * 4;
#pragma unroll
      for (int d = 0; d < DT; ++d)
        *reinterpret_cast<float4 *>(op + d * 16) =
            make_float4(oacc[qt][d][0], oacc[qt][d][1], oacc[qt][d][2], oacc[qt][d][3]);
      if (lg == 0) ws_ml[row] = make_float2(m_run[qt], l_tot);
    }
  }
}

// Merge the slices of one (b, h, node) row: weights 2^(m_s - M).  NS > 0:
// every slice's (m, l) and partial O are loaded in one round, NS loads each
// (slices past nsplit re-load the last one and are not summed); NS = 0: a loop
// over the slices.  The launcher passes NS = nsplit for 2-4 slices, so no load
// is wasted there, and 8 for 5-8.
template <int DH, int NS>
__global__ __launch_bounds__(256) void tree_attn_merge_bf16(int B, int nh, int T, int nsplit,
                                                            const float *__restrict__ ws_o,
                                                            const float2 *__restrict__ ws_ml,
                                                            uint16_t *__restrict__ out) {
  constexpr int TPR = DH / 4;  // threads per row, 4 values each
  const int row = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 4;
  const long nrows = (long)B * nh * T;
  if (row >= nrows) return;
  const size_t stride = (size_t)nrows;
  float l = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (NS > 0) {
    float2 ml[NS > 0 ? NS : 1];
    float4 po[NS > 0 ? NS : 1];
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int sl = s < nsplit ? s : nsplit - 1;
      ml[s] = ws_ml[sl * stride + row];
      po[s] = *reinterpret_cast<const float4 *>(ws_o + (sl * stride + row) * DH + c);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (s < nsplit) M = fmaxf(M, ml[s].x);
    const float Mu = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (s < nsplit) {
        const float w = exp2f(ml[s].x - Mu);
        l += w * ml[s].y;
        o.x += w * po[s].x;
        o.y += w * po[s].y;
        o.z += w * po[s].z;
        o.w += w * po[s].w;
      }
  } else {
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws_ml[s * stride + row].x);
    const float Mu = M == -INFINITY ? 0.f : M;
    for (int s = 0; s < nsplit; ++s) {
      const float2 ml = ws_ml[s * stride + row];
      const float w = exp2f(ml.x - Mu);
      l += w * ml.y;
      const float4 p = *reinterpret_cast<const float4 *>(ws_o + (s * stride + row) * DH + c);
      o.x += w * p.x;
      o.y += w * p.y;
      o.z += w * p.z;
      o.w += w * p.w;
    }
  }
  const float inv = 1.f / l;
  // row = (b*nh + h)*T + t  ->  out[b][t][h][:]
  const int t = row % T;
  const int bh = row / T;
  const int h = bh % nh, b = bh / nh;
  uint2 w;
  w.x = pack2(o.x * inv, o.y * inv);
  w.y = pack2(o.z * inv, o.w * inv);
  *reinterpret_cast<uint2 *>(out + (((size_t)b * T + t) * nh + h) * DH + c) = w;
}

// fp32 path: block = (b, h, 32 queries); keys = lanes.  The block's 4 waves
// are QW query waves (8 queries each, as many as the group's queries need) x
// KW key splits (KW = 4 / QW): wave (qw, kw) takes tiles kw, kw + KW, ... of
// the keys for its 8 queries, so a small tree (8 queries or fewer) spreads its
// tiles over all four waves.  Each wave stages its own V tile in its own LDS
// region (global_load_lds_dwordx4: the rows land in order, no staging
// registers) and needs no block barrier inside the loop.  Per 64-key tile
// each lane holds its own key's K row in registers and scores the wave's 8
// queries against it (Q rows read from LDS as broadcast float4s); the 8 rows
// of probabilities go to a per-wave LDS block laid out key-major, so the PV
// sum reads each V value once for all 8 queries and their 8 probabilities as
// two broadcast float4s.  Row statistics by DPP row steps and readlane.  At
// the end the KW partial (max, sum, O) of each query are merged through LDS.
constexpr int kF32Q = 32;

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dppf<kDppXor1>(v));
  v = fmaxf(v, dppf<kDppXor2>(v));
  v = fmaxf(v, dppf<kDppHalfMirror>(v));
  v = fmaxf(v, dppf<kDppMirror>(v));
  return fmaxf(fmaxf(readlanef(v, 0), readlanef(v, 16)), fmaxf(readlanef(v, 32), readlanef(v, 48)));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dppf<kDppXor1>(v);
  v += dppf<kDppXor2>(v);
  v += dppf<kDppHalfMirror>(v);
  v += dppf<kDppMirror>(v);
  return (readlanef(v, 0) + readlanef(v, 16)) + (readlanef(v, 32) + readlanef(v, 48));
}

// LDS of the fp32 kernel, in floats: per-wave V tiles, the Q rows of the
// group, per-wave probability blocks; the merge area reuses the V tiles
template <int DH>
struct F32Lds {
  static constexpr int kV = 0, kVWave = kKT * DH;
  static constexpr int kQ = 4 * kVWave;
  static constexpr int kP = kQ + kF32Q * DH;
  static constexpr int kTotal = kP + 4 * kKT * 8;
  static_assert(4 * 8 * (DH + 2) <= 4 * kVWave, "merge area");
  static_assert(kTotal * 4 <= 160 * 1024, "LDS");
};

template <int DH>
__global__ __launch_bounds__(256, 1) void tree_attn_f32(int B, int nh, int T, int W, int L, int Lstride,
                                                     const int32_t *__restrict__ seq_len, float scale,
                                                     int qgroups, const float *__restrict__ q,
                                                     const float *__restrict__ kt,
                                                     const float *__restrict__ vt,
                                                     const float *__restrict__ kc,
                                                     const float *__restrict__ vc,
                                                     const uint64_t *__restrict__ mask,
                                                     float *__restrict__ out) {
  using LY = F32Lds<DH>;
  constexpr int DPL = DH / 64;            // output dims per lane
  constexpr int D4 = DH / 4;
  constexpr int RPI = 64 / (DH / 4);      // V rows per 1 KiB wave load (16 bytes per lane)
  __shared__ __attribute__((aligned(16))) float lds[LY::kTotal];
  const int qg = blockIdx.x % qgroups;
  const int h = (blockIdx.x / qgroups) % nh;
  const int b = blockIdx.x / (qgroups * nh);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int Tq = min(kF32Q, T - qg * kF32Q);      // queries of this group
  const int QW = (Tq + 7) / 8, KW = 4 / QW;       // query waves x key splits
  const int qw = wave % QW, kw = wave / QW;
  const bool busy = kw < KW;
  float *qs = lds + LY::kQ;
  float *vs = lds + LY::kV + wave * LY::kVWave;
  float *pw = lds + LY::kP + wave * kKT * 8;
  for (int e = threadIdx.x; e < kF32Q * DH; e += 256) {
    const int qi = e / DH, d = e % DH, t = qg * kF32Q + qi;
    qs[e] = t < T ? q[(((size_t)b * T + t) * nh + h) * DH + d] : 0.f;
  }
  __syncthreads();
  float m[8], l[8], o[8][DPL];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    m[u] = -INFINITY;
    l[u] = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[u][j] = 0.f;
  }
  const int Lb = seq_len ? min(max(seq_len[b], 0), L) : L;
  const int ncache = (Lb + kKT - 1) / kKT;
  const int ntiles = ncache + (T + kKT - 1) / kKT;
  const int q0 = qg * kF32Q + qw * 8;   // the wave's first query
  for (int tile = busy ? kw : ntiles; tile < ntiles; tile += KW) {
    const bool is_tree = tile >= ncache;
    const int r0 = is_tree ? (tile - ncache) * kKT : tile * kKT;
    const int rend = is_tree ? T : Lb;
    const int key = r0 + lane;
    // the V tile straight into this wave's region (rows past the end: a valid
    // row, weighted 0), this lane's K row, the mask words of the 8 queries
    const float *vbase = is_tree ? vt + ((size_t)b * T * nh + h) * DH : vc + ((size_t)b * nh + h) * Lstride * DH;
    const long vstride = is_tree ? (long)nh * DH : (long)DH;
#pragma unroll
    for (int j = 0; j < kKT / RPI; ++j) {
      const int row = min(r0 + RPI * j + lane / (DH / 4), rend - 1);
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1))) *)(vbase + row * vstride + (lane % (DH / 4)) * 4),
          (void __attribute__((address_space(3))) *)(vs + j * RPI * DH), 16, 0, 0);
    }
    const int krow = min(key, rend - 1);
    const float *kp = is_tree ? kt + (((size_t)b * T + krow) * nh + h) * DH
                              : kc + (((size_t)b * nh + h) * Lstride + krow) * DH;
    float4 kr[D4];
#pragma unroll
    for (int i = 0; i < D4; ++i) kr[i] = *reinterpret_cast<const float4 *>(kp + 4 * i);
    uint64_t mw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) mw[u] = is_tree && q0 + u < T ? mask[(size_t)(q0 + u) * W + (tile - ncache)] : 0ull;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the V tile is in LDS
    // scores of the wave's 8 queries against this lane's key; online softmax
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < D4; ++i) {
        const float4 qv = *reinterpret_cast<const float4 *>(&qs[(qw * 8 + u) * DH + 4 * i]);
        s4[i & 3] += qv.x * kr[i].x + qv.y * kr[i].y + qv.z * kr[i].z + qv.w * kr[i].w;
      }
      bool ok = key < rend;
      if (is_tree) ok = ok && ((mw[u] >> lane) & 1ull);
      x[u] = ok ? ((s4[0] + s4[1]) + (s4[2] + s4[3])) * scale : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float m_new = fmaxf(m[u], wave_max_f32(x[u]));
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = expf(m[u] - m_use);
      const float p = expf(x[u] - m_use);
      l[u] = l[u] * alpha + wave_sum_f32(p);
      m[u] = m_new;
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[u][j] *= alpha;
      pw[lane * 8 + u] = p;  // the same wave reads it back below: LDS keeps the order
    }
    // O += P V: each V value once, the 8 probabilities of its key as two float4s
#pragma unroll 4
    for (int jk = 0; jk < kKT; ++jk) {
      const float4 pa = *reinterpret_cast<const float4 *>(&pw[jk * 8]);
      const float4 pb = *reinterpret_cast<const float4 *>(&pw[jk * 8 + 4]);
      const float pu[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const float v = vs[jk * DH + lane + 64 * j];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u][j] += pu[u] * v;
      }
    }
  }
  // merge the KW partials of each query: waves kw > 0 leave theirs in LDS
  // (over the V tiles), the kw = 0 wave of each query wave combines
  __syncthreads();
  float *mo = lds + LY::kV;
  if (busy && kw > 0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float *row = mo + (wave * 8 + u) * (DH + 2);
#pragma unroll
      for (int j = 0; j < DPL; ++j) row[lane + 64 * j] = o[u][j];
      if (lane == 0) {
        row[DH] = m[u];
        row[DH + 1] = l[u];
      }
    }
  }
  __syncthreads();
  if (!busy || kw > 0) return;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int t = q0 + u;
    if (t >= T) continue;
    float M = m[u];
    for (int k = 1; k < KW; ++k) M = fmaxf(M, mo[((qw + k * QW) * 8 + u) * (DH + 2) + DH]);
    const float w0 = expf(m[u] - M);
    float lt = l[u] * w0, ot[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) ot[j] = o[u][j] * w0;
    for (int k = 1; k < KW; ++k) {
      const float *row = mo + ((qw + k * QW) * 8 + u) * (DH + 2);
      const float wk = row[DH] == -INFINITY ? 0.f : expf(row[DH] - M);
      lt += row[DH + 1] * wk;
#pragma unroll
      for (int j = 0; j < DPL; ++j) ot[j] += row[lane + 64 * j] * wk;
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) out[(((size_t)b * T + t) * nh + h) * DH + lane + 64 * j] = ot[j] / lt;
  }
}


// ---------------------------------------------------------------------------
// Wide tree attention (bf16, dh = 128, 64 < T <= 384): one block per (b, head,
// prefix slice) with NW waves of 32 queries that together cover every tree
// node, so each prefix key is read from HBM once per (b, head) and staged once
// in LDS for all of them.  Scores are computed transposed on
// v_mfma_f32_32x32x16_bf16 (each lane owns one query and 16 of every 32 keys;
// the other 16 sit in lane ^ 32, one permlane32 swap away), and O^T += V^T P^T
// takes V^T straight from the row-major tile through the LDS transpose read.
// K/V tiles of 64 keys go from global memory straight into LDS
// (global_load_lds_dwordx4: lane i's 16 bytes land at the wave's base + 16 i)
// in three stages, the loads of tile t+2 issued while tile t is worked on, one
// barrier per tile.  The 16-byte chunks of each 256-byte row are XOR-swizzled
// (K: chunk ^ (row & 15), V: chunk ^ 4 (row & 3)) so that the 16 rows of a
// b128 K read hit distinct banks, and so do the two 16-lane groups of a
// half-wave transpose read (4 rows x 32 bytes each, the same 4 rows, their
// 32-byte column blocks 64 bytes apart); the loads apply the swizzle on the
// global side (lane i of a
// load fills physical chunk i % 16 and fetches the logical chunk that maps
// there), and a fragment's address is the lane's base XOR the step's offset.
// The tree mask rows of the block's nodes are copied to LDS once.  The
// softmax keeps a per-query reference maximum and re-references it (and
// rescales O) only when a score exceeds it by more than 2^8, so the common
// path per score is a third of a max3, one FMA, one exp2 and one add.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWideQ = 32;                 // queries per wave
constexpr int kWideStageVec = 2048;        // one stage: K (1024) then V (1024) 16-byte chunks, 64 keys x 128 dh each
constexpr int kWideMaskMax = 384 * 6;      // mask words of a 384-node tree
constexpr float kLazyRescale = 8.f;        // log2 headroom before the reference maximum moves

__shared__ u32x4_t wide_stage0[kWideStageVec];
__shared__ u32x4_t wide_stage1[kWideStageVec];
__shared__ u32x4_t wide_stage2[kWideStageVec];
__shared__ uint64_t wide_mask[kWideMaskMax];

template <int S>
__device__ __forceinline__ u32x4_t *wide_stage() {
  if (S == 0) return wide_stage0;
  if (S == 1) return wide_stage1;
  return wide_stage2;
}

// s_waitcnt with vmcnt = vm and lgkmcnt = lgkm (gfx9 encoding; expcnt left at its maximum)
#define ATT_WAITCNT(vm, lgkm) \
  __builtin_amdgcn_s_waitcnt(((vm) & 0xF) | ((((vm) >> 4) & 3) << 14) | (7 << 4) | (((lgkm) & 0xF) << 8))

__device__ __forceinline__ void lds_dma16(const uint16_t *g, u32x4_t *l) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)g,
                                   (void __attribute__((address_space(3))) *)l, 16, 0, 0);
}

__device__ __forceinline__ void wide_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// max of x over lanes l and l ^ 32 (in every lane), without LDS: permlane32
// swap exchanges the two 32-lane halves between its two results, so together
// with x they cover x[l] and x[l ^ 32]
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return fmaxf(x, fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])));
}

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void tree_attn_wide_bf16(
    int B, int nh, int T, int W, int L, int Lstride, const int32_t *__restrict__ seq_len, float scale_log2,
    int nsplit, int per_split, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kt,
    const uint16_t *__restrict__ vt, const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
    const uint64_t *__restrict__ mask, const uint32_t *__restrict__ tile_need, uint16_t *__restrict__ out,
    float *__restrict__ ws_o, float2 *__restrict__ ws_ml) {
  constexpr int DH = 128;
  constexpr int KS = DH / 16;          // 16-deep steps of the score product
  constexpr int DT = DH / 32;          // 32-wide output tiles
  constexpr int LW = NW < 8 ? NW : 8;  // waves that issue the tile loads
  constexpr int IPW = 16 / LW;         // 1 KiB K loads (and as many V loads) per loader wave per tile
  // the two 32-key halves of a tile unrolled where registers allow (two waves
  // per SIMD or fewer: 256 registers; with three, 168 do not hold both)
  constexpr int kHalves = NW <= 8 ? 2 : 1;
  const int split = blockIdx.x % nsplit;
  const int bh = blockIdx.x / nsplit;
  const int h = bh % nh, b = bh / nh;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: LDS bases stay scalar
  const int lane = threadIdx.x & 63;
  const int lq = lane & 31, hh = lane >> 5;
  const int tq = wave * kWideQ + lq;  // this lane's query (tree node)
  const bool qvalid = tq < T;
  const bool wave_live = wave * kWideQ < T;

  // Q^T as the B operand of step k: q[tq][16k + 8hh .. +8]
  u32x4_t qreg[KS];
  {
    const uint16_t *qp = q + (((size_t)b * T + (qvalid ? tq : 0)) * nh + h) * DH + hh * 8;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      qreg[k] = qvalid ? *reinterpret_cast<const u32x4_t *>(qp + k * 16) : u32x4_t{0u, 0u, 0u, 0u};
  }
  // the tree's mask rows, visible to all waves after the first barrier below
  for (int i = threadIdx.x; i < T * W; i += 64 * NW) wide_mask[i] = mask[i];
  ATT_WAITCNT(0, 15);  // nothing but the tile loads is outstanding from here on

  // keys: prefix slice [c0, c1) of this sequence's Lb cached keys, then (last
  // slice) the tree tiles that hold an ancestor of some node; a wave skips
  // the tree tiles none of its 32 nodes needs
  const int Lb = seq_len ? min(max(seq_len[b], 0), L) : L;
  const int c0 = split * per_split;
  const int c1 = min(Lb, c0 + per_split);
  const int ncache = c1 > c0 ? (c1 - c0 + kKT - 1) / kKT : 0;
  uint32_t need_block = 0u, need_wave = 0u;
  const int ngroups = (T + 15) / 16;
  for (int g = 0; g < ngroups; ++g) {
    const uint32_t nb = tile_need[g];
    need_block |= nb;
    if ((g >> 1) == wave) need_wave |= nb;
  }
  const int ntree = split == nsplit - 1 ? __builtin_popcount(need_block) : 0;
  const int ntiles = ncache + ntree;
  auto tree_tile = [&](int i) __attribute__((always_inline)) {  // i-th needed tree tile
    uint32_t m = need_block;
    for (int j = 0; j < i; ++j) m &= m - 1;
    return __builtin_ctz(m);
  };

  const uint16_t *kc_bh = kc + ((size_t)b * nh + h) * Lstride * DH;
  const uint16_t *vc_bh = vc + ((size_t)b * nh + h) * Lstride * DH;
  const uint16_t *kt_b = kt + ((size_t)b * T * nh + h) * DH;
  const uint16_t *vt_b = vt + ((size_t)b * T * nh + h) * DH;

  // load `ins` (< 16) of a loader wave fills K rows 4 ins .. 4 ins + 3 (V the
  // same, 16 KiB further on); lane i fills physical chunk i % 16 of row
  // 4 ins + i / 16 and fetches the logical chunk stored there
  auto issue = [&](int tile, u32x4_t *stg) __attribute__((always_inline)) {
    if (wave >= LW) return;
    const bool is_tree = tile >= ncache;
    const int r0 = is_tree ? tree_tile(tile - ncache) * kKT : c0 + tile * kKT;
    const int rend = is_tree ? T : c1;
    const long stride = is_tree ? (long)nh * DH : (long)DH;
    const uint16_t *kb = is_tree ? kt_b : kc_bh;
    const uint16_t *vb = is_tree ? vt_b : vc_bh;
    const int cv = (lane & 15) ^ ((lane >> 4) << 2);  // row & 3 == lane / 16
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int ins = IPW * wave + j;
      const int r = 4 * ins + (lane >> 4);
      const int row = min(r0 + r, rend - 1);  // past the end: a valid row whose scores are masked
      const int ck = (lane & 15) ^ (r & 15);
      lds_dma16(kb + row * stride + ck * 8, stg + ins * 64);
      lds_dma16(vb + row * stride + cv * 8, stg + 1024 + ins * 64);
    }
  };

  f32x16_t oacc[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
  float m_ref = -INFINITY, l_lane = 0.f;
  // per-lane LDS byte addresses.  K fragment of step k: row 32 st + lq,
  // logical chunk 2k + hh, physical (2k + hh) ^ (lq & 15) = base ^ 2k (the
  // step only flips bits 5-7 of the byte address).  V^T read by 16-lane group
  // g: rows 32 st + 16 ks + 4 (g >> 1) + (li >> 2) (+8), logical chunk
  // 4 d + 2 (g & 1) + (li & 3) / 2, physical that ^ 4 (li >> 2) = base ^ 4d
  // (over the 32 lanes of groups 2h, 2h+1 the physical chunks are 0..15 once
  // each: the half-wave read covers the 64 banks exactly).
  const int g = lane >> 4, li = lane & 15;
  const int kaddr = lq * 256 + ((hh ^ (lq & 1)) | (((lq & 15) >> 1) << 1)) * 16;
  const int vaddr = 16384 + (4 * (g >> 1) + (li >> 2)) * 256 +
                    ((2 * (g & 1) + ((li & 3) >> 1)) ^ ((li >> 2) << 2)) * 16 + (li & 1) * 8;

  auto consume = [&](int tile, const u32x4_t *stg) __attribute__((always_inline)) {
    if (!wave_live) return;
    const bool is_tree = tile >= ncache;
    const int tt = is_tree ? tree_tile(tile - ncache) : 0;
    if (is_tree && !((need_wave >> tt) & 1u)) return;
    const int kend = is_tree ? T - tt * kKT : c1 - (c0 + tile * kKT);
    const bool masked = is_tree || kend < kKT;
    const char *base = reinterpret_cast<const char *>(stg);
#pragma unroll kHalves
    for (int st = 0; st < 2; ++st) {  // 32-key halves of the tile
      // S^T: lane holds S[key 32 st + 8 j + 4 hh + i][tq] in s[4 j + i]
      f32x16_t s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
      const char *kp = base + st * 32 * 256;
#pragma unroll
      for (int k = 0; k < KS; ++k) s = mfma32(*reinterpret_cast<const u32x4_t *>(kp + (kaddr ^ (k << 5))), qreg[k], s);
      if (masked) {
        // visible keys of the tile as one word (a tree node's mask row has no
        // bit at or past T; a ragged prefix tile keeps its first kend keys),
        // then this lane's 16: bit 8 j + i is key 32 st + 8 j + 4 hh + i
        const uint64_t mw = is_tree ? (qvalid ? wide_mask[tq * W + tt] : 0ull)
                                    : (kend >= kKT ? ~0ull : (1ull << kend) - 1ull);
        const uint32_t mb = (static_cast<uint32_t>(mw >> (32 * st)) >> (4 * hh)) & 0x0F0F0F0Fu;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = ((mb >> (8 * (e >> 2) + (e & 3))) & 1u) ? s[e] : -INFINITY;
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, s[e]), s[e + 1]);
      mx = fmaxf(mx, s[15]);
      mx = xor32_max(mx);
      const float m_cand = mx * scale_log2;
      const bool move = m_cand > m_ref + kLazyRescale;
      if (__any(move)) {  // rare after the first keys: re-reference and rescale
        const float m_new = move ? m_cand : m_ref;
        const float alpha = m_new == m_ref ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
        for (int d = 0; d < DT; ++d) oacc[d] *= alpha;
        l_lane *= alpha;
        m_ref = m_new;
      }
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], scale_log2, -m_use));
        ps += s[e];
      }
      l_lane += ps;
      // P^T B operand of 16-key step ks: slot 8 hh + e is key 16 ks + 8 (e >> 2) + 4 hh + (e & 3),
      // i.e. this lane's own s[8 ks .. 8 ks + 7]
      u32x4_t pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pb[ks] = u32x4_t{pack2(s[8 * ks], s[8 * ks + 1]), pack2(s[8 * ks + 2], s[8 * ks + 3]),
                         pack2(s[8 * ks + 4], s[8 * ks + 5]), pack2(s[8 * ks + 6], s[8 * ks + 7])};
      // O^T += V^T P^T: lane i of group g receives V[row .. row + 3][column + i]
      const char *vp = base + st * 32 * 256;
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        const int va = vaddr ^ (64 * d);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint2 lo = read_tr(reinterpret_cast<const uint16_t *>(vp + va + 16 * ks * 256));
          const uint2 hi = read_tr(reinterpret_cast<const uint16_t *>(vp + va + (16 * ks + 8) * 256));
          oacc[d] = mfma32(u32x4_t{lo.x, lo.y, hi.x, hi.y}, pb[ks], oacc[d]);
        }
      }
    }
  };

  if (ntiles > 0) {
    // tile t lives in stage t % 3; its loads are issued two tiles ahead (past
    // the end the last tile is re-loaded into a stage nobody reads again)
    issue(0, wide_stage<0>());
    issue(min(1, ntiles - 1), wide_stage<1>());
    auto body = [&](int t, const u32x4_t *cur, u32x4_t *dst, bool issue_first) __attribute__((always_inline)) {
      ATT_WAITCNT(2 * IPW, 15);  // this wave's loads of tile t are in LDS (tile t+1's may still fly)
      wide_barrier();            // everyone's are, and everyone finished tile t-1 (the stage of t+2)
      if (issue_first) issue(min(t + 2, ntiles - 1), dst);
      consume(t, cur);
      if (!issue_first) issue(min(t + 2, ntiles - 1), dst);
    };
    // (the first body of each round issues after its compute: the compiler's
    // wait insertion cannot separate the stages at the loop head and would
    // otherwise wait for the loads it has just issued)
    for (int t = 0; t < ntiles; t += 3) {
      body(t, wide_stage<0>(), wide_stage<2>(), false);
      if (t + 1 < ntiles) body(t + 1, wide_stage<1>(), wide_stage<0>(), true);
      if (t + 2 < ntiles) body(t + 2, wide_stage<2>(), wide_stage<1>(), true);
    }
    ATT_WAITCNT(0, 15);  // the re-loads past the end land before the block's LDS is handed on
  }

  const float l_tot = l_lane + __shfl_xor(l_lane, 32);
  if (!qvalid) return;
  // lane holds O^T[32 d + 8 j + 4 hh + i][tq] in oacc[d][4 j + i]
  if (nsplit == 1) {
    const float inv = 1.f / l_tot;
    uint16_t *op = out + (((size_t)b * T + tq) * nh + h) * DH + 4 * hh;
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 w;
        w.x = pack2(oacc[d][4 * j] * inv, oacc[d][4 * j + 1] * inv);
        w.y = pack2(oacc[d][4 * j + 2] * inv, oacc[d][4 * j + 3] * inv);
        *reinterpret_cast<uint2 *>(op + 32 * d + 8 * j) = w;
      }
  } else {
    const size_t row = (((size_t)split * B + b) * nh + h) * T + tq;
    float *op = ws_o + row * DH + 4 * hh;
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4 *>(op + 32 * d + 8 * j) =
            make_float4(oacc[d][4 * j], oacc[d][4 * j + 1], oacc[d][4 * j + 2], oacc[d][4 * j + 3]);
    if (hh == 0) ws_ml[row] = make_float2(m_ref, l_tot);
  }
}

// The wide kernel serves dh = 128 trees of 129..384 tokens, and of 65..128
// tokens while the (b, head) pairs are at most one per CU; past that the
// 128-query kernel, two blocks per CU, is faster for the small trees
// (measured on MI355X, 128 nodes, KV 1024: wide 21.7 / 34.8 / 43.6 us at
// 32 / 128 / 256 pairs against 26.8 / 47.4 / 51.0, but 92.4 against 69.5 at
// 512 pairs, and 254.6 against 173.7 us at the 13B shape's 320 pairs with
// KV 4096).  (At batch 1 with the 64-node tree, two waves per block over 8
// prefix slices are slower than the 64-query kernel, 14.6 + 4.4 against
// 13.9 + 4.4 us.)
inline bool use_wide(medusa_dtype dt, int dh, int T, int B, int nh) {
  if (dt != MEDUSA_BF16 || dh != 128 || T <= kQB || T > 384) return false;
  return T > 2 * kQB || (long)B * nh <= device_compute_units();
}
inline int wide_waves(int T) { return T <= 128 ? 4 : T <= 256 ? 8 : 12; }

// One block per (b, head) already fills the chip from one block per CU; with
// fewer pairs the prefix is split (slices of at least 256 keys) until there
// are about as many blocks as CUs.
inline Split choose_split_wide(int B, int nh, int L) {
  const long pairs = (long)B * nh;
  const long cus = device_compute_units();
  int ns = pairs >= cus ? 1 : (int)((cus + pairs - 1) / pairs);
  const int max_ns = L / kMinKeysPerSplit > 1 ? L / kMinKeysPerSplit : 1;
  if (ns > max_ns) ns = max_ns;
  return split_into(L, ns);
}

// Cache layout [B][nh][Lstride][dh]; sequence b attends to its first
// seq_len[b] cached keys (all L when seq_len is NULL), clamped to [0, L].
struct Prefix {
  int L, Lstride;
  const int32_t *seq_len;
};

template <int DH, int QT, int STAGES = 1>
medusa_status launch_bf16(hipStream_t st, const medusa_tree *t, int B, int nh, Prefix pf, Split sp, float scale,
                          const void *q, const void *k_tree, const void *v_tree, const void *k_cache,
                          const void *v_cache, void *out, void *ws) {
  const int L = pf.L;
  const int qgroups = (t->T + kQB * QT - 1) / (kQB * QT);
  const long nblocks = (long)B * nh * qgroups * sp.nsplit;
  if (nblocks > 0x7fffffffL) return fail(MEDUSA_ERR_UNSUPPORTED, "tree_attention: grid too large");
  float *ws_o = nullptr;
  float2 *ws_ml = nullptr;
  if (sp.nsplit > 1) {
    ws_o = static_cast<float *>(ws);
    ws_ml = reinterpret_cast<float2 *>(ws_o + (size_t)sp.nsplit * B * nh * t->T * DH);
  }
  // blocks per CU the build is made for: three only for one query tile per wave
  auto kern = tree_attn_bf16<DH, QT, STAGES, 2>;
  if constexpr (QT == 1) {
    if (sp.three_per_cu) kern = tree_attn_bf16<DH, QT, STAGES, 3>;
  }
  MEDUSA_LAUNCH("tree_attention", kern, dim3((unsigned)nblocks), dim3(kThreads), 0, st, B, nh, t->T,
                     t->W, L, pf.Lstride, pf.seq_len, scale * kLog2e, qgroups, sp.nsplit, sp.per_split,
                     static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k_tree),
                     static_cast<const uint16_t *>(v_tree), static_cast<const uint16_t *>(k_cache),
                     static_cast<const uint16_t *>(v_cache), t->d_mask, t->d_tile_need,
                     static_cast<uint16_t *>(out), ws_o, ws_ml);
  medusa_status s = check_launch("tree_attention");
  if (s != MEDUSA_OK || sp.nsplit == 1) return s;
  const long rows = (long)B * nh * t->T;
  const int rpb = 256 / (DH / 4);
  auto merge = sp.nsplit == 2 ? tree_attn_merge_bf16<DH, 2>
             : sp.nsplit == 3 ? tree_attn_merge_bf16<DH, 3>
             : sp.nsplit == 4 ? tree_attn_merge_bf16<DH, 4>
             : sp.nsplit <= kMergeUnroll ? tree_attn_merge_bf16<DH, kMergeUnroll>
                                         : tree_attn_merge_bf16<DH, 0>;
  MEDUSA_LAUNCH("tree_attention", merge, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, st,
                     B, nh, t->T, sp.nsplit, ws_o, ws_ml, static_cast<uint16_t *>(out));
  return check_launch("tree_attention merge");
}


template <int NW>
medusa_status launch_wide(hipStream_t st, const medusa_tree *t, int B, int nh, Prefix pf, Split sp, float scale,
                          const void *q, const void *k_tree, const void *v_tree, const void *k_cache,
                          const void *v_cache, void *out, void *ws) {
  constexpr int DH = 128;
  const long nblocks = (long)B * nh * sp.nsplit;
  if (nblocks > 0x7fffffffL) return fail(MEDUSA_ERR_UNSUPPORTED, "tree_attention: grid too large");
  float *ws_o = nullptr;
  float2 *ws_ml = nullptr;
  if (sp.nsplit > 1) {
    ws_o = static_cast<float *>(ws);
    ws_ml = reinterpret_cast<float2 *>(ws_o + (size_t)sp.nsplit * B * nh * t->T * DH);
  }
  MEDUSA_LAUNCH("tree_attention", tree_attn_wide_bf16<NW>, dim3((unsigned)nblocks), dim3(64 * NW), 0, st, B, nh,
                t->T, t->W, pf.L, pf.Lstride, pf.seq_len, scale * kLog2e, sp.nsplit, sp.per_split,
                static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k_tree),
                static_cast<const uint16_t *>(v_tree), static_cast<const uint16_t *>(k_cache),
                static_cast<const uint16_t *>(v_cache), t->d_mask, t->d_tile_need, static_cast<uint16_t *>(out),
                ws_o, ws_ml);
  medusa_status s = check_launch("tree_attention");
  if (s != MEDUSA_OK || sp.nsplit == 1) return s;
  const long rows = (long)B * nh * t->T;
  const int rpb = 256 / (DH / 4);
  auto merge = sp.nsplit == 2 ? tree_attn_merge_bf16<DH, 2>
             : sp.nsplit == 3 ? tree_attn_merge_bf16<DH, 3>
             : sp.nsplit == 4 ? tree_attn_merge_bf16<DH, 4>
             : sp.nsplit <= kMergeUnroll ? tree_attn_merge_bf16<DH, kMergeUnroll>
                                         : tree_attn_merge_bf16<DH, 0>;
  MEDUSA_LAUNCH("tree_attention", merge, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, st,
                B, nh, t->T, sp.nsplit, ws_o, ws_ml, static_cast<uint16_t *>(out));
  return check_launch("tree_attention merge");
}

template <int DH>
medusa_status launch_f32(hipStream_t st, const medusa_tree *t, int B, int nh, Prefix pf, float scale,
                         const void *q, const void *k_tree, const void *v_tree, const void *k_cache,
                         const void *v_cache, void *out) {
  const int qgroups = (t->T + kF32Q - 1) / kF32Q;
  MEDUSA_LAUNCH("tree_attention", (tree_attn_f32<DH>), dim3(B * nh * qgroups), dim3(256), 0, st, B, nh, t->T, t->W, pf.L,
                     pf.Lstride, pf.seq_len, scale, qgroups, static_cast<const float *>(q), static_cast<const float *>(k_tree),
                     static_cast<const float *>(v_tree), static_cast<const float *>(k_cache),
                     static_cast<const float *>(v_cache), t->d_mask, static_cast<float *>(out));
  return check_launch("tree_attention");
}

}  // namespace

extern "C" size_t tree_attention_workspace(medusa_dtype dt, const medusa_tree *t, int B, int nh,
                                           int dh, int L) {
  if (!t || B < 1 || nh < 1 || dh < 1 || L < 0 || dt != MEDUSA_BF16) return 0;
  const Split sp = use_wide(dt, dh, t->T, B, nh) ? choose_split_wide(B, nh, L) : choose_split(B, nh, t->T, L);
  if (sp.nsplit == 1) return 0;
  return (size_t)sp.nsplit * B * nh * t->T * (dh + 2) * sizeof(float);
}

namespace {

medusa_status attention_entry(const char *who, medusa_stream_t stream, medusa_dtype dt, const medusa_tree *t,
                              int B, int nh, int dh, Prefix pf, float scale, const void *q, const void *k_tree,
                              const void *v_tree, const void *k_cache, const void *v_cache, void *out, void *ws,
                              size_t ws_bytes) {
  medusa_status s = check_tree_on_device(t);
  if (s != MEDUSA_OK) return s;
  const int L = pf.L;
  if (dt != MEDUSA_F32 && dt != MEDUSA_BF16) return fail(MEDUSA_ERR_ARG, "%s: unknown dtype", who);
  if (B < 1 || nh < 1 || L < 0 || pf.Lstride < L)
    return fail(MEDUSA_ERR_ARG, "%s: B=%d nh=%d L=%d stride=%d", who, B, nh, L, pf.Lstride);
  if (dh != 64 && dh != 128) return fail(MEDUSA_ERR_UNSUPPORTED, "%s: dh=%d not in {64, 128}", who, dh);
  if (!(scale >= 0.f) || !isfinite(scale)) return fail(MEDUSA_ERR_ARG, "%s: bad scale", who);
  if (!q || !k_tree || !v_tree || !out || (L > 0 && (!k_cache || !v_cache)))
    return fail(MEDUSA_ERR_ARG, "%s: NULL pointer", who);
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out) ||
      (L > 0 && (!aligned16(k_cache) || !aligned16(v_cache))))
    return fail(MEDUSA_ERR_ARG, "%s: pointers must be 16-byte aligned", who);
  const size_t need = tree_attention_workspace(dt, t, B, nh, dh, L);
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu", who, ws_bytes, need);
  if (need > 0 && !aligned16(ws)) return fail(MEDUSA_ERR_ARG, "%s: workspace must be 16-byte aligned", who);
  const float sc = scale == 0.f ? 1.0f / sqrtf((float)dh) : scale;
  hipStream_t st = as_stream(stream);
  if (use_wide(dt, dh, t->T, B, nh)) {
    const Split sp = choose_split_wide(B, nh, L);
    const int nw = wide_waves(t->T);
    return nw == 4 ? launch_wide<4>(st, t, B, nh, pf, sp, sc, q, k_tree, v_tree, k_cache, v_cache, out, ws)
         : nw == 8 ? launch_wide<8>(st, t, B, nh, pf, sp, sc, q, k_tree, v_tree, k_cache, v_cache, out, ws)
                   : launch_wide<12>(st, t, B, nh, pf, sp, sc, q, k_tree, v_tree, k_cache, v_cache, out, ws);
  }
  if (dt == MEDUSA_BF16) {
    const bool two = qtiles_for(t->T) == 2;
    const Split sp = choose_split(B, nh, t->T, L);
    if (dh == 128)
      return two ? launch_bf16<128, 2>(st, t, B, nh, pf, sp, sc, q, k_tree, v_tree, k_cache, v_cache, out, ws)
                 : launch_bf16<128, 1>(st, t, B, nh, pf, sp, sc, q, k_tree, v_tree, k_cache, v_cache, out, ws);
    return two ? launch_bf16<64, 2>(st, t, B, nh, pf, sp, sc, q, k_tree, v_tree, k_cache, v_cache, out, ws)
               : launch_bf16<64, 1>(st, t, B, nh, pf, sp, sc, q, k_tree, v_tree, k_cache, v_cache, out, ws);
  }
  return dh == 128 ? launch_f32<128>(st, t, B, nh, pf, sc, q, k_tree, v_tree, k_cache, v_cache, out)
                   : launch_f32<64>(st, t, B, nh, pf, sc, q, k_tree, v_tree, k_cache, v_cache, out);
}

}  // namespace

extern "C" medusa_status tree_attention(medusa_stream_t stream, medusa_dtype dt, const medusa_tree *t,
                                        int B, int nh, int dh, int L, float scale, const void *q,
                                        const void *k_tree, const void *v_tree, const void *k_cache,
                                        const void *v_cache, void *out, void *ws, size_t ws_bytes) {
  TraceRange tr("tree_attention");
  return attention_entry("tree_attention", stream, dt, t, B, nh, dh, Prefix{L, L, nullptr}, scale, q, k_tree,
                         v_tree, k_cache, v_cache, out, ws, ws_bytes);
}

extern "C" medusa_status tree_attention_ragged(medusa_stream_t stream, medusa_dtype dt, const medusa_tree *t,
                                               int B, int nh, int dh, int L_cap, int L_max,
                                               const int32_t *seq_len, float scale, const void *q,
                                               const void *k_tree, const void *v_tree, const void *k_cache,
                                               const void *v_cache, void *out, void *ws, size_t ws_bytes) {
  TraceRange tr("tree_attention_ragged");
  if (!seq_len) return fail(MEDUSA_ERR_ARG, "tree_attention_ragged: NULL seq_len");
  if (L_max > L_cap) return fail(MEDUSA_ERR_ARG, "tree_attention_ragged: L_max=%d > L_cap=%d", L_max, L_cap);
  return attention_entry("tree_attention_ragged", stream, dt, t, B, nh, dh, Prefix{L_max, L_cap, seq_len}, scale,
                         q, k_tree, v_tree, k_cache, v_cache, out, ws, ws_bytes);
}
