// Medusa head projections over many rows (the verify-pass shape: every tree
// node of every sequence, M = B*T rows; also the backbone's LM head, a head
// with W1 = 0, over the same rows).  Same arithmetic as the skinny kernels in
// heads.hip (bf16 products, fp32 accumulation, the same fused epilogues), but
// at M in the hundreds to ten-thousands the weights are re-used M times and
// the work is matrix-core bound, so the kernel is a classic block-tiled GEMM:
//
//   out[head][m][n] = sum_i W[head][n][i] * X[head][m][i]
//
// Block tile BN (weight rows n) x BM (activation rows m), reduction tile 64.
// Both operand tiles go global -> registers -> LDS: two LDS stages and two
// register sets, so while one stage feeds the MFMAs the next tile waits in
// registers and the one after is being loaded; one barrier per reduction
// tile.  LDS rows are padded to 144 bytes.  Eight waves per block, each owning a TN x TM sub-tile of
// v_mfma_f32_16x16x32_bf16 accumulators with the weight tile as the A operand,
// so D[n][m] lands as four consecutive n of one m per lane: one 16-byte fp32
// store (logits) or one 8-byte bf16 store (ResBlock) per fragment.
//
// Block order: consecutive block ids are dealt round-robin to the 8 XCDs, so
// ids are remapped to make each XCD run a contiguous range of tiles, and the
// range is ordered in groups of GM activation tiles (m fastest), so the blocks
// that run together on one XCD share both weight and activation tiles in its
// L2.
#include "common.h"
#include "gemm.h"

using namespace medusa;

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));


__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// BK: reduction tile (BK/32 MFMA k-steps); LDS rows padded by 16 bytes
template <int BN, int BM, int WGN, int WGM, int BK>
struct TileShape {
  static constexpr int kThreads = 64 * WGN * WGM;
  static constexpr int kLdk = BK + 8;                  // padded LDS row, elements
  static constexpr int CPR = BK / 8;                   // 16-byte chunks per row per k-tile
  static constexpr int SPT = BK / 32;                  // MFMA k-steps per k-tile
  static constexpr int TN = BN / WGN, TM = BM / WGM;   // wave sub-tile
  static constexpr int FN = TN / 16, FM = TM / 16;     // MFMA tiles per wave
  static constexpr int WCH = BN * CPR / kThreads;      // chunks per thread per k-tile
  static constexpr int XCH = BM * CPR / kThreads;
  static constexpr int kStage = (BN + BM) * kLdk;      // elements per LDS stage
  static constexpr size_t kLdsBytes = 2 * kStage * sizeof(uint16_t);
  static_assert(BK == 32 || BK == 64, "k-tile");
  static_assert(TN % 16 == 0 && TM % 16 == 0, "wave tile");
  static_assert((BN * CPR) % kThreads == 0 && (BM * CPR) % kThreads == 0, "load split");
  static_assert((kThreads / 64) % SPT == 0 && kThreads % CPR == 0, "affine slots");
  static_assert(BN % 16 == 0, "packed tiles");
};

template <int EPI, bool PACKED, int BN, int BM, int WGN, int WGM, int BK, int MINW>
__global__ __launch_bounds__(64 * WGN * WGM, MINW) void head_gemm_tiled(
    const uint16_t *__restrict__ W, const uint16_t *__restrict__ X, long x_head_stride, int N,
    int H, int M, int GM, int lgG, const uint16_t *__restrict__ resid, uint16_t *__restrict__ out_bf16,
    float *__restrict__ out_f32) {
  using S = TileShape<BN, BM, WGN, WGM, BK>;
  constexpr int kLdk = S::kLdk;
  extern __shared__ u32x4_t lds_raw[];
  uint16_t *lds = reinterpret_cast<uint16_t *>(lds_raw);

  // ---- tile of this block
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  const int per_head = tiles_n * tiles_m;
  int id = xcd_remap(blockIdx.x, gridDim.x);
  const int head = id / per_head;
  id -= head * per_head;
  const int span = GM * tiles_n;
  const int grp = id / span;
  const int mfirst = grp * GM;
  const int gm = min(GM, tiles_m - mfirst);
  const int rem = id - grp * span;
  const int m0 = (mfirst + rem % gm) * BM, n0 = (rem / gm) * BN;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int wn = wave % WGN, wm = wave / WGN;

  // ---- per-thread load slots: 32-bit byte offsets from the head's base (the
  // launcher checks that a head's operands span less than 4 GiB; rows past the
  // end re-read the last row) and LDS destinations, affine in the slot j.
  const int NTt = (N + 15) / 16, Ssteps = H / 32;
  const char *wbase = reinterpret_cast<const char *>(W) + (PACKED ? (size_t)head * packed_tiles(N) * Ssteps * 1024
                                                                   : (size_t)head * N * H * 2);
  const char *xbase = reinterpret_cast<const char *>(X) + (size_t)head * x_head_stride * 2;
  uint32_t woff[S::WCH], xoff[S::XCH];
#pragma unroll
  for (int j = 0; j < S::WCH; ++j) {
    const int c = tid + j * S::kThreads;
    if (PACKED) {
      // slot c: lane c%64 of fragment F = c/64: row tile F/SPT, k-step F%SPT
      const int F = c >> 6;
      const int t = min(n0 / 16 + F / S::SPT, NTt - 1);
      woff[j] = ((uint32_t)packed_fragment(t, F % S::SPT, Ssteps, lgG) * 64u + (uint32_t)(c & 63)) * 16u;
    } else {
      // slot c: row c/CPR, columns 8*(c%CPR)..+7 (each row's k-tile in CPR lanes)
      const int n = min(n0 + c / S::CPR, N - 1);
      woff[j] = ((uint32_t)n * (uint32_t)H + (uint32_t)(c % S::CPR) * 8u) * 2u;
    }
  }
#pragma unroll
  for (int j = 0; j < S::XCH; ++j) {
    const int c = tid + j * S::kThreads;
    const int m = min(m0 + c / S::CPR, M - 1);
    xoff[j] = ((uint32_t)m * (uint32_t)H + (uint32_t)(c % S::CPR) * 8u) * 2u;
  }
  // LDS destinations (elements): packed slot -> row 16*(F/SPT) + l%16, column
  // 32*(F%SPT) + 8*(l/16) with F = c/64, l = c%64; row-major slot -> row c/CPR,
  // column 8*(c%CPR)
  constexpr int kWdstStep = PACKED ? (S::kThreads / 64 / S::SPT) * 16 * kLdk : (S::kThreads / S::CPR) * kLdk;
  const int wdst0 = PACKED ? (((tid >> 6) / S::SPT) * 16 + (tid & 15)) * kLdk + ((tid >> 6) % S::SPT) * 32 +
                                 ((tid >> 4) & 3) * 8
                           : (tid / S::CPR) * kLdk + (tid % S::CPR) * 8;
  const int xdst0 = BN * kLdk + (tid / S::CPR) * kLdk + (tid % S::CPR) * 8;
  constexpr int kXdstStep = (S::kThreads / S::CPR) * kLdk;
  const uint32_t w_step = PACKED ? (S::SPT * 1024u) << lgG : BK * 2u;   // bytes per k-tile

  // two register sets: tile j is loaded into set j % 2
  u32x4_t wreg[2][S::WCH], xreg[2][S::XCH];
  auto load = [&](int kt, int set) {
    const uint32_t wk = (uint32_t)kt * w_step, xk = (uint32_t)kt * (BK * 2u);
#pragma unroll
    for (int j = 0; j < S::WCH; ++j) wreg[set][j] = *reinterpret_cast<const u32x4_t *>(wbase + (woff[j] + wk));
#pragma unroll
    for (int j = 0; j < S::XCH; ++j) xreg[set][j] = *reinterpret_cast<const u32x4_t *>(xbase + (xoff[j] + xk));
  };
  auto stash = [&](int set, int stage) {
    uint16_t *base = lds + stage * S::kStage;
#pragma unroll
    for (int j = 0; j < S::WCH; ++j) *reinterpret_cast<u32x4_t *>(base + wdst0 + j * kWdstStep) = wreg[set][j];
#pragma unroll
    for (int j = 0; j < S::XCH; ++j) *reinterpret_cast<u32x4_t *>(base + xdst0 + j * kXdstStep) = xreg[set][j];
  };

  f32x4_t acc[S::FN][S::FM];
#pragma unroll
  for (int f = 0; f < S::FN; ++f)
#pragma unroll
    for (int g = 0; g < S::FM; ++g) acc[f][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fragment read offsets within a stage (row lr of the tile, k slice 8*lg)
  const int a_off = (wn * S::TN + lr) * kLdk + lg * 8;
  const int b_off = BN * kLdk + (wm * S::TM + lr) * kLdk + lg * 8;
  auto compute = [&](int stage) {
    const uint16_t *base = lds + stage * S::kStage;
#pragma unroll
    for (int ks = 0; ks < S::SPT; ++ks) {
      u32x4_t a[S::FN], b[S::FM];
#pragma unroll
      for (int f = 0; f < S::FN; ++f) a[f] = *reinterpret_cast<const u32x4_t *>(base + a_off + f * 16 * kLdk + ks * 32);
#pragma unroll
      for (int g = 0; g < S::FM; ++g) b[g] = *reinterpret_cast<const u32x4_t *>(base + b_off + g * 16 * kLdk + ks * 32);
#pragma unroll
      for (int f = 0; f < S::FN; ++f)
#pragma unroll
        for (int g = 0; g < S::FM; ++g) acc[f][g] = mfma(a[f], b[g], acc[f][g]);
    }
  };

  // Software pipeline, two k-tiles per trip (H % (2*BK) == 0, so nk is even):
  // while stage s feeds the MFMAs, tile kt+1 waits in registers (loaded one
  // compute phase earlier) and tile kt+2 is being loaded, so every global
  // load has two compute phases to arrive.  Loads past the end re-read the
  // last tile into a stage that is never read again, keeping the trip
  // branch-free.
  const int nk = H / BK;
  load(0, 0);
  load(min(1, nk - 1), 1);
  stash(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    load(min(kt + 2, nk - 1), 0);
    compute(0);
    stash(1, 1);
    __syncthreads();
    load(min(kt + 3, nk - 1), 1);
    compute(1);
    stash(0, 0);
    __syncthreads();
  }

  // ---- epilogue: lane holds D[n + v][m], v < 4, for n = tile + 4*lg, m = tile + lr
  const bool vec = (N % 4) == 0;
#pragma unroll
  for (int g = 0; g < S::FM; ++g) {
    const int m = m0 + wm * S::TM + g * 16 + lr;
    if (m >= M) continue;
#pragma unroll
    for (int f = 0; f < S::FN; ++f) {
      const int n = n0 + wn * S::TN + f * 16 + lg * 4;
      if (n >= N) continue;
      const f32x4_t v = acc[f][g];
      const size_t o = ((size_t)head * M + m) * N + n;
      if (EPI == kEpiLogits) {
        if (vec) {
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t *>(out_f32 + o));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) out_f32[o + e] = v[e];
        }
      } else {
        // N == H here; H % 128 == 0 so the four columns are in range and aligned
        const u32x2_t hv = *reinterpret_cast<const u32x2_t *>(resid + (size_t)m * H + n);
        uint16_t hb[4] = {(uint16_t)(hv[0] & 0xffffu), (uint16_t)(hv[0] >> 16), (uint16_t)(hv[1] & 0xffffu),
                          (uint16_t)(hv[1] >> 16)};
        uint16_t r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float u = v[e];
          r[e] = f32_to_bf16_rne(bf16_to_f32(hb[e]) + u / (1.0f + expf(-u)));
        }
        const u32x2_t rv = {(uint32_t)r[0] | ((uint32_t)r[1] << 16), (uint32_t)r[2] | ((uint32_t)r[3] << 16)};
        *reinterpret_cast<u32x2_t *>(out_bf16 + o) = rv;
      }
    }
  }
}

template <int EPI, bool PACKED, int BN, int BM, int WGN, int WGM, int BK, int MINW>
medusa_status launch_tiled(hipStream_t st, const uint16_t *W, const uint16_t *X, long xhs, int K, int N,
                           int H, int M, int GM, int lgG, const uint16_t *resid, uint16_t *ob, float *of) {
  using S = TileShape<BN, BM, WGN, WGM, BK>;
  if (H % (2 * BK) != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "head projection: H %% %d != 0 (H=%d)", 2 * BK, H);
  auto kern = head_gemm_tiled<EPI, PACKED, BN, BM, WGN, WGM, BK, MINW>;
  static bool attr_set = false;   // per instantiation; setting it twice is harmless
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)S::kLdsBytes) != hipSuccess)
      return fail(MEDUSA_ERR_HIP, "head projection: cannot reserve %zu bytes of LDS", S::kLdsBytes);
    attr_set = true;
  }
  const long blocks = (long)K * ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
  if (blocks > 0x7fffffffL) return fail(MEDUSA_ERR_UNSUPPORTED, "head projection: %ld tiles", blocks);
  MEDUSA_LAUNCH("medusa heads (many rows)", kern, dim3((unsigned)blocks), dim3(S::kThreads), S::kLdsBytes, st, W, X, xhs, N, H, M,
                     GM, lgG, resid, ob, of);
  return check_launch(EPI == kEpiLogits ? "medusa_head_vocab (tiled)" : "medusa_head_resblock (tiled)");
}

// ---------------------------------------------------------------------------
// Fragment-fed variant for many rows (used when both operands are stored in
// matrix-core fragment order: the packed weights, and activations packed by
// pack_rows_kernel into a caller's workspace).
//
// Why a second kernel: with the activations row-major, every activation
// fragment is a gather of 16 rows x 64 bytes, and the load path (texture
// addresser) is the busiest unit; stored as 1 KiB fragments, both operands
// are single contiguous wave loads.  Those go straight from global memory into
// LDS (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16 * lane,
// i.e. a fragment stays in lane order), so there are no staging registers, no
// padding and no LDS bank conflicts, and a fragment is read back with one
// ds_read_b128 per lane.
//
// Block tile 256 (weight rows n) x 256 (activation rows m), one 32-deep
// reduction step per stage, four stages (4 x 32 KiB of LDS) with the loads for
// step s+3 issued while step s is worked on.  Eight waves, two per SIMD, each
// owning a 128 x 64 sub-tile (32 v_mfma_f32_16x16x32_bf16 per step from 8
// weight and 4 activation fragments).  Waves 0-3 and 4-7 run half a phase
// apart ("ping-pong"): while one wave of a SIMD issues its 32 MFMAs at raised
// priority, the other issues its loads and LDS reads, so the matrix core is
// fed by one wave while the other fills its registers.  Waves 4-7 take one
// extra barrier at the start and waves 0-3 one at the end, so every wave
// passes the same number of barriers.
//
// Ordering, for the wave's memory phase of step s (vmcnt counts this wave's
// loads, all into LDS):
//   issue the 4 loads of step s+3 into stage (s+3) % 4 == (s-1) % 4: both wave
//     groups finished reading step s-1 before the barrier that opened this
//     phase (each waits lgkmcnt(0) before closing its memory phase)
//   read step s's 12 fragments; wait vmcnt(8) (this wave's loads of step s+1
//     are in LDS; only steps s+2, s+3 may be outstanding) and lgkmcnt(0)
//   barrier; compute phase; barrier
// A stage is read by waves 0-3 in half-phase 2s and by waves 4-7 in 2s+1;
// every wave's loads of step s completed in its memory phase of step s-1,
// which ended by the barrier before half-phase 2s.
// The stages are four separate __shared__ arrays and the loop is unrolled by
// four, so the compiler's wait insertion can tell them apart (one shared
// array would make it wait for every outstanding load before each read).

typedef uint32_t u32x4_frag_t __attribute__((ext_vector_type(4)));
constexpr int kFragStageVec = 2048;                 // 32 fragments of 1 KiB, in 16-byte vectors
__shared__ u32x4_frag_t frag_stage0[kFragStageVec];
__shared__ u32x4_frag_t frag_stage1[kFragStageVec];
__shared__ u32x4_frag_t frag_stage2[kFragStageVec];
__shared__ u32x4_frag_t frag_stage3[kFragStageVec];

template <int B>
__device__ __forceinline__ u32x4_frag_t *frag_stage() {
  if (B == 0) return frag_stage0;
  if (B == 1) return frag_stage1;
  if (B == 2) return frag_stage2;
  return frag_stage3;
}

// s_waitcnt with vmcnt = vm and lgkmcnt = lgkm (gfx9 encoding; expcnt left at its maximum)
#define MEDUSA_WAITCNT(vm, lgkm) \
  __builtin_amdgcn_s_waitcnt(((vm) & 0xF) | ((((vm) >> 4) & 3) << 14) | (7 << 4) | (((lgkm) & 0xF) << 8))

__device__ __forceinline__ void dma16(const char *g, u32x4_frag_t *l) {
  // address-space casts (C-style: reinterpret_cast cannot change the address space)
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)g,
                                   (void __attribute__((address_space(3))) *)l, 16, 0, 0);
}

__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Activations [K][M][H] (head stride xhs elements) -> fragment order
// [K][ceil(M/16)][H/32][64 lanes][8]: lane l of fragment (row tile t, step s)
// holds row 16t + l % 16, columns 32s + 8(l / 16) .. + 7; rows >= M are zero.
__global__ void pack_rows_kernel(const uint16_t *__restrict__ X, long xhs, int K, int M, int H,
                                 uint16_t *__restrict__ Xp) {
  const int S = H / 32, MT = (M + 15) / 16;
  const size_t total = (size_t)K * MT * S * 64;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int l = (int)(i & 63);
  size_t f = i >> 6;
  const int s = (int)(f % S);
  f /= S;
  const int t = (int)(f % MT);
  const int k = (int)(f / MT);
  const int m = t * 16 + (l & 15);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (m < M) v = *reinterpret_cast<const u32x4_t *>(X + (size_t)k * xhs + (size_t)m * H + s * 32 + (l >> 4) * 8);
  *reinterpret_cast<u32x4_t *>(Xp + i * 8) = v;
}

template <int EPI>
__global__ __launch_bounds__(512, 1) void head_gemm_frag(const uint16_t *__restrict__ Wp, const uint16_t *__restrict__ Xp,
                                                          int x_heads, int N, int H, int M, int GM, int lgG,
                                                          const uint16_t *__restrict__ resid,
                                                          uint16_t *__restrict__ out_bf16, float *__restrict__ out_f32,
                                                          uint16_t *__restrict__ out_packed) {
  constexpr int BN = 256, BM = 256, kAhead = 3;
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  const int per_head = tiles_n * tiles_m;
  int id = xcd_remap(blockIdx.x, gridDim.x);
  const int head = id / per_head;
  id -= head * per_head;
  const int span = GM * tiles_n;
  const int grp = id / span;
  const int mfirst = grp * GM;
  const int gm = min(GM, tiles_m - mfirst);
  const int rem = id - grp * span;
  const int m0 = (mfirst + rem % gm) * BM, n0 = (rem / gm) * BN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS addresses stay scalar
  const int lr = lane & 15, lg = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;       // 128 (n) x 64 (m) sub-tile
  const bool late = wave >= 4;                   // the wave group running half a phase behind
  const int S = H / 32, NT = packed_tiles(N), MT = (M + 15) / 16;
  const char *wbase = reinterpret_cast<const char *>(Wp) + (size_t)head * NT * S * 1024;
  const char *xbase = reinterpret_cast<const char *>(Xp) + (x_heads > 1 ? (size_t)head * MT * S * 1024 : 0);
  // this wave loads weight fragments (row tiles) 2w, 2w+1 and activation fragments 2w, 2w+1 of
  // the block at every step; tiles past the end re-read the last one (their results are not stored)
  uint32_t woff[2], xoff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = min(n0 / 16 + 2 * wave + j, NT - 1);
    woff[j] = (uint32_t)packed_fragment(t, 0, S, lgG) * 1024u + lane * 16u;
    const int mt = min(m0 / 16 + 2 * wave + j, MT - 1);
    xoff[j] = (uint32_t)mt * S * 1024u + lane * 16u;
  }
  const uint32_t wstep = 1024u << lgG;   // bytes between one row tile's consecutive steps
  auto issue = [&](int s, u32x4_frag_t *stg) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dma16(wbase + woff[j] + (uint32_t)s * wstep, stg + (2 * wave + j) * 64);
      dma16(xbase + xoff[j] + (uint32_t)s * 1024u, stg + (16 + 2 * wave + j) * 64);
    }
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t a[8], b[4];
  const int aoff = wn * 8 * 64 + lane, boff = (16 + wm * 4) * 64 + lane;
  const int nsteps = S;   // a multiple of 4 (H % 128 == 0)

  issue(0, frag_stage<0>());
  issue(min(1, nsteps - 1), frag_stage<1>());
  issue(min(2, nsteps - 1), frag_stage<2>());
  MEDUSA_WAITCNT(8, 15);   // this wave's loads of step 0 are in LDS
  block_barrier();         // everyone's are
  if (late) block_barrier();

  auto body = [&](int s, const u32x4_frag_t *cur, u32x4_frag_t *dst) {
    issue(min(s + kAhead, nsteps - 1), dst);   // past the end: re-load the last step into a stage never read
#pragma unroll
    for (int f = 0; f < 8; ++f) a[f] = cur[aoff + f * 64];
#pragma unroll
    for (int g = 0; g < 4; ++g) b[g] = cur[boff + g * 64];
    MEDUSA_WAITCNT(8, 0);
    block_barrier();
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[f][g] = mfma(a[f], b[g], acc[f][g]);
    __builtin_amdgcn_s_setprio(0);
    block_barrier();
  };
  for (int s = 0; s < nsteps; s += 4) {
    body(s + 0, frag_stage<0>(), frag_stage<3>());
    body(s + 1, frag_stage<1>(), frag_stage<0>());
    body(s + 2, frag_stage<2>(), frag_stage<1>());
    body(s + 3, frag_stage<3>(), frag_stage<2>());
  }
  if (!late) block_barrier();
  MEDUSA_WAITCNT(0, 0);   // the re-loads past the end land before the block's LDS is handed on

  // epilogue: lane holds D[n + v][m], v < 4, for n = tile + 4*lg, m = tile + lr
  const bool vec = (N % 4) == 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int m = m0 + wm * 64 + g * 16 + lr;
    if (m >= M) continue;
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int n = n0 + wn * 128 + f * 16 + lg * 4;
      if (n >= N) continue;
      const f32x4_t v = acc[f][g];
      const size_t o = ((size_t)head * M + m) * N + n;
      if (EPI == kEpiLogits) {
        if (vec) {
          // a plain store: the neighbouring f writes the other half of each
          // 128-byte line, and the two halves meet in L2 (non-temporal stores
          // sent the half lines on separately: 889 against 850 us for the 4 x
          // 1024-row vocabulary projection)
          *reinterpret_cast<f32x4_t *>(out_f32 + o) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) out_f32[o + e] = v[e];
        }
      } else {
        const u32x2_t hv = *reinterpret_cast<const u32x2_t *>(resid + (size_t)m * H + n);
        uint16_t hb[4] = {(uint16_t)(hv[0] & 0xffffu), (uint16_t)(hv[0] >> 16), (uint16_t)(hv[1] & 0xffffu),
                          (uint16_t)(hv[1] >> 16)};
        uint16_t r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float u = v[e];
          r[e] = f32_to_bf16_rne(bf16_to_f32(hb[e]) + u / (1.0f + expf(-u)));
        }
        const u32x2_t rv = {(uint32_t)r[0] | ((uint32_t)r[1] << 16), (uint32_t)r[2] | ((uint32_t)r[3] << 16)};
        *reinterpret_cast<u32x2_t *>(out_bf16 + o) = rv;
        if (out_packed) {
          // the same four values in fragment order for the next contraction: fragment (row tile
          // m/16, step n/32) of this head, lane m%16 + 16 * ((n%32)/8), elements n%8 .. +3
          const size_t fo = (((size_t)head * MT + (m >> 4)) * S + (n >> 5)) * 512 +
                            (size_t)((m & 15) + 16 * ((n & 31) >> 3)) * 8 + (n & 7);
          *reinterpret_cast<u32x2_t *>(out_packed + fo) = rv;
        }
      }
    }
  }
}

}  // namespace

namespace medusa {

size_t packed_rows_bytes(int K, int M, int H) {
  if (K < 1 || M < 1 || H < 32 || H % 32 != 0) return 0;
  return (size_t)K * ((M + 15) / 16) * (H / 32) * 1024;
}

medusa_status pack_rows(hipStream_t st, const uint16_t *X, long xhs, int K, int M, int H, uint16_t *Xp) {
  const size_t lanes = packed_rows_bytes(K, M, H) / 16;
  MEDUSA_LAUNCH("medusa heads (many rows)", pack_rows_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, st, X, xhs, K, M, H, Xp);
  return check_launch("pack_rows");
}

medusa_status fragments_supported(int K, int N, int H, int M) {
  if (H % 128 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "head projection: H %% 128 != 0 (H=%d)", H);
  const size_t w_head = (size_t)packed_tiles(N) * (H / 32) * 1024;
  if (w_head >= (1ull << 32) || packed_rows_bytes(1, M, H) >= (1ull << 32))
    return fail(MEDUSA_ERR_UNSUPPORTED, "head projection: one head's operands exceed 4 GiB (N=%d M=%d H=%d)", N, M, H);
  const long blocks = (long)K * ((N + 255) / 256) * ((M + 255) / 256);
  if (blocks > 0x7fffffffL) return fail(MEDUSA_ERR_UNSUPPORTED, "head projection: %ld tiles", blocks);
  return MEDUSA_OK;
}

template <int EPI>
medusa_status head_gemm_fragments(hipStream_t st, const uint16_t *Wp, const uint16_t *Xp, int x_heads, int K, int N,
                                  int H, int M, int lgG, const uint16_t *resid, uint16_t *ob, float *of, uint16_t *obp) {
  medusa_status s = fragments_supported(K, N, H, M);
  if (s != MEDUSA_OK) return s;
  const long blocks = (long)K * ((N + 255) / 256) * ((M + 255) / 256);
  MEDUSA_LAUNCH("medusa heads (many rows)", head_gemm_frag<EPI>, dim3((unsigned)blocks), dim3(512), 0, st, Wp, Xp, x_heads, N, H, M, 8,
                     lgG, resid, ob, of, obp);
  return check_launch(EPI == kEpiLogits ? "medusa_head_vocab_packed_ws" : "medusa_head_resblock_packed_ws");
}

template medusa_status head_gemm_fragments<kEpiResblock>(hipStream_t, const uint16_t *, const uint16_t *, int, int,
                                                         int, int, int, int, const uint16_t *, uint16_t *, float *,
                                                         uint16_t *);
template medusa_status head_gemm_fragments<kEpiLogits>(hipStream_t, const uint16_t *, const uint16_t *, int, int,
                                                       int, int, int, int, const uint16_t *, uint16_t *, float *,
                                                       uint16_t *);

}  // namespace medusa

namespace medusa {

template <int EPI, bool PACKED>
medusa_status head_gemm_many_rows(hipStream_t st, const uint16_t *W, const uint16_t *X, long xhs, int K,
                                  int N, int H, int M, int lgG, const uint16_t *resid, uint16_t *ob, float *of) {
  const size_t w_head = PACKED ? (size_t)packed_tiles(N) * (H / 32) * 1024 : (size_t)N * H * 2;
  if (w_head >= (1ull << 32) || (size_t)M * H * 2 >= (1ull << 32))
    return fail(MEDUSA_ERR_UNSUPPORTED, "head projection: one head's operands exceed 4 GiB (N=%d M=%d H=%d)", N, M, H);
  // up to 64 rows the work is weight-streaming bound: 64-row activation
  // tiles, 128-row weight tiles and two blocks per CU (measured at 64 rows,
  // 7B shape: ResBlock 120 -> 38 us, vocabulary 287 -> 191 us, LM head
  // 157 -> 48 us against the 256 x 256 tile); 64-row weight tiles when the
  // 128-row ones would give at most half a block per CU (ResBlock: 38 -> 30 us)
  if (M <= 64 && (long)K * ((N + 127) / 128) <= 128)
    return launch_tiled<EPI, PACKED, 64, 64, 2, 2, 64, 2>(st, W, X, xhs, K, N, H, M, 8, lgG, resid, ob, of);
  if (M <= 64) return launch_tiled<EPI, PACKED, 128, 64, 2, 2, 64, 2>(st, W, X, xhs, K, N, H, M, 8, lgG, resid, ob, of);
  return launch_tiled<EPI, PACKED, 256, 256, 2, 4, 64, 1>(st, W, X, xhs, K, N, H, M, 8, lgG, resid, ob, of);
}

template medusa_status head_gemm_many_rows<kEpiResblock, false>(hipStream_t, const uint16_t *, const uint16_t *,
                                                                long, int, int, int, int, int, const uint16_t *,
                                                                uint16_t *, float *);
template medusa_status head_gemm_many_rows<kEpiResblock, true>(hipStream_t, const uint16_t *, const uint16_t *,
                                                               long, int, int, int, int, int, const uint16_t *,
                                                               uint16_t *, float *);
template medusa_status head_gemm_many_rows<kEpiLogits, false>(hipStream_t, const uint16_t *, const uint16_t *,
                                                              long, int, int, int, int, int, const uint16_t *,
                                                              uint16_t *, float *);
template medusa_status head_gemm_many_rows<kEpiLogits, true>(hipStream_t, const uint16_t *, const uint16_t *,
                                                             long, int, int, int, int, int, const uint16_t *,
                                                             uint16_t *, float *);

}  // namespace medusa
