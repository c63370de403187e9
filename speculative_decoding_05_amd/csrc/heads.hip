// Medusa heads: r = h + SiLU(W1_k h) and logits = W2_k r.
//
// At decode time the heads see one row per sequence (M <= 32), so both
// projections are skinny GEMMs whose cost is streaming W1 / W2 from HBM once.
// More rows (the verify-pass shape) go to the block-tiled kernel in gemm.hip.
// bf16 path: each wave owns 16*R output rows and a quarter of the reduction;
// the weight slab is the MFMA A operand (v_mfma_f32_16x16x32_bf16: lane l
// holds row l%16, reduction slice 8*(l/16)..+7), activations are the B operand
// (M padded to 16*C columns), partial sums of the 4 waves are added in LDS and
// the epilogue (SiLU + residual + bf16 rounding, or fp32 store) is fused.
//
// Two weight layouts are accepted.  Row-major [K][N][H]: every load
// instruction touches 16 rows x 64 bytes.  Packed (medusa_pack_weights, layout
// in gemm.h): each 16x32 A fragment is one contiguous 1 KiB block in lane
// order, so every load instruction of a wave reads 1 KiB of consecutive bytes
// -- the layout reaches the HBM streaming rate that the row-major pattern
// loses to scattered row segments.  Weights are read with non-temporal loads
// so the small activation block stays in L2.
#include "common.h"
#include "gemm.h"

using namespace medusa;

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

constexpr int EPI_RESBLOCK = kEpiResblock, EPI_LOGITS = kEpiLogits;

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// out[head][m0+m][n] = sum_i W[head][n][i] * X[head][m0+m][i]   (m < Mg <= 16*C)
// R row tiles per wave, C column tiles, U k-steps of 32 loaded per wave before
// the MFMAs, NW waves per block splitting the reduction.
template <int R, int C, int EPI, bool PACKED, int U, int NW>
__global__ __launch_bounds__(64 * NW) void head_gemm_bf16(
    const uint16_t *__restrict__ W, const uint16_t *__restrict__ X, long x_head_stride, int N,
    int H, int M_total, int m0, int Mg, int tiles_per_head, int lgG, const uint16_t *__restrict__ resid,
    uint16_t *__restrict__ out_bf16, float *__restrict__ out_f32, uint32_t *__restrict__ tile_img) {
  __shared__ float red[NW][16 * C][16 * R + 1];
  const int head = blockIdx.x / tiles_per_head;
  const int n0 = (blockIdx.x % tiles_per_head) * 16 * R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int kspan = H / NW;
  const int k0 = wave * kspan + lg * 8;
  const uint16_t *Wh = PACKED ? nullptr : W + (size_t)head * N * H;
  const uint16_t *Xh = X + (size_t)head * x_head_stride + (size_t)m0 * H;

  // a_step: elements between the A fragments of consecutive k-steps
  const uint16_t *arow[R];
  int a_step;
  if (PACKED) {
    // fragment f of a head at f*512 elements, lane l at +8*l; consecutive
    // steps of one tile are G = 2^lgG fragments apart
    const int S = H / 32, NT = (N + 15) / 16;
    const int t0 = n0 / 16;
    const uint16_t *Wh_p = W + (size_t)head * packed_tiles(N) * S * 512 + lane * 8;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int t = t0 + r < NT ? t0 + r : NT - 1;  // ragged tail: valid tile, result discarded
      arow[r] = Wh_p + packed_fragment(t, wave * (kspan / 32), S, lgG) * 512;
    }
    a_step = 512 << lgG;
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int n = n0 + r * 16 + lr;
      n = n < N ? n : N - 1;  // ragged tail: read a valid row, result discarded
      arow[r] = Wh + (size_t)n * H + k0;
    }
    a_step = 32;
  }
  const uint16_t *brow[C];
  bool bval[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int m = c * 16 + lr;
    bval[c] = m < Mg;
    brow[c] = Xh + (size_t)(bval[c] ? m : 0) * H + k0;
  }

  f32x4_t acc[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const u32x4_t zero = {0u, 0u, 0u, 0u};
  const int steps = kspan / 32;
  int s = 0;
  for (; s + U <= steps; s += U) {
    u32x4_t a[U][R], b[U][C];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
        a[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(arow[r] + (s + u) * a_step));
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < C; ++c)
        b[u][c] = bval[c] ? *reinterpret_cast<const u32x4_t *>(brow[c] + (s + u) * 32) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[r][c] = mfma(a[u][r], b[u][c], acc[r][c]);
  }
  for (; s < steps; ++s) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(arow[r] + s * a_step));
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const u32x4_t b = bval[c] ? *reinterpret_cast<const u32x4_t *>(brow[c] + s * 32) : zero;
        acc[r][c] = mfma(a, b, acc[r][c]);
      }
    }
  }

  // D layout: lane l holds D[row 4*(l/16)+v][col l%16]; rows are n, cols are m
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][c * 16 + lr][r * 16 + lg * 4 + v] = acc[r][c][v];
  __syncthreads();

  // The lanes active in an iteration are whole waves (16*C*16*R is a multiple
  // of 256, the stride of 64), and the 16 lanes of a row hold the 16 columns
  // of one weight tile for one activation row: the optional tile maxima are
  // one row reduction.
  for (int e = threadIdx.x; e < 16 * C * 16 * R; e += 64 * NW) {
    const int m = e / (16 * R), nl = e % (16 * R);
    const int n = n0 + nl;
    const bool ok = m < Mg && n < N;
    const size_t o = ((size_t)head * M_total + m0 + m) * N + n;
    if (EPI == EPI_LOGITS) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][m][nl];
      if (ok) out_f32[o] = v;
      if (tile_img) {
        const uint32_t t = row_max_u32(ok ? order_image(v) : 0u);
        if (ok && (nl & 15) == 0) tile_img[((size_t)head * M_total + m0 + m) * ((N + 15) / 16) + n / 16] = t;
      }
    } else {
      if (!ok) continue;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][m][nl];
      const float hv = bf16_to_f32(resid[(size_t)(m0 + m) * H + n]);
      out_bf16[o] = f32_to_bf16_rne(hv + v / (1.0f + expf(-v)));
    }
  }
}

// fp32 path: one wave per (head, output row n, group of 8 rows m); lanes
// stride the reduction with float4 loads; wave-level sum.
template <int EPI>
__global__ __launch_bounds__(256) void head_gemm_f32(const float *__restrict__ W,
                                                     const float *__restrict__ X, long x_head_stride,
                                                     int K, int N, int H, int M,
                                                     const float *__restrict__ resid,
                                                     float *__restrict__ out) {
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int mgroups = (M + 7) / 8;
  const long total = (long)K * N * mgroups;
  if (gw >= total) return;
  const int mg = gw % mgroups;
  const int n = (gw / mgroups) % N;
  const int head = gw / (mgroups * N);
  const float *w = W + ((size_t)head * N + n) * H;
  const float *x = X + (size_t)head * x_head_stride;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int i = lane * 4; i < H; i += 256) {
    const float4 wv = *reinterpret_cast<const float4 *>(w + i);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = mg * 8 + j;
      if (m < M) {
        const float4 xv = *reinterpret_cast<const float4 *>(x + (size_t)m * H + i);
        acc[j] += wv.x * xv.x + wv.y * xv.y + wv.z * xv.z + wv.w * xv.w;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    for (int off = 32; off > 0; off >>= 1) acc[j] += __shfl_xor(acc[j], off);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = mg * 8 + j;
      if (m >= M) continue;
      const size_t o = ((size_t)head * M + m) * N + n;
      const float v = acc[j];
      if (EPI == EPI_LOGITS)
        out[o] = v;
      else
        out[o] = resid[(size_t)m * H + n] + v / (1.0f + expf(-v));
    }
  }
}


// Packed layout (gemm.h), G = 2^lgG:
// Wp[k][g][s][j][l][e] = W[k][16(G g + j) + l%16][32s + 8(l/16) + e]
// (g < packed_tiles(N)/G, s < H/32, j < G, l < 64, e < 8; rows >= N are zero).
// One thread moves one 16-byte lane slice.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t *__restrict__ W,
                                                           uint16_t *__restrict__ Wp, int K, int N,
                                                           int H, int lgG) {
  const int G = 1 << lgG;
  const int S = H / 32, NG = packed_tiles(N) >> lgG;
  const size_t total = (size_t)K * NG * S * G * 64;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int l = (int)(i % 64);
  size_t f = i / 64;
  const int j = (int)(f & (G - 1));
  f >>= lgG;
  const int s = (int)(f % S);
  f /= S;
  const int g = (int)(f % NG);
  const int k = (int)(f / NG);
  const int n = ((g << lgG) + j) * 16 + (l & 15);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (n < N) v = *reinterpret_cast<const u32x4_t *>(W + ((size_t)k * N + n) * H + s * 32 + (l >> 4) * 8);
  *reinterpret_cast<u32x4_t *>(Wp + i * 8) = v;
}

template <int R, int C, int EPI, bool PACKED, int U, int NW>
medusa_status launch_one(hipStream_t st, const uint16_t *W, const uint16_t *X, long xhs, int K, int N, int H, int M,
                int m0, int Mg, int lgG, const uint16_t *resid, uint16_t *ob, float *of, uint32_t *timg) {
  const int tiles = (N + 16 * R - 1) / (16 * R);
  MEDUSA_LAUNCH("medusa heads", (head_gemm_bf16<R, C, EPI, PACKED, U, NW>), dim3(tiles * K), dim3(64 * NW), 0, st, W, X, xhs,
                     N, H, M, m0, Mg, tiles, lgG, resid, ob, of, timg);
  return MEDUSA_OK;
}

// Tiling by shape (measured on MI355X).  Vocabulary projection (N = V, many
// tiles): up to 4 rows, one row tile per wave with 16 k-steps in flight;
// 5-8 rows, two row tiles per wave; 9-32 rows, eight row tiles per wave share
// every activation fragment (it is the activation loads, not the weight
// stream, that limit these), with two waves splitting the reduction.
// ResBlock (N = H, few tiles): more waves per block split the reduction so
// enough loads are in flight (16 waves x 4 k-steps for up to 4 rows, 8 waves
// up to 8 rows, and for 9-32 rows 8 waves of four row tiles sharing each
// activation fragment; at 16 rows that took the 7B ResBlock from 26.4 to
// 22.3 us, at 5 rows it would be slower).
template <int EPI, bool PACKED>
medusa_status launch_bf16(hipStream_t st, const uint16_t *W, const uint16_t *X, long xhs, int K,
                          int N, int H, int M, int lgG, const uint16_t *resid, uint16_t *ob, float *of,
                          uint32_t *timg = nullptr) {
  if (M >= kManyRows) return head_gemm_many_rows<EPI, PACKED>(st, W, X, xhs, K, N, H, M, lgG, resid, ob, of);
  const int m0 = 0, Mg = M;   // one group: the weights are streamed once
  medusa_status s;
  if (EPI == EPI_RESBLOCK && Mg <= 4 && H % (32 * 16) == 0)
    s = launch_one<1, 1, EPI, PACKED, 4, 16>(st, W, X, xhs, K, N, H, M, m0, Mg, lgG, resid, ob, of, timg);
  else if (EPI == EPI_RESBLOCK && Mg <= 8 && H % (32 * 8) == 0)
    s = launch_one<1, 1, EPI, PACKED, 4, 8>(st, W, X, xhs, K, N, H, M, m0, Mg, lgG, resid, ob, of, timg);
  else if (EPI == EPI_RESBLOCK && Mg <= 16 && H % (32 * 8) == 0)
    s = launch_one<4, 1, EPI, PACKED, 2, 8>(st, W, X, xhs, K, N, H, M, m0, Mg, lgG, resid, ob, of, timg);
  else if (Mg <= 4 && (H / kWaves / 32) % 16 == 0)
    s = launch_one<1, 1, EPI, PACKED, 16, 4>(st, W, X, xhs, K, N, H, M, m0, Mg, lgG, resid, ob, of, timg);
  else if (Mg <= 4)
    s = launch_one<1, 1, EPI, PACKED, 8, 4>(st, W, X, xhs, K, N, H, M, m0, Mg, lgG, resid, ob, of, timg);
  else if (EPI == EPI_LOGITS && Mg > 8 && Mg <= 16)
    s = launch_one<8, 1, EPI, PACKED, 2, 2>(st, W, X, xhs, K, N, H, M, m0, Mg, lgG, resid, ob, of, timg);
  else if (EPI == EPI_LOGITS && Mg > 16)
    s = launch_one<8, 2, EPI, PACKED, 2, 2>(st, W, X, xhs, K, N, H, M, m0, Mg, lgG, resid, ob, of, timg);
  else if (Mg <= 16)
    s = launch_one<2, 1, EPI, PACKED, 8, 4>(st, W, X, xhs, K, N, H, M, m0, Mg, lgG, resid, ob, of, timg);
  else if (H % (32 * 8) == 0)
    s = launch_one<4, 2, EPI, PACKED, 2, 8>(st, W, X, xhs, K, N, H, M, m0, Mg, lgG, resid, ob, of, timg);
  else
    s = launch_one<2, 2, EPI, PACKED, 8, 4>(st, W, X, xhs, K, N, H, M, m0, Mg, lgG, resid, ob, of, timg);
  if (s != MEDUSA_OK) return s;
  return check_launch(EPI == EPI_LOGITS ? "medusa_head_vocab" : "medusa_head_resblock");
}

template <int EPI>
medusa_status launch_f32(hipStream_t st, const float *W, const float *X, long xhs, int K, int N,
                         int H, int M, const float *resid, float *out) {
  const long waves = (long)K * N * ((M + 7) / 8);
  const dim3 grid((unsigned)((waves + 3) / 4));
  MEDUSA_LAUNCH("medusa heads", (head_gemm_f32<EPI>), grid, dim3(256), 0, st, W, X, xhs, K, N, H, M, resid, out);
  return check_launch(EPI == EPI_LOGITS ? "medusa_head_vocab" : "medusa_head_resblock");
}

medusa_status check_common(const char *who, medusa_dtype dt, int K, int M, int H) {
  if (dt != MEDUSA_F32 && dt != MEDUSA_BF16) return fail(MEDUSA_ERR_ARG, "%s: unknown dtype %d", who, (int)dt);
  if (K < 1 || M < 1 || H < 1) return fail(MEDUSA_ERR_ARG, "%s: K=%d M=%d H=%d must be >= 1", who, K, M, H);
  if (dt == MEDUSA_BF16 && H % 128 != 0)
    return fail(MEDUSA_ERR_UNSUPPORTED, "%s: bf16 needs H %% 128 == 0 (H=%d)", who, H);
  if (dt == MEDUSA_F32 && H % 4 != 0)
    return fail(MEDUSA_ERR_UNSUPPORTED, "%s: f32 needs H %% 4 == 0 (H=%d)", who, H);
  return MEDUSA_OK;
}

}  // namespace

extern "C" medusa_status medusa_head_resblock(medusa_stream_t stream, medusa_dtype dt, int K, int M,
                                              int H, const void *h, const void *W1, void *r) {
  TraceRange tr("medusa_head_resblock");
  medusa_status s = check_common("medusa_head_resblock", dt, K, M, H);
  if (s != MEDUSA_OK) return s;
  if (!h || !W1 || !r) return fail(MEDUSA_ERR_ARG, "medusa_head_resblock: NULL pointer");
  if (!aligned16(h) || !aligned16(W1) || !aligned16(r))
    return fail(MEDUSA_ERR_ARG, "medusa_head_resblock: pointers must be 16-byte aligned");
  hipStream_t st = as_stream(stream);
  if (dt == MEDUSA_BF16)
    return launch_bf16<EPI_RESBLOCK, false>(st, static_cast<const uint16_t *>(W1), static_cast<const uint16_t *>(h),
                                     0, K, H, H, M, 0, static_cast<const uint16_t *>(h),
                                     static_cast<uint16_t *>(r), nullptr);
  return launch_f32<EPI_RESBLOCK>(st, static_cast<const float *>(W1), static_cast<const float *>(h), 0,
                                  K, H, H, M, static_cast<const float *>(h), static_cast<float *>(r));
}

extern "C" medusa_status medusa_head_vocab(medusa_stream_t stream, medusa_dtype dt, int K, int M,
                                           int H, int V, const void *r, const void *W2,
                                           float *logits) {
  TraceRange tr("medusa_head_vocab");
  medusa_status s = check_common("medusa_head_vocab", dt, K, M, H);
  if (s != MEDUSA_OK) return s;
  if (V < 1) return fail(MEDUSA_ERR_ARG, "medusa_head_vocab: V=%d", V);
  if (!r || !W2 || !logits) return fail(MEDUSA_ERR_ARG, "medusa_head_vocab: NULL pointer");
  if (!aligned16(r) || !aligned16(W2) || !aligned16(logits))
    return fail(MEDUSA_ERR_ARG, "medusa_head_vocab: pointers must be 16-byte aligned");
  hipStream_t st = as_stream(stream);
  const long xhs = (long)M * H;
  if (dt == MEDUSA_BF16)
    return launch_bf16<EPI_LOGITS, false>(st, static_cast<const uint16_t *>(W2), static_cast<const uint16_t *>(r),
                                   xhs, K, V, H, M, 0, nullptr, nullptr, logits);
  return launch_f32<EPI_LOGITS>(st, static_cast<const float *>(W2), static_cast<const float *>(r), xhs,
                                K, V, H, M, nullptr, logits);
}

extern "C" medusa_status medusa_heads(medusa_stream_t stream, medusa_dtype dt, int K, int M, int H,
                                      int V, const void *h, const void *W1, const void *W2, void *r,
                                      float *logits) {
  TraceRange tr("medusa_heads");
  medusa_status s = check_common("medusa_heads", dt, K, M, H);
  if (s != MEDUSA_OK) return s;
  if (V < 1) return fail(MEDUSA_ERR_ARG, "medusa_heads: V=%d", V);
  if (!h || !W1 || !W2 || !r || !logits) return fail(MEDUSA_ERR_ARG, "medusa_heads: NULL pointer");
  if (!aligned16(h) || !aligned16(W1) || !aligned16(W2) || !aligned16(r) || !aligned16(logits))
    return fail(MEDUSA_ERR_ARG, "medusa_heads: pointers must be 16-byte aligned");
  s = medusa_head_resblock(stream, dt, K, M, H, h, W1, r);
  if (s != MEDUSA_OK) return s;
  return medusa_head_vocab(stream, dt, K, M, H, V, r, W2, logits);
}

// ---------------------------------------------------------------------------
// packed-weight entry points (bf16)
extern "C" size_t medusa_packed_weight_bytes(int K, int N, int H) {
  if (K < 1 || N < 1 || H < 32 || H % 32 != 0) return 0;
  return (size_t)K * packed_tiles(N) * (H / 32) * 512 * sizeof(uint16_t);
}

// log2 of a packed layout's tile group, or -1 if the group is not 1, 2, 4 or 8
static int group_log2(int group) {
  switch (group) {
    case 1: return 0;
    case 2: return 1;
    case 4: return 2;
    case 8: return 3;
  }
  return -1;
}

extern "C" int medusa_pack_group_for_rows(int M) { return M <= 8 ? 1 : kPackGroupMax; }

extern "C" medusa_status medusa_pack_weights(medusa_stream_t stream, int K, int N, int H, int group,
                                             const void *W, void *Wp) {
  TraceRange tr("medusa_pack_weights");
  if (K < 1 || N < 1 || H < 1) return fail(MEDUSA_ERR_ARG, "medusa_pack_weights: K=%d N=%d H=%d", K, N, H);
  const int lgG = group_log2(group);
  if (lgG < 0) return fail(MEDUSA_ERR_ARG, "medusa_pack_weights: group=%d not in {1, 2, 4, 8}", group);
  if (H % 128 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "medusa_pack_weights: needs H %% 128 == 0 (H=%d)", H);
  if (!W || !Wp) return fail(MEDUSA_ERR_ARG, "medusa_pack_weights: NULL pointer");
  if (!aligned16(W) || !aligned16(Wp)) return fail(MEDUSA_ERR_ARG, "medusa_pack_weights: pointers must be 16-byte aligned");
  const size_t lanes = medusa_packed_weight_bytes(K, N, H) / 16;
  MEDUSA_LAUNCH("medusa heads", pack_weights_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, as_stream(stream),
                     static_cast<const uint16_t *>(W), static_cast<uint16_t *>(Wp), K, N, H, lgG);
  return check_launch("medusa_pack_weights");
}

extern "C" medusa_status medusa_head_resblock_packed(medusa_stream_t stream, int K, int M, int H, int group,
                                                     const void *h, const void *W1p, void *r) {
  TraceRange tr("medusa_head_resblock_packed");
  medusa_status s = check_common("medusa_head_resblock_packed", MEDUSA_BF16, K, M, H);
  if (s != MEDUSA_OK) return s;
  const int lgG = group_log2(group);
  if (lgG < 0) return fail(MEDUSA_ERR_ARG, "medusa_head_resblock_packed: group=%d not in {1, 2, 4, 8}", group);
  if (!h || !W1p || !r) return fail(MEDUSA_ERR_ARG, "medusa_head_resblock_packed: NULL pointer");
  if (!aligned16(h) || !aligned16(W1p) || !aligned16(r))
    return fail(MEDUSA_ERR_ARG, "medusa_head_resblock_packed: pointers must be 16-byte aligned");
  return launch_bf16<EPI_RESBLOCK, true>(as_stream(stream), static_cast<const uint16_t *>(W1p),
                                         static_cast<const uint16_t *>(h), 0, K, H, H, M, lgG,
                                         static_cast<const uint16_t *>(h), static_cast<uint16_t *>(r), nullptr);
}

extern "C" medusa_status medusa_head_vocab_packed(medusa_stream_t stream, int K, int M, int H, int V, int group,
                                                  const void *r, const void *W2p, float *logits) {
  TraceRange tr("medusa_head_vocab_packed");
  medusa_status s = check_common("medusa_head_vocab_packed", MEDUSA_BF16, K, M, H);
  if (s != MEDUSA_OK) return s;
  const int lgG = group_log2(group);
  if (lgG < 0) return fail(MEDUSA_ERR_ARG, "medusa_head_vocab_packed: group=%d not in {1, 2, 4, 8}", group);
  if (V < 1) return fail(MEDUSA_ERR_ARG, "medusa_head_vocab_packed: V=%d", V);
  if (!r || !W2p || !logits) return fail(MEDUSA_ERR_ARG, "medusa_head_vocab_packed: NULL pointer");
  if (!aligned16(r) || !aligned16(W2p) || !aligned16(logits))
    return fail(MEDUSA_ERR_ARG, "medusa_head_vocab_packed: pointers must be 16-byte aligned");
  return launch_bf16<EPI_LOGITS, true>(as_stream(stream), static_cast<const uint16_t *>(W2p),
                                       static_cast<const uint16_t *>(r), (long)M * H, K, V, H, M, lgG, nullptr,
                                       nullptr, logits);
}

extern "C" medusa_status medusa_head_vocab_packed_tmax(medusa_stream_t stream, int K, int M, int H, int V,
                                                       int group, const void *r, const void *W2p, float *logits,
                                                       uint32_t *tile_max) {
  TraceRange tr("medusa_head_vocab_packed_tmax");
  medusa_status s = check_common("medusa_head_vocab_packed_tmax", MEDUSA_BF16, K, M, H);
  if (s != MEDUSA_OK) return s;
  const int lgG = group_log2(group);
  if (lgG < 0) return fail(MEDUSA_ERR_ARG, "medusa_head_vocab_packed_tmax: group=%d not in {1, 2, 4, 8}", group);
  if (V < 1) return fail(MEDUSA_ERR_ARG, "medusa_head_vocab_packed_tmax: V=%d", V);
  if (M > MEDUSA_MAX_HEADS_M)
    return fail(MEDUSA_ERR_UNSUPPORTED, "medusa_head_vocab_packed_tmax: M=%d > %d", M, MEDUSA_MAX_HEADS_M);
  if (!r || !W2p || !logits || !tile_max) return fail(MEDUSA_ERR_ARG, "medusa_head_vocab_packed_tmax: NULL pointer");
  if (!aligned16(r) || !aligned16(W2p) || !aligned16(logits) || (reinterpret_cast<uintptr_t>(tile_max) & 3u))
    return fail(MEDUSA_ERR_ARG, "medusa_head_vocab_packed_tmax: misaligned pointer");
  return launch_bf16<EPI_LOGITS, true>(as_stream(stream), static_cast<const uint16_t *>(W2p),
                                       static_cast<const uint16_t *>(r), (long)M * H, K, V, H, M, lgG, nullptr,
                                       nullptr, logits, tile_max);
}

// Workspace variants: from kFragmentRows rows the activations are first
// packed into the workspace in fragment order, then both operands stream as
// whole 1 KiB fragments (head_gemm_fragments); below that they run the calls
// above unchanged (the workspace is not touched).  Results are bit-identical
// to the calls above: the same products summed in the same order.
extern "C" size_t medusa_head_workspace(int K, int M, int H) {
  if (K < 1 || M < kFragmentRows || H < 128 || H % 128 != 0) return 0;
  return packed_rows_bytes(K, M, H);
}

static medusa_status check_ws(const char *who, int K, int M, int H, const void *ws, size_t ws_bytes) {
  const size_t need = medusa_head_workspace(K, M, H);
  if (ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
  if (!ws) return fail(MEDUSA_ERR_ARG, "%s: NULL workspace", who);
  if (!aligned16(ws)) return fail(MEDUSA_ERR_ARG, "%s: workspace must be 16-byte aligned", who);
  return MEDUSA_OK;
}

extern "C" medusa_status medusa_head_resblock_packed_ws(medusa_stream_t stream, int K, int M, int H, int group,
                                                        const void *h, const void *W1p, void *r, void *ws,
                                                        size_t ws_bytes) {
  TraceRange tr("medusa_head_resblock_packed_ws");
  if (M < kFragmentRows || H % 128 != 0) return medusa_head_resblock_packed(stream, K, M, H, group, h, W1p, r);
  const char *who = "medusa_head_resblock_packed_ws";
  medusa_status s = check_common(who, MEDUSA_BF16, K, M, H);
  if (s != MEDUSA_OK) return s;
  const int lgG = group_log2(group);
  if (lgG < 0) return fail(MEDUSA_ERR_ARG, "%s: group=%d not in {1, 2, 4, 8}", who, group);
  if (!h || !W1p || !r) return fail(MEDUSA_ERR_ARG, "%s: NULL pointer", who);
  if (!aligned16(h) || !aligned16(W1p) || !aligned16(r))
    return fail(MEDUSA_ERR_ARG, "%s: pointers must be 16-byte aligned", who);
  if ((s = check_ws(who, K, M, H, ws, ws_bytes)) != MEDUSA_OK) return s;
  if ((s = fragments_supported(K, H, H, M)) != MEDUSA_OK) return s;      // before anything is enqueued
  hipStream_t st = as_stream(stream);
  const uint16_t *hb = static_cast<const uint16_t *>(h);
  uint16_t *hp = static_cast<uint16_t *>(ws);
  if ((s = pack_rows(st, hb, 0, 1, M, H, hp)) != MEDUSA_OK) return s;   // one h shared by every head
  return head_gemm_fragments<kEpiResblock>(st, static_cast<const uint16_t *>(W1p), hp, 1, K, H, H, M, lgG, hb,
                                           static_cast<uint16_t *>(r), nullptr, nullptr);
}

extern "C" medusa_status medusa_head_vocab_packed_ws(medusa_stream_t stream, int K, int M, int H, int V, int group,
                                                     const void *r, const void *W2p, float *logits, void *ws,
                                                     size_t ws_bytes) {
  TraceRange tr("medusa_head_vocab_packed_ws");
  if (M < kFragmentRows || H % 128 != 0) return medusa_head_vocab_packed(stream, K, M, H, V, group, r, W2p, logits);
  const char *who = "medusa_head_vocab_packed_ws";
  medusa_status s = check_common(who, MEDUSA_BF16, K, M, H);
  if (s != MEDUSA_OK) return s;
  const int lgG = group_log2(group);
  if (lgG < 0) return fail(MEDUSA_ERR_ARG, "%s: group=%d not in {1, 2, 4, 8}", who, group);
  if (V < 1) return fail(MEDUSA_ERR_ARG, "%s: V=%d", who, V);
  if (!r || !W2p || !logits) return fail(MEDUSA_ERR_ARG, "%s: NULL pointer", who);
  if (!aligned16(r) || !aligned16(W2p) || !aligned16(logits))
    return fail(MEDUSA_ERR_ARG, "%s: pointers must be 16-byte aligned", who);
  if ((s = check_ws(who, K, M, H, ws, ws_bytes)) != MEDUSA_OK) return s;
  if ((s = fragments_supported(K, V, H, M)) != MEDUSA_OK) return s;      // before anything is enqueued
  hipStream_t st = as_stream(stream);
  uint16_t *rp = static_cast<uint16_t *>(ws);
  if ((s = pack_rows(st, static_cast<const uint16_t *>(r), (long)M * H, K, M, H, rp)) != MEDUSA_OK) return s;
  return head_gemm_fragments<kEpiLogits>(st, static_cast<const uint16_t *>(W2p), rp, K, K, V, H, M, lgG, nullptr,
                                         nullptr, logits, nullptr);
}

// Both projections in one call: the ResBlock's epilogue writes r row-major
// (the output) and again in fragment order into the workspace, where the
// vocabulary projection reads it, so r is not copied a second time.
extern "C" size_t medusa_heads_workspace(int K, int M, int H) {
  if (K < 1 || M < kFragmentRows || H < 128 || H % 128 != 0) return 0;
  return packed_rows_bytes(K + 1, M, H);   // packed h, then packed r of the K heads
}

extern "C" medusa_status medusa_heads_packed_ws(medusa_stream_t stream, int K, int M, int H, int V, int group,
                                                const void *h, const void *W1p, const void *W2p, void *r,
                                                float *logits, void *ws, size_t ws_bytes) {
  TraceRange tr("medusa_heads_packed_ws");
  if (M < kFragmentRows || H % 128 != 0)
    return medusa_heads_packed(stream, K, M, H, V, group, h, W1p, W2p, r, logits);
  const char *who = "medusa_heads_packed_ws";
  medusa_status s = check_common(who, MEDUSA_BF16, K, M, H);
  if (s != MEDUSA_OK) return s;
  const int lgG = group_log2(group);
  if (lgG < 0) return fail(MEDUSA_ERR_ARG, "%s: group=%d not in {1, 2, 4, 8}", who, group);
  if (V < 1) return fail(MEDUSA_ERR_ARG, "%s: V=%d", who, V);
  if (!h || !W1p || !W2p || !r || !logits) return fail(MEDUSA_ERR_ARG, "%s: NULL pointer", who);
  if (!aligned16(h) || !aligned16(W1p) || !aligned16(W2p) || !aligned16(r) || !aligned16(logits))
    return fail(MEDUSA_ERR_ARG, "%s: pointers must be 16-byte aligned", who);
  const size_t need = medusa_heads_workspace(K, M, H);
  if (ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
  if (!ws) return fail(MEDUSA_ERR_ARG, "%s: NULL workspace", who);
  if (!aligned16(ws)) return fail(MEDUSA_ERR_ARG, "%s: workspace must be 16-byte aligned", who);
  // both contractions' limits before anything is enqueued
  if ((s = fragments_supported(K, H, H, M)) != MEDUSA_OK || (s = fragments_supported(K, V, H, M)) != MEDUSA_OK)
    return s;
  hipStream_t st = as_stream(stream);
  const uint16_t *hb = static_cast<const uint16_t *>(h);
  uint16_t *hp = static_cast<uint16_t *>(ws);
  uint16_t *rp = hp + packed_rows_bytes(1, M, H) / sizeof(uint16_t);
  if ((s = pack_rows(st, hb, 0, 1, M, H, hp)) != MEDUSA_OK) return s;
  if ((s = head_gemm_fragments<kEpiResblock>(st, static_cast<const uint16_t *>(W1p), hp, 1, K, H, H, M, lgG, hb,
                                             static_cast<uint16_t *>(r), nullptr, rp)) != MEDUSA_OK)
    return s;
  return head_gemm_fragments<kEpiLogits>(st, static_cast<const uint16_t *>(W2p), rp, K, K, V, H, M, lgG, nullptr,
                                         nullptr, logits, nullptr);
}

extern "C" medusa_status medusa_heads_packed(medusa_stream_t stream, int K, int M, int H, int V, int group,
                                             const void *h, const void *W1p, const void *W2p, void *r,
                                             float *logits) {
  TraceRange tr("medusa_heads_packed");
  medusa_status s = check_common("medusa_heads_packed", MEDUSA_BF16, K, M, H);
  if (s != MEDUSA_OK) return s;
  if (V < 1) return fail(MEDUSA_ERR_ARG, "medusa_heads_packed: V=%d", V);
  if (!h || !W1p || !W2p || !r || !logits) return fail(MEDUSA_ERR_ARG, "medusa_heads_packed: NULL pointer");
  if (!aligned16(h) || !aligned16(W1p) || !aligned16(W2p) || !aligned16(r) || !aligned16(logits))
    return fail(MEDUSA_ERR_ARG, "medusa_heads_packed: pointers must be 16-byte aligned");
  s = medusa_head_resblock_packed(stream, K, M, H, group, h, W1p, r);
  if (s != MEDUSA_OK) return s;
  return medusa_head_vocab_packed(stream, K, M, H, V, group, r, W2p, logits);
}
