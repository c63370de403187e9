// Medusa heads: r = h + SiLU(W1_k h) and logits = W2_k r.
//
// At decode time the heads see one row per sequence (M <= 32), so both
// projections are skinny GEMMs whose cost is streaming W1 / W2 from HBM once.
// bf16 path: each wave owns 16*R output rows and a quarter of the reduction;
// the weight slab is the MFMA A operand (v_mfma_f32_16x16x32_bf16, lane l
// holds row l%16, reduction slice 8*(l/16)..+7), activations are the B
// operand (M padded to 16*C columns), partial sums of the 4 waves are added in
// LDS and the epilogue (SiLU + residual + bf16 rounding, or fp32 store) is
// fused.  Weights are read with non-temporal loads so the small activation
// block stays resident in L2.
#include "common.h"

using namespace medusa;

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kUnroll = 8;  // k-steps of 32 in flight per wave

enum { EPI_RESBLOCK = 0, EPI_LOGITS = 1 };

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// out[head][m0+m][n] = sum_i W[head][n][i] * X[head][m0+m][i]   (m < Mg <= 16*C)
template <int R, int C, int EPI>
__global__ __launch_bounds__(kThreads) void head_gemm_bf16(
    const uint16_t *__restrict__ W, const uint16_t *__restrict__ X, long x_head_stride, int N,
    int H, int M_total, int m0, int Mg, int tiles_per_head, const uint16_t *__restrict__ resid,
    uint16_t *__restrict__ out_bf16, float *__restrict__ out_f32) {
  __shared__ float red[kWaves][16 * C][16 * R + 1];
  const int head = blockIdx.x / tiles_per_head;
  const int n0 = (blockIdx.x % tiles_per_head) * 16 * R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int kspan = H / kWaves;
  const int k0 = wave * kspan + lg * 8;
  const uint16_t *Wh = W + (size_t)head * N * H;
  const uint16_t *Xh = X + (size_t)head * x_head_stride + (size_t)m0 * H;

  const uint16_t *arow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int n = n0 + r * 16 + lr;
    n = n < N ? n : N - 1;  // ragged tail: read a valid row, result discarded
    arow[r] = Wh + (size_t)n * H + k0;
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
  for (; s + kUnroll <= steps; s += kUnroll) {
    u32x4_t a[kUnroll][R], b[kUnroll][C];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
        a[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(arow[r] + (s + u) * 32));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int c = 0; c < C; ++c)
        b[u][c] = bval[c] ? *reinterpret_cast<const u32x4_t *>(brow[c] + (s + u) * 32) : zero;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[r][c] = mfma(a[u][r], b[u][c], acc[r][c]);
  }
  for (; s < steps; ++s) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(arow[r] + s * 32));
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

  for (int e = threadIdx.x; e < 16 * C * 16 * R; e += kThreads) {
    const int m = e / (16 * R), nl = e % (16 * R);
    const int n = n0 + nl;
    if (m >= Mg || n >= N) continue;
    const float v = red[0][m][nl] + red[1][m][nl] + red[2][m][nl] + red[3][m][nl];
    const size_t o = ((size_t)head * M_total + m0 + m) * N + n;
    if (EPI == EPI_LOGITS) {
      out_f32[o] = v;
    } else {
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

template <int EPI>
medusa_status launch_bf16(hipStream_t st, const uint16_t *W, const uint16_t *X, long xhs, int K,
                          int N, int H, int M, const uint16_t *resid, uint16_t *ob, float *of) {
  constexpr int R = EPI == EPI_LOGITS ? 2 : 1;
  const int tiles = (N + 16 * R - 1) / (16 * R);
  const dim3 grid(tiles * K);
  for (int m0 = 0; m0 < M; m0 += MEDUSA_MAX_HEADS_M) {
    const int Mg = M - m0 < MEDUSA_MAX_HEADS_M ? M - m0 : MEDUSA_MAX_HEADS_M;
    if (Mg <= 16)
      hipLaunchKernelGGL((head_gemm_bf16<R, 1, EPI>), grid, dim3(kThreads), 0, st, W, X, xhs, N, H,
                         M, m0, Mg, tiles, resid, ob, of);
    else
      hipLaunchKernelGGL((head_gemm_bf16<R, 2, EPI>), grid, dim3(kThreads), 0, st, W, X, xhs, N, H,
                         M, m0, Mg, tiles, resid, ob, of);
    medusa_status s = check_launch(EPI == EPI_LOGITS ? "medusa_head_vocab" : "medusa_head_resblock");
    if (s != MEDUSA_OK) return s;
  }
  return MEDUSA_OK;
}

template <int EPI>
medusa_status launch_f32(hipStream_t st, const float *W, const float *X, long xhs, int K, int N,
                         int H, int M, const float *resid, float *out) {
  const long waves = (long)K * N * ((M + 7) / 8);
  const dim3 grid((unsigned)((waves + 3) / 4));
  hipLaunchKernelGGL((head_gemm_f32<EPI>), grid, dim3(256), 0, st, W, X, xhs, K, N, H, M, resid, out);
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
  medusa_status s = check_common("medusa_head_resblock", dt, K, M, H);
  if (s != MEDUSA_OK) return s;
  if (!h || !W1 || !r) return fail(MEDUSA_ERR_ARG, "medusa_head_resblock: NULL pointer");
  if (!aligned16(h) || !aligned16(W1) || !aligned16(r))
    return fail(MEDUSA_ERR_ARG, "medusa_head_resblock: pointers must be 16-byte aligned");
  hipStream_t st = as_stream(stream);
  if (dt == MEDUSA_BF16)
    return launch_bf16<EPI_RESBLOCK>(st, static_cast<const uint16_t *>(W1), static_cast<const uint16_t *>(h),
                                     0, K, H, H, M, static_cast<const uint16_t *>(h),
                                     static_cast<uint16_t *>(r), nullptr);
  return launch_f32<EPI_RESBLOCK>(st, static_cast<const float *>(W1), static_cast<const float *>(h), 0,
                                  K, H, H, M, static_cast<const float *>(h), static_cast<float *>(r));
}

extern "C" medusa_status medusa_head_vocab(medusa_stream_t stream, medusa_dtype dt, int K, int M,
                                           int H, int V, const void *r, const void *W2,
                                           float *logits) {
  medusa_status s = check_common("medusa_head_vocab", dt, K, M, H);
  if (s != MEDUSA_OK) return s;
  if (V < 1) return fail(MEDUSA_ERR_ARG, "medusa_head_vocab: V=%d", V);
  if (!r || !W2 || !logits) return fail(MEDUSA_ERR_ARG, "medusa_head_vocab: NULL pointer");
  if (!aligned16(r) || !aligned16(W2) || !aligned16(logits))
    return fail(MEDUSA_ERR_ARG, "medusa_head_vocab: pointers must be 16-byte aligned");
  hipStream_t st = as_stream(stream);
  const long xhs = (long)M * H;
  if (dt == MEDUSA_BF16)
    return launch_bf16<EPI_LOGITS>(st, static_cast<const uint16_t *>(W2), static_cast<const uint16_t *>(r),
                                   xhs, K, V, H, M, nullptr, nullptr, logits);
  return launch_f32<EPI_LOGITS>(st, static_cast<const float *>(W2), static_cast<const float *>(r), xhs,
                                K, V, H, M, nullptr, logits);
}

extern "C" medusa_status medusa_heads(medusa_stream_t stream, medusa_dtype dt, int K, int M, int H,
                                      int V, const void *h, const void *W1, const void *W2, void *r,
                                      float *logits) {
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
