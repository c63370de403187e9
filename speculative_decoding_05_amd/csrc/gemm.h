// Block-tiled bf16 head projection for many rows (gemm.hip).
#pragma once

#include "common.h"

namespace medusa {

enum { kEpiResblock = 0, kEpiLogits = 1 };

// Packed weight layout (medusa_pack_weights).  A fragment is one 16 x 32
// block of W (16 output rows, 32 reduction elements) stored as 1 KiB in MFMA
// lane order: lane l holds row l%16, elements 8(l/16)..+7.  Fragments are
// grouped by G = 2^lgG consecutive row tiles (G = 1, 2, 4 or 8): within a
// head, fragment (tile t, step s) is number ((t/G)*S + s)*G + t%G, S = H/32,
// so the G tiles of a group lie side by side at every step.  G = 1 keeps each
// tile's steps contiguous (fastest to stream one tile per wave, few rows);
// G = 8 gives 8 KiB runs to waves that own 8 tiles (9-32 rows).  Row tiles
// are padded with zeros to a multiple of 8 whatever G is.
constexpr int kPackGroupMax = 8;
__host__ __device__ inline int packed_tiles(int N) {
  return (N + 16 * kPackGroupMax - 1) / (16 * kPackGroupMax) * kPackGroupMax;
}
__host__ __device__ inline size_t packed_fragment(int t, int s, int S, int lgG) {
  return ((((size_t)(t >> lgG)) * S + s) << lgG) + (t & ((1 << lgG) - 1));
}

// out[head][m][n] = sum_i W[head][n][i] * X[head*xhs + m*H + i], m < M, n < N:
//   kEpiLogits:   of[head][m][n] = the sum (fp32)
//   kEpiResblock: ob[head][m][n] = bf16(resid[m][n] + SiLU(sum))   (N == H)
// W row-major [K][N][H] or packed (medusa_pack_weights).  H % 64 == 0.
// lgG: log2 of the packed layout's tile group (packed weights only).
template <int EPI, bool PACKED>
medusa_status head_gemm_many_rows(hipStream_t st, const uint16_t *W, const uint16_t *X, long xhs, int K,
                                  int N, int H, int M, int lgG, const uint16_t *resid, uint16_t *ob, float *of);

// Activations in fragment order (the packed-weight layout with G = 1, applied to
// [K][M][H] rows): K * ceil(M/16) * (H/32) KiB; 0 for invalid sizes.
size_t packed_rows_bytes(int K, int M, int H);
// X [K][M][H] (head stride xhs elements) -> Xp (packed_rows_bytes(K, M, H) bytes)
medusa_status pack_rows(hipStream_t st, const uint16_t *X, long xhs, int K, int M, int H, uint16_t *Xp);
// As head_gemm_many_rows with packed weights, the activations given in fragment
// order: x_heads = 1 shares one packed [M][H] among all heads (the ResBlock's
// h), x_heads = K gives each head its own.  H % 128 == 0.  obp (ResBlock only,
// may be NULL): r written a second time, in fragment order (K heads, as Xp
// of the vocabulary projection; rows >= M of the last row tile not written).
template <int EPI>
medusa_status head_gemm_fragments(hipStream_t st, const uint16_t *Wp, const uint16_t *Xp, int x_heads, int K, int N,
                                  int H, int M, int lgG, const uint16_t *resid, uint16_t *ob, float *of,
                                  uint16_t *obp);
// The shape limits of head_gemm_fragments (H % 128 == 0, each head's packed
// operands under 4 GiB, the grid under 2^31 blocks), checked before anything
// is enqueued: MEDUSA_OK or the error (message set).
medusa_status fragments_supported(int K, int N, int H, int M);
// From this many rows the workspace variants of the packed calls run
// head_gemm_fragments (below it the weight-streaming and 64-row kernels).
constexpr int kFragmentRows = 65;

// From this many rows the tiled kernel replaces the weight-streaming one (one
// group of MEDUSA_MAX_HEADS_M rows streams the weights once; past that the
// tiled kernel re-uses each weight tile across up to 256 rows).
constexpr int kManyRows = MEDUSA_MAX_HEADS_M + 1;

}  // namespace medusa
