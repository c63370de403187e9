// Block-tiled bf16 head projection for many rows (gemm.hip).
#pragma once

#include "common.h"

namespace medusa {

enum { kEpiResblock = 0, kEpiLogits = 1 };

// out[head][m][n] = sum_i W[head][n][i] * X[head*xhs + m*H + i], m < M, n < N:
//   kEpiLogits:   of[head][m][n] = the sum (fp32)
//   kEpiResblock: ob[head][m][n] = bf16(resid[m][n] + SiLU(sum))   (N == H)
// W row-major [K][N][H] or packed (medusa_pack_weights).  H % 64 == 0.
template <int EPI, bool PACKED>
medusa_status head_gemm_many_rows(hipStream_t st, const uint16_t *W, const uint16_t *X, long xhs, int K,
                                  int N, int H, int M, const uint16_t *resid, uint16_t *ob, float *of);

// From this many rows the tiled kernel replaces the weight-streaming one (one
// group of MEDUSA_MAX_HEADS_M rows streams the weights once; past that the
// tiled kernel re-uses each weight tile across up to 256 rows).
constexpr int kManyRows = MEDUSA_MAX_HEADS_M + 1;

}  // namespace medusa
