// Achievable peaks of the two roofs the step is measured against, run in the
// same process as the measurement: a read-only stream over a large buffer
// (HBM bandwidth; the vocabulary projection, attention and acceptance are
// bound by it) and a loop of independent bf16 matrix-core products (the
// verify-pass contractions and the dense-tree attention are bound by it).
#include "common.h"

using namespace medusa;

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;       // 16-byte loads in flight per thread
constexpr int kMfmaThreads = 256;    // one wave per SIMD
constexpr int kMfmaChains = 4;       // independent accumulators per wave

// Each thread reads kReadUnroll 16-byte chunks, strided by the block size so
// every load instruction of a wave covers 1 KiB of consecutive bytes, with the
// non-temporal hint; the XOR of everything read decides a store that the data
// never triggers, so no load can be dropped.
__global__ __launch_bounds__(kReadThreads) void peak_read_kernel(const u32x4_t *__restrict__ p, size_t n16,
                                                                 uint32_t magic, uint32_t *__restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * kReadThreads * kReadUnroll + threadIdx.x;
  u32x4_t v[kReadUnroll];
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) {
    const size_t i = base + (size_t)u * kReadThreads;
    v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4_t{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0u;
#pragma unroll
  for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == magic) sink[threadIdx.x & 3] = acc;
}

// kMfmaChains independent v_mfma_f32_32x32x16_bf16 chains per wave, `iters`
// rounds; operands depend on a run-time seed, and the sum of the results
// decides a store that never happens for finite seeds.  (The 32x32 form:
// measured on MI355X it keeps the matrix cores ~95 % busy with two chains,
// while the compiler's allocation of 16x16x32 accumulators in a loop like
// this one moves them between registers every trip and halves the rate.)
__global__ __launch_bounds__(kMfmaThreads) void peak_mfma_kernel(int iters, float seed, float *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(seed * (lane + e + 1) * 1e-3f);
    b[e] = static_cast<__bf16>(seed * (lane - e) * 1e-3f);
  }
  f32x16_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  if (s == INFINITY) sink[lane & 3] = s;
}

}  // namespace

extern "C" medusa_status medusa_peak_hbm_read(medusa_stream_t stream, const void *buf, size_t bytes, uint32_t *sink) {
  TraceRange tr("medusa_peak_hbm_read");
  if (!buf || !sink || bytes < 16) return fail(MEDUSA_ERR_ARG, "medusa_peak_hbm_read: NULL pointer or empty buffer");
  if (!aligned16(buf) || !aligned16(sink)) return fail(MEDUSA_ERR_ARG, "medusa_peak_hbm_read: pointers must be 16-byte aligned");
  const size_t n16 = bytes / 16;
  const size_t per_block = (size_t)kReadThreads * kReadUnroll;
  const size_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > 0x7fffffffu) return fail(MEDUSA_ERR_UNSUPPORTED, "medusa_peak_hbm_read: buffer too large");
  MEDUSA_LAUNCH("medusa_peak_hbm_read", peak_read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0,
                as_stream(stream), static_cast<const u32x4_t *>(buf), n16, 0x9e3779b9u, sink);
  return check_launch("medusa_peak_hbm_read");
}

extern "C" double medusa_peak_mfma_flops(int blocks, int iters) {
  if (blocks < 1 || iters < 1) return 0.0;
  return (double)blocks * (kMfmaThreads / 64) * kMfmaChains * iters * (2.0 * 32 * 32 * 16);
}

extern "C" medusa_status medusa_peak_mfma_bf16(medusa_stream_t stream, int blocks, int iters, float *sink) {
  TraceRange tr("medusa_peak_mfma_bf16");
  if (!sink || blocks < 1 || iters < 1) return fail(MEDUSA_ERR_ARG, "medusa_peak_mfma_bf16: blocks=%d iters=%d", blocks, iters);
  if (!aligned16(sink)) return fail(MEDUSA_ERR_ARG, "medusa_peak_mfma_bf16: sink must be 16-byte aligned");
  MEDUSA_LAUNCH("medusa_peak_mfma_bf16", peak_mfma_kernel, dim3((unsigned)blocks), dim3(kMfmaThreads), 0,
                as_stream(stream), iters, 1.0f, sink);
  return check_launch("medusa_peak_mfma_bf16");
}

extern "C" medusa_status medusa_device_info(int *compute_units, int *clock_khz, int *memory_clock_khz) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MEDUSA_ERR_HIP, "medusa_device_info: no HIP device");
  int v = 0;
  if (compute_units) *compute_units = device_compute_units();
  if (clock_khz) *clock_khz = hipDeviceGetAttribute(&v, hipDeviceAttributeClockRate, dev) == hipSuccess ? v : 0;
  if (memory_clock_khz)
    *memory_clock_khz = hipDeviceGetAttribute(&v, hipDeviceAttributeMemoryClockRate, dev) == hipSuccess ? v : 0;
  return MEDUSA_OK;
}
