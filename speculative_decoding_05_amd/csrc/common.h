// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "medusa.h"
#include "tree.h"

namespace medusa {

medusa_status check_launch(const char *what);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hipStream_t as_stream(medusa_stream_t s) { return reinterpret_cast<hipStream_t>(s); }
medusa_status check_tree_on_device(const medusa_tree *t);
// Debug facilities (environment variables, see debug.hip).
bool fault_injected();    // MEDUSA_FAULT=launch: every launch fails before it is enqueued
bool validate_enabled();  // MEDUSA_VALIDATE=1: device checks of the inputs before the kernels
class TraceRange {        // MEDUSA_TRACE=1: roctx range for the lifetime of the object
 public:
  explicit TraceRange(const char *name);
  ~TraceRange();
  TraceRange(const TraceRange &) = delete;
  TraceRange &operator=(const TraceRange &) = delete;

 private:
  bool on_ = false;
};
// What validate mode checks: up to two float arrays (NaN, and +inf where
// posinf_bad, is an error) and one int32 token array (ids outside [0, V)).
struct ValidateSpec {
  const float *a = nullptr;
  size_t na = 0;
  const float *b = nullptr;
  size_t nb = 0;
  bool posinf_bad = false;
  const int32_t *tok = nullptr;
  size_t nt = 0;
  int V = 0;
};
// Runs the checks on `st` and waits for them; ERR_NONFINITE / ERR_ARG on a
// finding, ERR_STATE under graph capture.
medusa_status validate_inputs(hipStream_t st, const char *who, const ValidateSpec &v);

// compute units of the current device (queried once per device; 256 if the
// query fails)
int device_compute_units();

// bf16 helpers (bit patterns held in uint16)
__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}
__host__ __device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // nan
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Launch-wide XCD-aware block index: the hardware deals consecutive block ids
// round-robin over the 8 XCDs; remapping makes consecutive *logical* ids land
// on one XCD so that blocks sharing data share that XCD's L2.
__device__ inline int xcd_remap(int bid, int nblocks) {
  const int n8 = nblocks / 8;
  if (bid >= n8 * 8) return bid;
  return (bid % 8) * n8 + bid / 8;
}


// ---------------------------------------------------------------------------
// Wave reductions without LDS: four DPP steps combine the 16 lanes of each row
// (partners lane^1, lane^2, then the half-row and row mirrors), after which
// every lane holds its row's result; readlane fetches the four row results.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(uint32_t, v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  return (static_cast<uint64_t>(dpp<CTRL>(static_cast<uint32_t>(v >> 32))) << 32) | dpp<CTRL>(static_cast<uint32_t>(v));
}
__device__ __forceinline__ uint32_t readlane(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}
__device__ __forceinline__ float readlanef(float v, int lane) {
  return __builtin_bit_cast(float, readlane(__builtin_bit_cast(uint32_t, v), lane));
}

// max over the 16 lanes of each row (result in every lane of the row)
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp64<kDppXor1>(v); v = o > v ? o : v;
  o = dpp64<kDppXor2>(v); v = o > v ? o : v;
  o = dpp64<kDppHalfMirror>(v); v = o > v ? o : v;
  o = dpp64<kDppMirror>(v); v = o > v ? o : v;
  return v;
}
// Buffer resource word 3 on gfx9 for raw 32-bit loads.  A raw buffer load
// whose byte offset (in the vector register) is at or past the resource's size
// returns 0 without touching memory, so bounds checks need no branch.
constexpr int kBufferWord3 = 0x00020000;

// max over the 16 lanes of each row (result in every lane of the row)
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  uint32_t o;
  o = dpp<kDppXor1>(v); v = o > v ? o : v;
  o = dpp<kDppXor2>(v); v = o > v ? o : v;
  o = dpp<kDppHalfMirror>(v); v = o > v ? o : v;
  o = dpp<kDppMirror>(v); v = o > v ? o : v;
  return v;
}

// Order-preserving 32-bit image of a float, -0.0 folded onto +0.0: for
// non-NaN a, b, a > b exactly when image(a) > image(b).  Positive NaNs map
// above +inf, negative NaNs below -inf (the all-ones pattern to 0).
__device__ __forceinline__ uint32_t order_image(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t o;
  o = dpp<kDppXor1>(v); v = o > v ? o : v;
  o = dpp<kDppXor2>(v); v = o > v ? o : v;
  o = dpp<kDppHalfMirror>(v); v = o > v ? o : v;
  o = dpp<kDppMirror>(v); v = o > v ? o : v;
  const uint32_t a = readlane(v, 0), b = readlane(v, 16), c = readlane(v, 32), d = readlane(v, 48);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

}  // namespace medusa

// Launch through the fault gate: with MEDUSA_FAULT=launch the enclosing call
// returns MEDUSA_ERR_HIP before anything is enqueued.
#define MEDUSA_LAUNCH(who, ...)                                                                   \
  do {                                                                                            \
    if (medusa::fault_injected())                                                                 \
      return medusa::fail(MEDUSA_ERR_HIP, "%s: injected launch failure (MEDUSA_FAULT=launch)", who); \
    hipLaunchKernelGGL(__VA_ARGS__);                                                              \
  } while (0)
