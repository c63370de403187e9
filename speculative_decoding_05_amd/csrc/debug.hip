// Debug facilities of the library, all off unless an environment variable
// asks for them:
//   MEDUSA_VALIDATE=1  device checks of the calls' data before their kernels
//                      run (one extra kernel and one stream synchronisation
//                      per call): NaN (and, for acceptance, +inf) logits give
//                      MEDUSA_ERR_NONFINITE, token ids outside [0, V) give
//                      MEDUSA_ERR_ARG; nothing else is enqueued then, so the
//                      outputs are untouched.
//   MEDUSA_FAULT=launch  every kernel launch of the library fails before it
//                      is enqueued with MEDUSA_ERR_HIP (tests of the error
//                      path on a machine whose launches succeed).
//   MEDUSA_TRACE=1     a roctx range named after the call around each device
//                      call (shown by `rocprofv3 --marker-trace`); the roctx
//                      library is opened at run time, so the library does not
//                      depend on it otherwise.
#include <dlfcn.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "common.h"

namespace medusa {

namespace {

bool env_is(const char *name, const char *value) {
  const char *v = getenv(name);
  return v && strcmp(v, value) == 0;
}

// flag bits of the validation kernel
constexpr unsigned kFlagNonfinite = 1u, kFlagToken = 2u;
constexpr int kMaxDevices = 64;

__device__ unsigned int g_validate_flag;

// Grid-stride pass over up to two float arrays and one int32 array: NaN (and
// +inf where posinf_bad) sets kFlagNonfinite, an id outside [0, V) sets
// kFlagToken.  Only vector stores and atomics to the one flag word.
__global__ __launch_bounds__(256) void validate_kernel(const float *__restrict__ a, size_t na,
                                                       const float *__restrict__ b, size_t nb, int posinf_bad,
                                                       const int32_t *__restrict__ tok, size_t nt, int V,
                                                       unsigned int *flag) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned bad = 0u;
  for (size_t i = i0; i < na; i += stride) {
    const float x = a[i];
    if (x != x || (posinf_bad && x == INFINITY)) bad |= kFlagNonfinite;
  }
  for (size_t i = i0; i < nb; i += stride) {
    const float x = b[i];
    if (x != x || (posinf_bad && x == INFINITY)) bad |= kFlagNonfinite;
  }
  for (size_t i = i0; i < nt; i += stride) {
    const int32_t t = tok[i];
    if (t < 0 || t >= V) bad |= kFlagToken;
  }
  if (bad) atomicOr(flag, bad);
}

void *roctx_lib() {
  static void *h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
  return h;
}
typedef int (*push_fn)(const char *);
typedef int (*pop_fn)();

}  // namespace

bool fault_injected() { return env_is("MEDUSA_FAULT", "launch"); }
bool validate_enabled() { return env_is("MEDUSA_VALIDATE", "1"); }

TraceRange::TraceRange(const char *name) {
  static const bool trace = env_is("MEDUSA_TRACE", "1");
  static push_fn push = trace && roctx_lib() ? (push_fn)dlsym(roctx_lib(), "roctxRangePushA") : nullptr;
  on_ = push != nullptr;
  if (on_) push(name);
}

TraceRange::~TraceRange() {
  static pop_fn pop = roctx_lib() ? (pop_fn)dlsym(roctx_lib(), "roctxRangePop") : nullptr;
  if (on_ && pop) pop();
}

medusa_status validate_inputs(hipStream_t st, const char *who, const ValidateSpec &v) {
  // one validation at a time in the process: the flag word is per device
  static std::mutex mu;
  static std::atomic<unsigned int *> flag_of[kMaxDevices];
  std::lock_guard<std::mutex> lock(mu);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
    return fail(MEDUSA_ERR_STATE, "%s: MEDUSA_VALIDATE=1 synchronises the stream and cannot run under graph capture",
                who);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(MEDUSA_ERR_HIP, "%s: validate: no usable HIP device", who);
  unsigned int *flag = flag_of[dev].load();
  if (!flag) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_validate_flag)) != hipSuccess || !p)
      return fail(MEDUSA_ERR_HIP, "%s: validate: flag address not found", who);
    flag = static_cast<unsigned int *>(p);
    flag_of[dev].store(flag);
  }
  if (fault_injected()) return fail(MEDUSA_ERR_HIP, "%s: injected launch failure (MEDUSA_FAULT=launch)", who);
  if (hipMemsetAsync(flag, 0, sizeof(unsigned int), st) != hipSuccess)
    return fail(MEDUSA_ERR_HIP, "%s: validate: clearing the flag failed", who);
  const size_t n = v.na > v.nb ? (v.na > v.nt ? v.na : v.nt) : (v.nb > v.nt ? v.nb : v.nt);
  const size_t blocks_needed = (n + 255) / 256;
  const unsigned blocks = (unsigned)(blocks_needed < 4096 ? (blocks_needed > 0 ? blocks_needed : 1) : 4096);
  hipLaunchKernelGGL(validate_kernel, dim3(blocks), dim3(256), 0, st, v.a, v.na, v.b, v.nb, v.posinf_bad ? 1 : 0,
                     v.tok, v.nt, v.V, flag);
  medusa_status s = check_launch(who);
  if (s != MEDUSA_OK) return s;
  unsigned int host_flag = 0u;
  if (hipMemcpyAsync(&host_flag, flag, sizeof host_flag, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(MEDUSA_ERR_HIP, "%s: validate: reading the flag failed", who);
  if (host_flag & kFlagNonfinite)
    return fail(MEDUSA_ERR_NONFINITE, "%s: logits hold NaN%s (MEDUSA_VALIDATE=1)", who,
                v.posinf_bad ? " or +inf" : "");
  if (host_flag & kFlagToken) return fail(MEDUSA_ERR_ARG, "%s: a token id lies outside [0, %d) (MEDUSA_VALIDATE=1)", who, v.V);
  return MEDUSA_OK;
}

}  // namespace medusa
