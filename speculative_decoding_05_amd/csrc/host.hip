// HIP side of the host code: launch checks, the device's compute-unit count,
// and the candidate tree's device copy (upload and free).  The tree itself is
// built in tree.cpp.  No kernels live here.
#include <algorithm>
#include <atomic>

#include "common.h"

namespace medusa {

medusa_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MEDUSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return MEDUSA_OK;
}

medusa_status check_tree_on_device(const medusa_tree *t) {
  if (!t) return fail(MEDUSA_ERR_ARG, "tree is NULL");
  if (!t->d_base) return fail(MEDUSA_ERR_STATE, "tree has no device copy: call medusa_tree_upload first");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != t->device)
    return fail(MEDUSA_ERR_STATE, "tree was uploaded to device %d, current device is %d", t->device, dev);
  return MEDUSA_OK;
}

int device_compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];  // 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
  cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace medusa

using medusa::fail;


extern "C" medusa_status medusa_tree_upload(medusa_tree *t) {
  if (!t) return fail(MEDUSA_ERR_ARG, "tree_upload: tree is NULL");
  if (t->d_base) return MEDUSA_OK;
  const size_t T = t->T;
  const size_t mask_b = T * t->W * sizeof(uint64_t);
  const size_t ints = 4 * T + t->internal.size() + t->dstart.size() + t->tile_need.size() + t->cstart.size() +
                      t->clist.size();
  const size_t bytes = mask_b + ints * sizeof(int32_t);
  std::vector<unsigned char> img(bytes);
  unsigned char *p = img.data();
  std::copy(reinterpret_cast<const unsigned char *>(t->mask.data()),
            reinterpret_cast<const unsigned char *>(t->mask.data()) + mask_b, p);
  int32_t *q = reinterpret_cast<int32_t *>(p + mask_b);
  std::copy(t->parent.begin(), t->parent.end(), q);
  std::copy(t->depth.begin(), t->depth.end(), q + T);
  std::copy(t->rank.begin(), t->rank.end(), q + 2 * T);
  std::copy(t->slot.begin(), t->slot.end(), q + 3 * T);
  std::copy(t->internal.begin(), t->internal.end(), q + 4 * T);
  std::copy(t->dstart.begin(), t->dstart.end(), q + 4 * T + t->internal.size());
  int32_t *qc = q + 4 * T + t->internal.size() + t->dstart.size();
  std::copy(t->tile_need.begin(), t->tile_need.end(), reinterpret_cast<uint32_t *>(qc));
  qc += t->tile_need.size();
  std::copy(t->cstart.begin(), t->cstart.end(), qc);
  std::copy(t->clist.begin(), t->clist.end(), qc + t->cstart.size());
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MEDUSA_ERR_HIP, "tree_upload: no HIP device");
  void *d = nullptr;
  hipError_t e = hipMalloc(&d, bytes);
  if (e != hipSuccess) return fail(MEDUSA_ERR_HIP, "tree_upload: hipMalloc: %s", hipGetErrorString(e));
  e = hipMemcpy(d, img.data(), bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(d);
    return fail(MEDUSA_ERR_HIP, "tree_upload: hipMemcpy: %s", hipGetErrorString(e));
  }
  t->d_base = d;
  t->device = dev;
  unsigned char *b = static_cast<unsigned char *>(d);
  t->d_mask = reinterpret_cast<const uint64_t *>(b);
  const int32_t *di = reinterpret_cast<const int32_t *>(b + mask_b);
  t->d_parent = di;
  t->d_depth = di + T;
  t->d_rank = di + 2 * T;
  t->d_slot = di + 3 * T;
  t->d_internal = di + 4 * T;
  t->d_dstart = di + 4 * T + t->internal.size();
  t->d_tile_need = reinterpret_cast<const uint32_t *>(t->d_dstart + t->dstart.size());
  t->d_cstart = t->d_dstart + t->dstart.size() + t->tile_need.size();
  t->d_clist = t->d_cstart + t->cstart.size();
  return MEDUSA_OK;
}

extern "C" void medusa_tree_free(medusa_tree *t) {
  if (!t) return;
  if (t->d_base) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != t->device) (void)hipSetDevice(t->device);
    (void)hipFree(t->d_base);
    if (cur != t->device && cur >= 0) (void)hipSetDevice(cur);
  }
  medusa::tree_delete_host(t);
}
