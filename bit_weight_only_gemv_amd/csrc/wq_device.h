// Host-side helpers of the HIP launchers (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq_internal.h"

namespace wqd {

// LDS one workgroup may request: gfx950 gives a workgroup up to the whole
// 160 KB of a CU (launches above 64 KB raise the kernel's dynamic-LDS limit
// first, see allow_lds).
constexpr size_t kMaxLdsBytes = 160 * 1024;
constexpr size_t kDefaultLdsBytes = 64 * 1024;

// Raises a kernel's dynamic-LDS limit when a launch needs more than 64 KB.
inline bool allow_lds(const void* kernel, size_t bytes) {
  if (bytes <= kDefaultLdsBytes) return true;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) ==
         hipSuccess;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device (cached per device; 0 if unknown).
inline int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev] = v;
  }
  return cached[dev];
}

// A field of an explicit kernel-variant choice (wq.h, wq_variant), or `def`
// when there is none (v NULL or the field negative).
inline int variant_or(const wq_variant* v, int32_t wq_variant::*f, int def) {
  return (v != nullptr && v->*f >= 0) ? (int)(v->*f) : def;
}

// Turns a failed launch into WQ_ERR_HIP with the runtime's message.
inline int check_launch(const char* who) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wq::fail(WQ_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
  return wq::ok();
}

}  // namespace wqd
