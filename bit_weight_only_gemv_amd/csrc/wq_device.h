// Host-side helpers of the HIP launchers (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq_internal.h"

namespace wqd {

// LDS one workgroup may request (gfx950 has 160 KB per CU; we stay within the
// 64 KB that every launch may take without attributes).
constexpr size_t kMaxLdsBytes = 64 * 1024;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Turns a failed launch into WQ_ERR_HIP with the runtime's message.
inline int check_launch(const char* who) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wq::fail(WQ_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
  return wq::ok();
}

}  // namespace wqd
