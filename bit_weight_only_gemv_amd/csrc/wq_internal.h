// Internal helpers shared by the host encoder (wq_host.cpp) and the HIP
// launchers (wq_device.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "wq.h"

namespace wq {

// Records `msg` as this thread's last error and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears this thread's last error and returns WQ_OK.
int ok();

// Shape rules shared by every entry point (see wq.h "Supported shapes").
int check_shape(int64_t N, int64_t K, const char* who);
int check_outlier_args(const int32_t* idx, const uint16_t* out_w, int64_t n_out, int64_t K,
                       const char* who);

}  // namespace wq
