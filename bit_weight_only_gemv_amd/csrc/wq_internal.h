// Internal helpers shared by the host encoder (wq_host.cpp) and the HIP
// launchers.  Not part of the public ABI.
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

// Geometry of the tiled M = 1 layout (wq.h, "Tiled layout"): row blocks of 16
// rows, K-slices of 512 channels, outlier chunks of 8 slab positions; three
// sections, each starting at a multiple of 256 bytes.
struct TiledGeometry {
  int64_t nrb, nks, nch;    // row blocks, K-slices, outlier chunks
  int64_t slice_bytes;      // code bytes of one row in one slice (W4 256, W2 128)
  int64_t meta_tile;        // bytes of one scale/zero tile (1024; W4P 640)
  int64_t codes_off, meta_off, slab_off, total;
};
inline TiledGeometry tiled_geometry(int fmt, int64_t N, int64_t K, int64_t n_out) {
  TiledGeometry g{};
  g.nrb = (N + 15) / 16;
  g.nks = (K + 511) / 512;
  g.nch = (n_out + 7) / 8;
  g.slice_bytes = fmt == WQ_FMT_W2 ? 128 : 256;
  g.meta_tile = fmt == WQ_FMT_W4P ? 640 : 1024;
  auto up = [](int64_t v) { return (v + 255) / 256 * 256; };
  g.codes_off = 0;
  g.meta_off = up(g.nrb * g.nks * 16 * g.slice_bytes);
  g.slab_off = g.meta_off + up(g.nrb * g.nks * g.meta_tile);
  g.total = g.slab_off + up(g.nrb * g.nch * 256);
  return g;
}

}  // namespace wq
