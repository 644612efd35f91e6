// Matrix-core GEMV launcher (wq_mma.hip), called by the GEMV entry points.
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq.h"

// Launches the matrix-core M = 1 kernel when the shape suits it and sets
// *launched; otherwise returns WQ_OK with *launched = false and the caller
// uses the VALU kernels.  `mode`: 0 = never, 1 = when the plan prefers it,
// 2 = whenever the shape is supported.  With `tiled`, `codes` is the tiled
// layer (wq.h "Tiled layout") and scales / zeros / out_w are not used.
int wqd_gemv_mma(int fmt, bool tiled, const uint8_t* codes, const uint16_t* scales,
                 const uint16_t* zeros, int64_t N, int64_t K, const int32_t* out_idx,
                 const uint16_t* out_w, int64_t n_out, const uint16_t* x, uint16_t* y,
                 hipStream_t stream, const char* who, int mode, bool* launched);

// The same matrix-core kernel for M = 1 to 4 activation rows (W2: 1 or 2),
// X [M][K] -> Y [M][N]: the rows share the 16 A-row slots, each slice taken in
// M windows of 16 / M groups (3 rows run as 4); same contract and `mode` values
// as wqd_gemv_mma.
int wqd_mma_rows(int fmt, bool tiled, const uint8_t* codes, const uint16_t* scales,
                 const uint16_t* zeros, int64_t N, int64_t K, const int32_t* out_idx,
                 const uint16_t* out_w, int64_t n_out, const uint16_t* X, int64_t M, uint16_t* Y,
                 hipStream_t stream, const char* who, int mode, bool* launched);

// Launches the matrix-core batched kernel (2 <= M <= 16) when the shape suits
// it (same contract and `mode` values as wqd_gemv_mma).
int wqd_gemm_mma(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                 int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
                 int64_t n_out, const uint16_t* X, int64_t M, uint16_t* Y, const wq_variant* v,
                 hipStream_t stream, const char* who, int mode, bool* launched);

// The batched kernel (2 <= M <= 16) on the tiled layout of the M = 1 kernel
// (the same buffer): each wave load is four contiguous 256-byte runs of a
// tile.  Launches when the shape suits it and sets *launched.
int wqd_gemm_mma_tiled(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                       const int32_t* out_idx, int64_t n_out, const uint16_t* X, int64_t M,
                       uint16_t* Y, const wq_variant* v, hipStream_t stream, const char* who,
                       bool* launched);

// The tiled M = 1 kernel with the runtime top-k refinement fused in: y =
// FP16(layer x + sum over the k largest |x_i| of each chunk of x_i C[:, i]),
// C in the W4 format along N ([K][N / 2] codes, [K][N / 32] scales and zeros).
// The selection and the add run on helper waves added to the workgroup (up to
// 12 waves in all) while the others stream the weights.  Launches when the
// shape suits it (at most 4 refinement units of (chunk, 32 picks, row block)
// per helper lane, LDS within the limit) and sets *launched;
// otherwise returns WQ_OK with *launched = false.  sel_out, when not NULL,
// receives the selection (chunk c's picks at c min(k, chunk)).
int wqd_gemv_refine_mma(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                        const int32_t* out_idx, int64_t n_out, const uint16_t* x, uint16_t* y,
                        const uint8_t* rcodes, const uint16_t* rscales, const uint16_t* rzeros,
                        int64_t chunk, int64_t k, int32_t* sel_out, const wq_variant* v,
                        hipStream_t stream, const char* who, bool* launched);
