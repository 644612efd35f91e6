// Small-M batched product on gfx950 matrix cores (wq_gemm_wq), 1 <= M <= 16.
//
// What is computed (SPECTRA page, section 4.2: the batched W4A16 kernel with
// in-kernel outlier fusion, M a runtime argument; the same contract for W2):
//   Y[m][n] = FP16( sum_{k not in outliers} X[m][k] w_hat[n][k]
//                   + sum_j out_w[n][j] X[m][out_idx[j]] ),   FP32 accumulation.
//
// How: one v_mfma_f32_16x16x32_f16 covers 16 activation rows (M padded to 16
// with zeros) x 16 weight rows x one group of 32 channels.  Lane l supplies
// weight row n = l % 16 and the 8 channels of quarter l / 16 of the group:
//   W4: one 32-bit load of bytes 4q..4q+3 of the group -> 8 codes, turned into
//       exact FP16 (q - z) with the 1024 bit-trick and one packed subtract;
//       the group's scale is applied to the MFMA result (4 FMAs per lane).
//   W2: one 16-bit load of bytes 2q, 2q+1 -> 8 codes -> FP16 centroids with one
//       byte permute per two codes; S multiplies the MFMA result and
//       Z * sum(x over the group) is added from a per-(group, m) table.
// Activations are staged per block of 16 groups in LDS, already laid out as
// MFMA A fragments in the same channel order the decoder produces, and masked
// at the outlier columns.  Outliers are a second, dense MFMA over the n_out
// gathered activations against the FP16 outlier slab.

#include "wq_common.cuh"
#include "wq_device.h"
#include "wq_mma.h"


namespace wqd {

struct GemmArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* zeros;
  const int32_t* out_idx;
  const uint16_t* out_w;
  const uint16_t* X;
  uint16_t* Y;
  int N, K, M, n_out, fuse;
};

constexpr int kGemmWaves = 4;
constexpr int kGemmRows = 16 * kGemmWaves;   // weight rows per workgroup
constexpr int kKB = 16;                      // groups per staged block

// Channel (0..31) of the group held in element e (0..7) of quarter q's fragment.
template <int FMT>
__device__ __forceinline__ int frag_channel(int q, int e) {
  if (FMT != 2) {
    // lo0 = (4q, 4q+2), hi0 = (4q+16, 4q+18), lo1 = (4q+1, 4q+3), hi1 = (4q+17, 4q+19)
    const int base[8] = {0, 2, 16, 18, 1, 3, 17, 19};
    return 4 * q + base[e];
  } else {
    // pairs (8q + p, 8q + 4 + p), p = 0..3
    return 8 * q + (e >> 1) + 4 * (e & 1);
  }
}

template <int FMT>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = a.K / kGroup;
  const int n_chunks = (a.fuse && a.n_out > 0) ? (a.n_out + 31) / 32 : 0;
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(smem);                           // [G]
  h8* s_xa = reinterpret_cast<h8*>(smem + ((4 * G + 15) & ~15));                 // [kKB][16][4]
  float* s_sx = reinterpret_cast<float*>(s_xa + kKB * 64);                        // [kKB][16]
  h8* s_xo = reinterpret_cast<h8*>(s_sx + kKB * 16);                              // [n_chunks][16][4]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int fn = lane & 15;     // weight row within the wave's 16 / activation row of A
  const int fq = lane >> 4;     // quarter of the group's channels
  const int row0 = blockIdx.x * kGemmRows;
  const int rows_here = min(kGemmRows, a.N - row0);
  const int my_row = min(wave * 16 + fn, rows_here - 1);   // clamped for loads

  for (int i = tid; i < G; i += blockDim.x) s_mask[i] = 0u;
  __syncthreads();
  for (int j = tid; j < a.n_out; j += blockDim.x) {
    const uint32_t c = (uint32_t)a.out_idx[j];
    if (c < (uint32_t)a.K) atomicOr(&s_mask[c >> 5], 1u << (c & 31));
  }
  // outlier activations as A fragments: element e of quarter q of chunk c is
  // outlier j = 32c + 8q + e
  for (int it = tid; it < n_chunks * 64; it += blockDim.x) {
    const int c = it >> 6, m = (it >> 2) & 15, q = it & 3;
    h8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 32 * c + 8 * q + e;
      uint16_t v = 0;
      if (m < a.M && j < a.n_out) {
        const uint32_t col = (uint32_t)a.out_idx[j];
        if (col < (uint32_t)a.K) v = a.X[(size_t)m * a.K + col];
      }
      f[e] = __builtin_bit_cast(_Float16, v);
    }
    s_xo[it] = f;
  }

  const uint32_t row_bytes = (uint32_t)(FMT != 2 ? a.K / 2 : a.K / 4);
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(a.codes + (uint64_t)row0 * row_bytes,
                                               clamp_bytes((uint64_t)rows_here * row_bytes));
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(a.scales + (uint64_t)row0 * G, clamp_bytes((uint64_t)rows_here * G * 2));
  // W4P (FMT 5): zero points packed two per byte, (G + 1) / 2 bytes per row
  const uint64_t zrow = FMT == 5 ? (uint64_t)(G + 1) / 2 : (uint64_t)G * 2;
  const __amdgpu_buffer_rsrc_t zrs =
      make_rsrc(reinterpret_cast<const unsigned char*>(a.zeros) + (uint64_t)row0 * zrow,
                clamp_bytes((uint64_t)rows_here * zrow));
  const __amdgpu_buffer_rsrc_t xrs =
      make_rsrc(a.X, clamp_bytes((uint64_t)a.M * a.K * 2));

  f4 acc = {0.f, 0.f, 0.f, 0.f};
  const f4 zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < G; kb += kKB) {
    __syncthreads();   // previous block consumed (and mask / outliers staged)
    {
      // stage: thread -> (group gl, activation row m); 256 threads = 16 x 16
      const int gl = tid >> 4, m = tid & 15;
      const int g = kb + gl;
      uint32_t xw[16];
      const bool live = (m < a.M) && (g < G);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        u4v t = {0u, 0u, 0u, 0u};
        if (live) t = ld128(xrs, (uint32_t)(((size_t)m * a.K + (size_t)g * 32) * 2 + 16 * v));
        xw[4 * v + 0] = t.x;
        xw[4 * v + 1] = t.y;
        xw[4 * v + 2] = t.z;
        xw[4 * v + 3] = t.w;
      }
      const uint32_t mk = live ? s_mask[g] : 0xFFFFFFFFu;
      float sum = 0.f;
      uint16_t xs[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const uint16_t v = (uint16_t)(xw[k >> 1] >> ((k & 1) * 16));
        xs[k] = ((mk >> k) & 1u) ? (uint16_t)0 : v;
        sum += h2f(xs[k]);
      }
      s_sx[gl * 16 + m] = sum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = __builtin_bit_cast(_Float16, xs[frag_channel<FMT>(q, e)]);
        s_xa[(gl * 16 + m) * 4 + q] = f;
      }
    }
    __syncthreads();

    const int gend = min(kKB, G - kb);
#pragma unroll 4
    for (int gl = 0; gl < gend; ++gl) {
      const uint32_t g = (uint32_t)(kb + gl);
      const uint32_t mo = ((uint32_t)my_row * (uint32_t)G + g) * 2u;
      const float s = h2f(ld16(srs, mo));
      const float z = FMT == 5 ? packed_zero(ld8(zrs, (uint32_t)my_row * (uint32_t)zrow + g / 2u), g)
                               : h2f(ld16(zrs, mo));
      h8 b;
      if constexpr (FMT != 2) {
        const uint32_t w = ld32(crs, (uint32_t)my_row * row_bytes + g * 16u + 4u * fq);
        const uint32_t zz = (uint32_t)f2h(1024.0f + z);
        const h2 nz = as_h2(zz | (zz << 16)) * (_Float16)(-1.0f);
        const h2 d0 = as_h2((w & 0x000F000Fu) | 0x64006400u) + nz;
        const h2 d1 = as_h2(((w >> 4) & 0x000F000Fu) | 0x64006400u) + nz;
        const h2 d2 = as_h2(((w >> 8) & 0x000F000Fu) | 0x64006400u) + nz;
        const h2 d3 = as_h2(((w >> 12) & 0x000F000Fu) | 0x64006400u) + nz;
        b = (h8){d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
      } else {
        const uint32_t v = ld16(crs, (uint32_t)my_row * row_bytes + g * 8u + 2u * fq);
        const uint32_t wv = (v & 0xFFu) | ((v & 0xFF00u) << 8);
        const h2 c0 = as_h2(w2_centroid_pair(wv & 0x00030003u));
        const h2 c1 = as_h2(w2_centroid_pair((wv >> 2) & 0x00030003u));
        const h2 c2 = as_h2(w2_centroid_pair((wv >> 4) & 0x00030003u));
        const h2 c3 = as_h2(w2_centroid_pair((wv >> 6) & 0x00030003u));
        b = (h8){c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
      }
      const h8 av = s_xa[(gl * 16 + fn) * 4 + fq];
      const f4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b, zero4, 0, 0, 0);
      if constexpr (FMT != 2) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[jj] = __builtin_fmaf(s, p[jj], acc[jj]);
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          acc[jj] = __builtin_fmaf(s, p[jj], acc[jj]);
          acc[jj] = __builtin_fmaf(z, s_sx[gl * 16 + 4 * fq + jj], acc[jj]);
        }
      }
    }
  }

  if (n_chunks) {
    const __amdgpu_buffer_rsrc_t ors =
        make_rsrc(a.out_w + (uint64_t)row0 * a.n_out, clamp_bytes((uint64_t)rows_here * a.n_out * 2));
    for (int c = 0; c < n_chunks; ++c) {
      h8 b;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 32 * c + 8 * fq + e;
        uint16_t v = 0;
        if (j < a.n_out) v = ld16(ors, ((uint32_t)my_row * (uint32_t)a.n_out + (uint32_t)j) * 2u);
        b[e] = __builtin_bit_cast(_Float16, v);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(s_xo[(c * 16 + fn) * 4 + fq], b, acc, 0, 0, 0);
    }
  }

  const int n_local = wave * 16 + fn;
  if (n_local < rows_here) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int m = 4 * fq + jj;
      if (m < a.M) a.Y[(size_t)m * a.N + row0 + n_local] = f2h(acc[jj]);
    }
  }
}

}  // namespace wqd

using namespace wqd;

extern "C" int wq_gemm_wq_v(int fmt, const uint8_t* codes, const uint16_t* scales,
                            const uint16_t* zeros, int64_t N, int64_t K, const int32_t* out_idx,
                            const uint16_t* out_w, int64_t n_out, uint32_t flags,
                            const uint16_t* X, int64_t M, uint16_t* Y, const wq_variant* v,
                            void* stream) {
  const char* who = "wq_gemm_wq";
  if (fmt != WQ_FMT_W4 && fmt != WQ_FMT_W2 && fmt != WQ_FMT_W4P)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: fmt must be WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2", who);
  if (int r = wq::check_shape(N, K, who)) return r;
  if (int r = wq::check_outlier_args(out_idx, out_w, n_out, K, who)) return r;
  if (M < 1) return wq::fail(WQ_ERR_INVALID_ARG, "%s: M must be >= 1", who);
  if (M > WQ_GEMM_MAX_M)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: M above %d is not supported", who, WQ_GEMM_MAX_M);
  if (!codes || !scales || !zeros || !X || !Y)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(zeros) || !aligned16(X) ||
      !aligned16(Y) || (n_out > 0 && (!aligned16(out_idx) || !aligned16(out_w))))
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: device pointers must be 16-byte aligned", who);
  if ((uint64_t)M * (uint64_t)K * 2 > 0xFFFFFFF0ull)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: X larger than 4 GB", who);
  GemmArgs a{codes, scales, zeros, out_idx, out_w, X, Y, (int)N, (int)K, (int)M, (int)n_out,
             (flags & WQ_FUSE_OUTLIERS) ? 1 : 0};
  hipStream_t s = (hipStream_t)stream;
  // M = 1 is the GEMV; 2 <= M <= 16 goes to the persistent matrix-core kernel
  // when its plan fits (it fuses the outlier pass; an unfused call with
  // outlier columns stays here)
  if (M == 1)
    return wq_gemv_v(fmt, codes, scales, zeros, N, K, out_idx, out_w, n_out, flags, X, Y, v,
                     stream);
  if (a.fuse || n_out == 0) {
    const int mode = variant_or(v, &wq_variant::gemm_kernel, 1);
    bool launched = false;
    // up to four rows (two for W2): the M = 1 matrix-core kernel with its group
    // slots shared by the rows (its decode needs no FP16 weights)
    if (M <= 4 && mode != 0 && variant_or(v, &wq_variant::gemm_rows, 1) != 0) {
      const int r = wqd_mma_rows(fmt, false, codes, scales, zeros, N, K, out_idx, out_w,
                                 a.fuse ? n_out : 0, X, M, Y, s, who, 2, &launched);
      if (r != WQ_OK || launched) return r;
    }
    const int r = wqd_gemm_mma(fmt, codes, scales, zeros, N, K, out_idx, out_w, a.fuse ? n_out : 0,
                               X, M, Y, v, s, who, mode, &launched);
    if (r != WQ_OK || launched) return r;
  }
  const int G = (int)(K / kGroup);
  const int n_chunks = (a.fuse && n_out > 0) ? (int)((n_out + 31) / 32) : 0;
  const size_t lds = (size_t)((4 * G + 15) & ~15) + (size_t)kKB * 64 * 16 + (size_t)kKB * 16 * 4 +
                     (size_t)n_chunks * 64 * 16;
  if (lds > kMaxLdsBytes)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: %zu bytes of LDS needed (n_out too large)", who, lds);
  const dim3 grid((unsigned)((N + kGemmRows - 1) / kGemmRows)), block(kGemmWaves * 64);
  const void* k = fmt == WQ_FMT_W4    ? reinterpret_cast<const void*>(&gemm_kernel<4>)
                  : fmt == WQ_FMT_W4P ? reinterpret_cast<const void*>(&gemm_kernel<5>)
                                      : reinterpret_cast<const void*>(&gemm_kernel<2>);
  if (!allow_lds(k, lds)) return wq::fail(WQ_ERR_HIP, "%s: cannot raise the LDS limit", who);
  if (fmt == WQ_FMT_W4)
    hipLaunchKernelGGL(gemm_kernel<4>, grid, block, lds, s, a);
  else if (fmt == WQ_FMT_W4P)
    hipLaunchKernelGGL(gemm_kernel<5>, grid, block, lds, s, a);
  else
    hipLaunchKernelGGL(gemm_kernel<2>, grid, block, lds, s, a);
  return check_launch(who);
}

extern "C" int wq_gemm_wq(int fmt, const uint8_t* codes, const uint16_t* scales,
                          const uint16_t* zeros, int64_t N, int64_t K, const int32_t* out_idx,
                          const uint16_t* out_w, int64_t n_out, uint32_t flags, const uint16_t* X,
                          int64_t M, uint16_t* Y, void* stream) {
  return wq_gemm_wq_v(fmt, codes, scales, zeros, N, K, out_idx, out_w, n_out, flags, X, M, Y,
                      nullptr, stream);
}
