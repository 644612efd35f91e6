// Fused M = 1 dequantize-and-multiply for gfx950 (wq_gemv_w4 / wq_gemv_w2).
//
// What is computed (SPECTRA page, section 4.1; OTF-LLM v4.0 page, section 5
// and "Architecture & Key Innovations"):
//   y[n] = FP16( sum_{k not in outliers} w_hat[n][k] x[k]
//                + sum_j out_w[n][j] x[out_idx[j]] ),   FP32 accumulation,
// with w_hat = (q - z) s (W4) or S C[q] + Z (W2) per group of 32 along K.
//
// How (gfx950, wave64):
//  * The K axis is cut into slices of 64 lanes x GPL groups; a wave owns one
//    slice (K-wave) and keeps the matching 64*GPL*... activations in VGPRs,
//    already paired the way the code decoder produces weights.  A workgroup is
//    wk K-waves x wr row-waves; every row-wave sweeps rows of the tile.
//  * Per row, each lane streams its groups' packed codes with one buffer load
//    per group (16 B for W4, 8 B for W2; a wave covers 1 KB / 512 B of the row,
//    fully coalesced) plus the FP16 scale and zero.
//  * The group's scale and zero are factored out of the inner loop:
//      W4: sum (q - z) s x = s (sum (1024 + q) x - z sum x - 1024 sum x),
//          the (1024 + q) values coming straight out of a bit-OR into FP16 1024;
//      W2: sum (S C[q] + Z) x = S sum C[q] x + Z sum x,
//          the FP16 centroids coming out of one byte permute per two codes.
//    The per-group sums of x are computed once per lane at start.  Products
//    are v_dot2 (two FP16 products into an FP32 accumulator).
//  * Outlier columns: x is masked at those columns for the background (an LDS
//    bitmask), and the FP16 outlier row slab is dotted with the gathered
//    outlier activations into the same per-lane accumulator before the
//    reduction, so the outlier pass costs no extra reduction or launch.
//  * Reduction: DPP within 16-lane rows, then the 4 x wk partial sums of a
//    row are added in a fixed order from LDS (deterministic, no atomics).

#include "wq_common.cuh"
#include "wq_device.h"
#include "wq_mma.h"


#include <algorithm>

namespace wqd {

struct GemvArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* zeros;
  const int32_t* out_idx;
  const uint16_t* out_w;
  const uint16_t* x;
  uint16_t* y;
  int N, K, n_out;
  int wk, wr, rpw;   // K-waves, row-waves, rows per row-wave
  int fuse;          // add the outlier columns in this launch
};

constexpr int kRowsPerStep = 4;   // rows whose loads are in flight together per wave

template <int FMT>
struct Fmt;
template <>
struct Fmt<4> {
  static constexpr int kGroupBytes = 16;
  static constexpr int kRowBytesPerK = 2;   // row bytes = K / 2
  typedef u4v Codes;
};
template <>
struct Fmt<2> {
  static constexpr int kGroupBytes = 8;
  static constexpr int kRowBytesPerK = 4;   // row bytes = K / 4
  typedef u2 Codes;
};
// W4P: the W4 codes; only the zero points are stored differently (packed).
template <>
struct Fmt<5> : Fmt<4> {};

// Masked FP16 activation k of a group whose 32 values sit in 16 packed words.
__device__ __forceinline__ uint16_t xh(const uint32_t (&xw)[16], uint32_t mask, int k) {
  const uint16_t v = (uint16_t)(xw[k >> 1] >> ((k & 1) * 16));
  return ((mask >> k) & 1u) ? (uint16_t)0 : v;
}

// Masks one group's 32 activations (bit k of `mask` set = column k is an
// outlier, or the group is past K) and pairs them the way the decoder emits
// weights: W4 word j gives (4j, 4j+2), (4j+16, 4j+18), (4j+1, 4j+3),
// (4j+17, 4j+19); W2 word j, byte h, position p gives (16j+4h+p, +8).
// Also returns the float sum of the masked activations.
template <int FMT>
__device__ __forceinline__ void pair_group(const uint32_t (&xw)[16], uint32_t m,
                                           uint32_t (&out)[16], float& sum) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) s += h2f(xh(xw, m, k));
  sum = s;
  if constexpr (FMT != 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[4 * j + 0] = pack2(xh(xw, m, 4 * j), xh(xw, m, 4 * j + 2));
      out[4 * j + 1] = pack2(xh(xw, m, 4 * j + 16), xh(xw, m, 4 * j + 18));
      out[4 * j + 2] = pack2(xh(xw, m, 4 * j + 1), xh(xw, m, 4 * j + 3));
      out[4 * j + 3] = pack2(xh(xw, m, 4 * j + 17), xh(xw, m, 4 * j + 19));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int k = 16 * j + 4 * h + p;
          out[8 * j + 4 * h + p] = pack2(xh(xw, m, k), xh(xw, m, k + 8));
        }
  }
}

__device__ __forceinline__ void load_group_x(__amdgpu_buffer_rsrc_t xrs, uint32_t off,
                                             uint32_t (&xw)[16]) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const u4v t = ld128(xrs, off == 0x80000000u ? off : off + 16u * v);
    xw[4 * v + 0] = t.x;
    xw[4 * v + 1] = t.y;
    xw[4 * v + 2] = t.z;
    xw[4 * v + 3] = t.w;
  }
}

constexpr int kOutRegs = 4;   // outlier columns per lane kept in registers
constexpr uint32_t kOob = 0x80000000u;   // buffer offset past any range: loads return 0

// One wave's loads for up to kRowsPerStep rows: codes, scale, zero of its
// groups, and the outlier weights of the outlier columns it owns.
template <int FMT, int GPL>
struct RowBatch {
  typename Fmt<FMT>::Codes cw[kRowsPerStep][GPL];
  uint16_t sv[kRowsPerStep][GPL], zv[kRowsPerStep][GPL];
  uint16_t ow[kRowsPerStep][kOutRegs];
};

// Contiguous byte range [b0, b0 + len) of a global array staged into LDS by
// the whole workgroup with 16-byte loads (at most kStageSlots per thread;
// larger ranges fall back to a loop).  Loads are issued first (issue) and
// written to LDS later (commit), so the wait for them can come after other
// loads were issued.  Data starts at dst + shift in LDS.
constexpr int kStageSlots = 2;
struct Stage {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t shift, nchunks;
  u4v v[kStageSlots];
  __device__ __forceinline__ void issue(const void* base, uint64_t b0, uint64_t len,
                                        uint64_t total, int tid, int nthr) {
    const uint64_t a0 = b0 & ~(uint64_t)15;
    shift = (uint32_t)(b0 - a0);
    nchunks = (uint32_t)((shift + len + 15) / 16);
    // A 16-byte load that reaches past the record count returns all zeros, so
    // the count is rounded up to whole chunks: the few bytes past the array end
    // stay inside the 16-byte block (and page) of its last element, and are
    // never used.
    rs = make_rsrc(static_cast<const unsigned char*>(base) + a0,
                   clamp_bytes((total - a0 + 15) & ~(uint64_t)15));
#pragma unroll
    for (int i = 0; i < kStageSlots; ++i) {
      const uint32_t c = (uint32_t)(tid + nthr * i);
      v[i] = ld128(rs, c < nchunks ? c * 16u : 0x80000000u);
    }
  }
  __device__ __forceinline__ void commit(unsigned char* dst, int tid, int nthr) const {
    u4v* d = reinterpret_cast<u4v*>(dst);
#pragma unroll
    for (int i = 0; i < kStageSlots; ++i) {
      const uint32_t c = (uint32_t)(tid + nthr * i);
      if (c < nchunks) d[c] = v[i];
    }
    for (uint32_t c = (uint32_t)(tid + nthr * kStageSlots); c < nchunks; c += (uint32_t)nthr)
      d[c] = ld128(rs, c * 16u);
  }
};

__device__ __forceinline__ size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

// Bytes of LDS the main kernel needs (host and device agree on this layout).
constexpr int kLutCopies = 4;   // W2 byte table: 256 entries x 4 lane-sliced copies
__host__ __device__ inline size_t gemv_lds_bytes(int K, int RT, int wk, int n_out, bool has_out,
                                                 int fmt) {
  const size_t G = (size_t)K / kGroup;
  size_t off = ((size_t)16 * RT * wk + 15) & ~(size_t)15;              // partial sums
  if (fmt == 2) off += (size_t)256 * kLutCopies * 8;                    // W2 centroid table
  off += ((size_t)RT * G * 2 + 16 + 15) & ~(size_t)15;                 // scales
  off += ((size_t)RT * (fmt == 5 ? (G + 1) / 2 : G * 2) + 16 + 15) & ~(size_t)15;   // zeros
  if (has_out) {
    off += ((size_t)RT * n_out * 2 + 16 + 15) & ~(size_t)15;           // outlier slab rows
    off += ((size_t)n_out * 4 + 16 + 15) & ~(size_t)15;                // outlier indices
  }
  return off + (size_t)K * 2;                                          // activations
}

template <int FMT, int GPL, bool HAS_OUT>
__device__ __forceinline__ void load_rows(RowBatch<FMT, GPL>& b, __amdgpu_buffer_rsrc_t crs,
                                          __amdgpu_buffer_rsrc_t srs, __amdgpu_buffer_rsrc_t zrs,
                                          __amdgpu_buffer_rsrc_t ors, int r_first, int r_end,
                                          uint32_t row_bytes, uint32_t G, int kw, int lane,
                                          const bool (&gvalid)[GPL], const bool (&oval)[kOutRegs],
                                          int wk, int n_out) {
  typedef Fmt<FMT> F;
#pragma unroll
  for (int u = 0; u < kRowsPerStep; ++u) {
    const bool rv = r_first + u < r_end;
    const uint32_t rl = (uint32_t)(r_first + u);
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const uint32_t g = (uint32_t)((kw * GPL + i) * kWave + lane);
      const bool ok = rv && gvalid[i];
      const uint32_t co = ok ? rl * row_bytes + g * F::kGroupBytes : kOob;
      const uint32_t mo = ok ? (rl * G + g) * 2u : kOob;
      if constexpr (FMT != 2)
        b.cw[u][i] = ld128(crs, co);
      else
        b.cw[u][i] = ld64(crs, co);
      b.sv[u][i] = ld16(srs, mo);
      if constexpr (FMT == 5)   // the byte holding the zero point (rows of (G + 1) / 2 bytes)
        b.zv[u][i] = ld8(zrs, ok ? rl * ((G + 1u) / 2u) + g / 2u : kOob);
      else
        b.zv[u][i] = ld16(zrs, mo);
    }
    if constexpr (HAS_OUT) {
#pragma unroll
      for (int t = 0; t < kOutRegs; ++t) {
        const int j = (kw + wk * t) * kWave + lane;
        const bool ok = rv && oval[t];
        b.ow[u][t] = ld16(ors, ok ? (rl * (uint32_t)n_out + (uint32_t)j) * 2u : kOob);
      }
    }
  }
}

// One W4 group: codes enter v_dot2 as FP16 subnormals q * 2^-24 (low nibbles)
// and 16 q * 2^-24 (high nibbles); sum (q - z) s x = s (2^24 (lo + hi / 16) - z sum x).
__device__ __forceinline__ float w4_group_dot(const u4v& cw, const uint32_t (&xr)[16], float s,
                                              float z, float sx, float acc) {
  float alo = 0.f, ahi = 0.f;
  const uint32_t wv[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t lo0, hi0, lo1, hi1;
    w4_word_sub(wv[j], lo0, hi0, lo1, hi1);
    alo = __builtin_amdgcn_fdot2(as_h2(lo0), as_h2(xr[4 * j + 0]), alo, false);
    ahi = __builtin_amdgcn_fdot2(as_h2(hi0), as_h2(xr[4 * j + 1]), ahi, false);
    alo = __builtin_amdgcn_fdot2(as_h2(lo1), as_h2(xr[4 * j + 2]), alo, false);
    ahi = __builtin_amdgcn_fdot2(as_h2(hi1), as_h2(xr[4 * j + 3]), ahi, false);
  }
  float v = __builtin_fmaf(ahi, 0.0625f, alo) * 16777216.0f;
  v = __builtin_fmaf(-z, sx, v);
  return __builtin_fmaf(s, v, acc);
}

// Group g of slot i of lane `lane` in K-wave kw.  W4 (and W2 with one group
// per lane): slot i covers 64 consecutive groups, one per lane, so a wave's
// load of a slot is one contiguous stretch of the row.  W2 with an even count:
// a lane owns GPL consecutive groups, so two W2 groups (16 bytes) are one
// 16-byte load.
template <int FMT, int GPL>
__device__ __forceinline__ int group_of(int kw, int i, int lane) {
  if constexpr (FMT == 2 && GPL % 2 == 0)
    return kw * GPL * kWave + GPL * lane + i;
  else
    return (kw * GPL + i) * kWave + lane;
}

// Main kernel.  Per workgroup (RT rows): the scales, zeros and outlier
// weights of its rows, the outlier indices and x are each one contiguous
// range and are staged into LDS with 16-byte loads by the whole workgroup;
// x is masked in LDS (one 16-bit store per outlier column).  The packed codes
// are the only per-lane global loads.  Each wave then reads its K-slice of x,
// pairs it the way the decoder emits weights, and sweeps its rows.
template <int FMT, int GPL, bool HAS_OUT, int XC>
__global__ void __launch_bounds__(512) gemv_lds_kernel(GemvArgs a) {
  typedef Fmt<FMT> F;
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = a.K / kGroup;
  const int RT = a.wr * a.rpw;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int kw = wave % a.wk;
  const int rw = wave / a.wk;
  const int tile0 = blockIdx.x * RT;
  const int rows_here = min(RT, a.N - tile0);
  const int r_first = rw * a.rpw;
  const int r_end = min(r_first + a.rpw, rows_here);
  const bool do_out = a.fuse && a.n_out > 0;
  const int jstride = a.wk * kWave;
  const int n_cap = jstride * kOutRegs;
  const int T = min(kOutRegs, (a.n_out + jstride - 1) / jstride);
  const int nch = a.K / 8;   // 16-byte chunks of x

  size_t off = align16((size_t)16 * RT * a.wk);
  float* s_part = reinterpret_cast<float*>(smem);
  u2* s_lut = reinterpret_cast<u2*>(smem + off);   // W2: [256][kLutCopies]
  if (FMT == 2) off += (size_t)256 * kLutCopies * 8;
  unsigned char* s_sc = smem + off;
  off += align16((size_t)RT * G * 2 + 16);
  unsigned char* s_zr = smem + off;
  const int Gz = FMT == 5 ? (G + 1) / 2 : G * 2;   // bytes of zero points per row
  off += align16((size_t)RT * Gz + 16);
  unsigned char* s_ow = smem + off;
  if (HAS_OUT) off += align16((size_t)RT * a.n_out * 2 + 16);
  int32_t* s_idx = reinterpret_cast<int32_t*>(smem + off);
  if (HAS_OUT) off += align16((size_t)a.n_out * 4 + 16);
  uint16_t* s_x = reinterpret_cast<uint16_t*>(smem + off);
  u4v* s_x16 = reinterpret_cast<u4v*>(smem + off);

  // ---- (1) loads, in the order they are needed; all branch-free
  Stage st_idx, st_sc, st_zr, st_ow;
  if constexpr (HAS_OUT) st_idx.issue(a.out_idx, 0, (uint64_t)a.n_out * 4, (uint64_t)a.n_out * 4, tid, nthr);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x, (uint32_t)a.K * 2u);
  u4v xc[XC];
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int c = tid + nthr * i;
    xc[i] = ld128(xrs, c < nch ? (uint32_t)c * 16u : kOob);
  }
  const uint64_t meta_total = (uint64_t)a.N * G * 2;
  st_sc.issue(a.scales, (uint64_t)tile0 * G * 2, (uint64_t)rows_here * G * 2, meta_total, tid, nthr);
  st_zr.issue(a.zeros, (uint64_t)tile0 * Gz, (uint64_t)rows_here * Gz, (uint64_t)a.N * Gz, tid,
              nthr);
  if constexpr (HAS_OUT)
    st_ow.issue(a.out_w, (uint64_t)tile0 * a.n_out * 2, (uint64_t)rows_here * a.n_out * 2,
                (uint64_t)a.N * a.n_out * 2, tid, nthr);
  const uint64_t row_bytes = (uint64_t)a.K / F::kRowBytesPerK;
  const __amdgpu_buffer_rsrc_t crs =
      make_rsrc(a.codes + (uint64_t)tile0 * row_bytes, clamp_bytes((uint64_t)rows_here * row_bytes));
  bool gvalid[GPL];
#pragma unroll
  for (int i = 0; i < GPL; ++i) gvalid[i] = group_of<FMT, GPL>(kw, i, lane) < G;
  typename F::Codes cw[kRowsPerStep][GPL];
#pragma unroll
  for (int u = 0; u < kRowsPerStep; ++u) {
    const bool rv = r_first + u < r_end;
    const uint32_t rb = (uint32_t)(r_first + u) * (uint32_t)row_bytes;
    if constexpr (FMT == 2 && GPL % 2 == 0) {
#pragma unroll
      for (int i = 0; i < GPL; i += 2) {
        const uint32_t g = (uint32_t)group_of<FMT, GPL>(kw, i, lane);
        // G is even here (K % 64 == 0), so both groups of the pair are valid or neither
        const u4v v = ld128(crs, (rv && gvalid[i]) ? rb + g * 8u : kOob);
        cw[u][i] = (u2){v.x, v.y};
        cw[u][i + 1] = (u2){v.z, v.w};
      }
    } else {
#pragma unroll
      for (int i = 0; i < GPL; ++i) {
        const uint32_t g = (uint32_t)group_of<FMT, GPL>(kw, i, lane);
        const uint32_t co = (rv && gvalid[i]) ? rb + g * F::kGroupBytes : kOob;
        if constexpr (FMT != 2)
          cw[u][i] = ld128(crs, co);
        else
          cw[u][i] = ld64(crs, co);
      }
    }
  }

  // ---- (2) staged ranges into LDS
  if constexpr (HAS_OUT) st_idx.commit(reinterpret_cast<unsigned char*>(s_idx), tid, nthr);
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int c = tid + nthr * i;
    if (c < nch) s_x16[c] = xc[i];
  }
  for (int c = tid + nthr * XC; c < nch; c += nthr) s_x16[c] = ld128(xrs, (uint32_t)c * 16u);
  st_sc.commit(s_sc, tid, nthr);
  st_zr.commit(s_zr, tid, nthr);
  if constexpr (HAS_OUT) st_ow.commit(s_ow, tid, nthr);
  if constexpr (FMT == 2) {
    // entry e = one code byte (four codes) -> their four FP16 centroids; lane l
    // reads copy l % kLutCopies, which spreads a wave's reads over more banks
    for (int i = tid; i < 256 * kLutCopies; i += nthr) {
      const uint32_t e = (uint32_t)i / kLutCopies;
      s_lut[i] = (u2){w2_centroid_pair((e & 3u) | (((e >> 2) & 3u) << 16)),
                      w2_centroid_pair(((e >> 4) & 3u) | ((e >> 6) << 16))};
    }
  }
  lds_barrier();

  // ---- (3) outlier activations, then the outlier columns of x zeroed
  float xo[kOutRegs];
  if constexpr (HAS_OUT) {
#pragma unroll
    for (int t = 0; t < kOutRegs; ++t) {
      const int j = (kw + a.wk * t) * kWave + lane;
      const uint32_t c = (t < T && j < a.n_out) ? (uint32_t)s_idx[j] : 0xFFFFFFFFu;
      xo[t] = c < (uint32_t)a.K ? h2f(s_x[c]) : 0.f;
    }
    lds_barrier();
    for (int j = tid; j < a.n_out; j += nthr) {
      const uint32_t c = (uint32_t)s_idx[j];
      if (c < (uint32_t)a.K) s_x[c] = 0;
    }
    lds_barrier();
  }

  // ---- (4) this wave's activations, paired as the decoder emits weights
  uint32_t xr[GPL][16];
  float sx[GPL];
  const uint32_t one2 = 0x3C003C00u;   // FP16 (1, 1)
#pragma unroll
  for (int i = 0; i < GPL; ++i) {
    const int g = gvalid[i] ? group_of<FMT, GPL>(kw, i, lane) : 0;
    uint32_t xw[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u4v t = s_x16[g * 4 + v];
      xw[4 * v + 0] = t.x;
      xw[4 * v + 1] = t.y;
      xw[4 * v + 2] = t.z;
      xw[4 * v + 3] = t.w;
    }
    float sum = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) sum = __builtin_amdgcn_fdot2(as_h2(xw[m]), as_h2(one2), sum, false);
    sx[i] = sum;
    if constexpr (FMT != 2) {
      // (4j, 4j+2), (4j+16, 4j+18), (4j+1, 4j+3), (4j+17, 4j+19)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xr[i][4 * j + 0] = __builtin_amdgcn_perm(xw[2 * j + 1], xw[2 * j], 0x05040100u);
        xr[i][4 * j + 1] = __builtin_amdgcn_perm(xw[2 * j + 9], xw[2 * j + 8], 0x05040100u);
        xr[i][4 * j + 2] = __builtin_amdgcn_perm(xw[2 * j + 1], xw[2 * j], 0x07060302u);
        xr[i][4 * j + 3] = __builtin_amdgcn_perm(xw[2 * j + 9], xw[2 * j + 8], 0x07060302u);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 16; ++m) xr[i][m] = xw[m];   // natural pairs (2m, 2m + 1)
    }
  }
  const uint32_t lut_lane = (uint32_t)(lane & (kLutCopies - 1)) * 8u;
  const unsigned char* lut8 = reinterpret_cast<const unsigned char*>(s_lut);

  // ---- (5) the rows
  const uint16_t* sc16 = reinterpret_cast<const uint16_t*>(s_sc + st_sc.shift);
  const uint16_t* zr16 = reinterpret_cast<const uint16_t*>(s_zr + st_zr.shift);
  const uint16_t* ow16 = reinterpret_cast<const uint16_t*>(s_ow + (HAS_OUT ? st_ow.shift : 0));
#pragma unroll
  for (int u = 0; u < kRowsPerStep; ++u) {
    const int rl = r_first + u;
    if (rl >= r_end) break;   // uniform across the wave
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      if (!gvalid[i]) continue;
      const int g = group_of<FMT, GPL>(kw, i, lane);
      const float s = h2f(sc16[rl * G + g]);
      const float z = FMT == 5 ? packed_zero(s_zr[st_zr.shift + rl * Gz + (g >> 1)], (uint32_t)g)
                               : h2f(zr16[rl * G + g]);
      if constexpr (FMT != 2) {
        acc = w4_group_dot(cw[u][i], xr[i], s, z, sx[i], acc);
      } else {
        // byte b of the group = codes 4b .. 4b + 3 = activation words 2b, 2b + 1
        float ac = 0.f;
        const uint32_t wv[2] = {cw[u][i].x, cw[u][i].y};
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int by = 0; by < 4; ++by) {
            const uint32_t e = (wv[j] >> (8 * by)) & 0xFFu;
            const u2 c4 = *reinterpret_cast<const u2*>(lut8 + e * (kLutCopies * 8u) + lut_lane);
            ac = __builtin_amdgcn_fdot2(as_h2(c4.x), as_h2(xr[i][8 * j + 2 * by]), ac, false);
            ac = __builtin_amdgcn_fdot2(as_h2(c4.y), as_h2(xr[i][8 * j + 2 * by + 1]), ac, false);
          }
        acc = __builtin_fmaf(s, ac, acc);
        acc = __builtin_fmaf(z, sx[i], acc);
      }
    }
    if (HAS_OUT && do_out) {
#pragma unroll
      for (int t = 0; t < kOutRegs; ++t) {
        const int j = (kw + a.wk * t) * kWave + lane;
        if (t < T && j < a.n_out) acc = __builtin_fmaf(h2f(ow16[rl * a.n_out + j]), xo[t], acc);
      }
      for (int j = n_cap + kw * kWave + lane; j < a.n_out; j += jstride) {
        const uint32_t c = (uint32_t)s_idx[j];
        acc = __builtin_fmaf(h2f(ow16[rl * a.n_out + j]),
                             c < (uint32_t)a.K ? h2f(a.x[c]) : 0.f, acc);
      }
    }
    acc = row16_sum(acc);
    if ((lane & 15) == 0) s_part[(rl * a.wk + kw) * 4 + (lane >> 4)] = acc;
  }
  __syncthreads();
  for (int t = tid; t < rows_here; t += nthr) {
    float sum = 0.f;
    for (int k = 0; k < a.wk; ++k) {
      const float* p = s_part + (t * a.wk + k) * 4;
      sum += (p[0] + p[1]) + (p[2] + p[3]);
    }
    a.y[tile0 + t] = f2h(sum);
  }
}

template <int FMT, int GPL, bool HAS_OUT>
__global__ void __launch_bounds__(512) gemv_reg_kernel(GemvArgs a) {
  typedef Fmt<FMT> F;
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = a.K / kGroup;
  const int RT = a.wr * a.rpw;
  // LDS: outlier bitmask, later reused for the partial sums (every wave has
  // read its mask words before the first partial is written)
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(smem);                 // [G] outlier bits
  float* s_part = reinterpret_cast<float*>(smem);                       // [RT][wk][4]

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int kw = wave % a.wk;
  const int rw = wave / a.wk;
  const int tile0 = blockIdx.x * RT;
  const int rows_here = min(RT, a.N - tile0);
  const int r_first = rw * a.rpw;                       // tile-local
  const int r_end = min(r_first + a.rpw, rows_here);
  const bool do_out = a.fuse && a.n_out > 0;

  // Outlier columns this lane owns: j_t = (kw + wk t) * 64 + lane.  Every
  // column below n_cap has exactly one owner per row-wave; the rest (only when
  // n_out > n_cap) go through a slower per-row loop.
  const int jstride = a.wk * kWave;
  const int n_cap = jstride * kOutRegs;
  const int T = min(kOutRegs, (a.n_out + jstride - 1) / jstride);   // wave-uniform

  // ---- (1) loads, issued in the order they are needed (loads return in order)
  // All prologue loads are branch-free (invalid lanes read past the buffer and
  // get 0), so the compiler's wait counters can let them overlap.
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(a.out_idx, (uint32_t)a.n_out * 4u);
  uint32_t oraw[kOutRegs];
  bool oval[kOutRegs];
#pragma unroll
  for (int t = 0; t < kOutRegs; ++t) {
    const int j = (kw + a.wk * t) * kWave + lane;
    oval[t] = HAS_OUT && t < T && j < a.n_out;
    oraw[t] = HAS_OUT ? ld32(irs, oval[t] ? (uint32_t)j * 4u : kOob) : 0u;
  }
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x, (uint32_t)a.K * 2u);
  uint32_t xw[GPL][16];
#pragma unroll
  for (int i = 0; i < GPL; ++i) {
    const uint32_t g = (uint32_t)((kw * GPL + i) * kWave + lane);
    load_group_x(xrs, g < (uint32_t)G ? g * 64u : kOob, xw[i]);
  }
  const uint64_t row_bytes = (uint64_t)a.K / F::kRowBytesPerK;
  const __amdgpu_buffer_rsrc_t crs =
      make_rsrc(a.codes + (uint64_t)tile0 * row_bytes, clamp_bytes((uint64_t)rows_here * row_bytes));
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(a.scales + (uint64_t)tile0 * G, clamp_bytes((uint64_t)rows_here * G * 2));
  const uint64_t zrow = FMT == 5 ? (uint64_t)(G + 1) / 2 : (uint64_t)G * 2;   // bytes per row
  const __amdgpu_buffer_rsrc_t zrs =
      make_rsrc(reinterpret_cast<const unsigned char*>(a.zeros) + (uint64_t)tile0 * zrow,
                clamp_bytes((uint64_t)rows_here * zrow));
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(
      do_out ? a.out_w + (uint64_t)tile0 * a.n_out : a.out_w,
      do_out ? clamp_bytes((uint64_t)rows_here * a.n_out * 2) : 0u);
  bool gvalid[GPL];
#pragma unroll
  for (int i = 0; i < GPL; ++i) gvalid[i] = (kw * GPL + i) * kWave + lane < G;

  RowBatch<FMT, GPL> b;
  load_rows<FMT, GPL, HAS_OUT>(b, crs, srs, zrs, ors, r_first, r_end, (uint32_t)row_bytes,
                               (uint32_t)G, kw, lane, gvalid, oval, a.wk, a.n_out);

  // ---- (2) outlier bitmask in LDS (the background skips these columns)
  if constexpr (HAS_OUT) {
    for (int i = tid; i < G; i += nthr) s_mask[i] = 0u;
    lds_barrier();
#pragma unroll
    for (int t = 0; t < kOutRegs; ++t)
      if (oval[t] && oraw[t] < (uint32_t)a.K) atomicOr(&s_mask[oraw[t] >> 5], 1u << (oraw[t] & 31));
    for (int j = n_cap + tid; j < a.n_out; j += nthr) {
      const uint32_t c = (uint32_t)a.out_idx[j];
      if (c < (uint32_t)a.K) atomicOr(&s_mask[c >> 5], 1u << (c & 31));
    }
    lds_barrier();
  }

  // ---- (3) outlier activations (gathered now, used after the background)
  uint16_t xo[kOutRegs];
#pragma unroll
  for (int t = 0; t < kOutRegs; ++t)
    xo[t] = ld16(xrs, (HAS_OUT && oval[t] && oraw[t] < (uint32_t)a.K) ? oraw[t] * 2u : kOob);

  // ---- (4) activations, masked and paired as the decoder emits weights
  uint32_t xr[GPL][16];
  float sx[GPL];
#pragma unroll
  for (int i = 0; i < GPL; ++i) {
    const int g = (kw * GPL + i) * kWave + lane;
    const uint32_t m = !gvalid[i] ? 0xFFFFFFFFu : (HAS_OUT ? s_mask[g] : 0u);
    pair_group<FMT>(xw[i], m, xr[i], sx[i]);
  }

  // ---- (5) the rows (s_part aliases s_mask: wait until every wave has read its mask)
  if constexpr (HAS_OUT) lds_barrier();
  {
#pragma unroll
    for (int u = 0; u < kRowsPerStep; ++u) {
      const int rl = r_first + u;
      if (rl >= r_end) break;   // uniform across the wave
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < GPL; ++i) {
        if (!gvalid[i]) continue;
        const float s = h2f(b.sv[u][i]);
        const float z = FMT == 5 ? packed_zero(b.zv[u][i], (uint32_t)((kw * GPL + i) * kWave + lane))
                                 : h2f(b.zv[u][i]);
        if constexpr (FMT != 2) {
          acc = w4_group_dot(b.cw[u][i], xr[i], s, z, sx[i], acc);
        } else {
          float ac = 0.f;
          const uint32_t wv[2] = {b.cw[u][i].x, b.cw[u][i].y};
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int p = 0; p < 4; ++p) {
                const uint32_t t = (wv[j] >> (2 * p + 8 * h)) & 0x00030003u;
                ac = __builtin_amdgcn_fdot2(as_h2(w2_centroid_pair(t)),
                                            as_h2(xr[i][8 * j + 4 * h + p]), ac, false);
              }
          acc = __builtin_fmaf(s, ac, acc);
          acc = __builtin_fmaf(z, sx[i], acc);
        }
      }
      if (HAS_OUT && do_out) {
#pragma unroll
        for (int t = 0; t < kOutRegs; ++t) acc = __builtin_fmaf(h2f(b.ow[u][t]), h2f(xo[t]), acc);
        for (int j = n_cap + kw * kWave + lane; j < a.n_out; j += jstride) {
          const uint32_t c = (uint32_t)a.out_idx[j];
          const float xv = c < (uint32_t)a.K ? h2f(a.x[c]) : 0.f;
          acc = __builtin_fmaf(h2f(ld16(ors, ((uint32_t)rl * (uint32_t)a.n_out + (uint32_t)j) * 2u)),
                               xv, acc);
        }
      }
      acc = row16_sum(acc);
      if ((lane & 15) == 0) s_part[(rl * a.wk + kw) * 4 + (lane >> 4)] = acc;
    }
  }
  __syncthreads();
  for (int t = tid; t < rows_here; t += nthr) {
    float s = 0.f;
    for (int k = 0; k < a.wk; ++k) {
      const float* p = s_part + (t * a.wk + k) * 4;
      s += (p[0] + p[1]) + (p[2] + p[3]);
    }
    a.y[tile0 + t] = f2h(s);
  }
}

// ------------------------------------------------------------- launch plan

struct GemvPlan {
  int gpl, wk, wr, rpw, rt, blocks, xc;
  size_t lds;
  bool lds_path;   // gemv_lds_kernel (x and the W2 table in LDS) or gemv_reg_kernel
};

static GemvPlan plan_gemv(int fmt, int64_t N, int64_t K, int64_t n_out, const wq_variant* v) {
  const int G = (int)(K / kGroup);
  GemvPlan p{};
  // Fewest idle lanes, at most 8 K-waves; on a tie prefer 2 groups per lane,
  // then 1, then 4.
  int best = -1;
  for (int gpl : {2, 1, 4}) {
    const int wk = (G + kWave * gpl - 1) / (kWave * gpl);
    if (wk > 8) continue;
    const int waste = wk * kWave * gpl - G;
    if (best < 0 || waste < best) {
      best = waste;
      p.gpl = gpl;
      p.wk = wk;
    }
  }
  p.wr = p.wk >= 4 ? 1 : 4 / p.wk;
  // Rows per wave step: the fewest rows on the busiest compute unit (blocks
  // spread evenly over the units), the most rows per wave among equals.
  // Measured on the decode step's small layers: q|k|v 6144 x 4096 takes 3
  // (6.0 -> 5.7 us), k / v 1024 x 4096 takes 1 (4.0 -> 3.4 us).
  p.rpw = kRowsPerStep;
  const int cus = device_cus() > 0 ? device_cus() : 256;
  int64_t best_rows = -1;
  for (int r = kRowsPerStep; r >= 1; --r) {
    const int64_t rt = (int64_t)p.wr * r;
    const int64_t blocks = (N + rt - 1) / rt;
    const int64_t rows = (blocks + cus - 1) / cus * rt;
    if (best_rows < 0 || rows < best_rows) {
      best_rows = rows;
      p.rpw = r;
    }
  }
  const int rpw = variant_or(v, &wq_variant::gemv_rows_per_wave, p.rpw);
  if (rpw >= 1 && rpw <= kRowsPerStep) p.rpw = rpw;
  p.rt = p.wr * p.rpw;
  p.blocks = (int)((N + p.rt - 1) / p.rt);
  const size_t part = (size_t)16 * p.rt * p.wk;
  p.lds = gemv_lds_bytes((int)K, p.rt, p.wk, (int)n_out, n_out > 0, fmt);
  p.lds_path = p.lds <= kMaxLdsBytes;
  // the W2 pairing of consecutive groups needs an even group count
  if (fmt == 2 && p.gpl % 2 == 0 && G % 2 != 0) p.lds_path = false;
  p.lds_path = p.lds_path && variant_or(v, &wq_variant::gemv_lds_x, 1) != 0;
  if (!p.lds_path) p.lds = std::max((size_t)4 * G, part);
  // 16-byte chunks of x per thread, loaded before the weights
  const int nthr = p.wk * p.wr * kWave;
  const int64_t chunks = (K / 8 + nthr - 1) / nthr;
  p.xc = chunks <= 2 ? 2 : chunks <= 4 ? 4 : 8;
  return p;
}

template <int FMT>
static int launch_gemv(const GemvArgs& a0, hipStream_t stream, const char* who,
                       const wq_variant* v) {
  GemvArgs a = a0;
  const GemvPlan p = plan_gemv(FMT, a.N, a.K, a.n_out, v);
  if (p.gpl == 0) return wq::fail(WQ_ERR_UNSUPPORTED, "%s: K=%d not supported", who, a.K);
  if (p.lds > kMaxLdsBytes)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: %zu bytes of LDS needed", who, p.lds);
  a.wk = p.wk;
  a.wr = p.wr;
  a.rpw = p.rpw;
  const dim3 grid(p.blocks), block(p.wk * p.wr * kWave);
  const bool out = a.n_out > 0;
#define WQ_GEMV_LAUNCH(KERNEL)                                                                \
  do {                                                                                       \
    if (!allow_lds(reinterpret_cast<const void*>(&KERNEL), p.lds))                          \
      return wq::fail(WQ_ERR_HIP, "%s: cannot raise the LDS limit to %zu bytes", who, p.lds); \
    hipLaunchKernelGGL(KERNEL, grid, block, p.lds, stream, a);                               \
  } while (0)
#define WQ_GEMV_CASE(G_, O_)                                                                 \
  if (p.gpl == G_ && out == O_) {                                                            \
    if (!p.lds_path)                                                                         \
      WQ_GEMV_LAUNCH((gemv_reg_kernel<FMT, G_, O_>));                                        \
    else if (p.xc == 2)                                                                      \
      WQ_GEMV_LAUNCH((gemv_lds_kernel<FMT, G_, O_, 2>));                                     \
    else if (p.xc == 4)                                                                      \
      WQ_GEMV_LAUNCH((gemv_lds_kernel<FMT, G_, O_, 4>));                                     \
    else                                                                                     \
      WQ_GEMV_LAUNCH((gemv_lds_kernel<FMT, G_, O_, 8>));                                     \
    return check_launch(who);                                                                \
  }
  WQ_GEMV_CASE(1, false) WQ_GEMV_CASE(1, true) WQ_GEMV_CASE(2, false) WQ_GEMV_CASE(2, true)
  WQ_GEMV_CASE(4, false) WQ_GEMV_CASE(4, true)
#undef WQ_GEMV_CASE
#undef WQ_GEMV_LAUNCH
  return wq::fail(WQ_ERR_UNSUPPORTED, "%s: no kernel for this shape", who);
}

}  // namespace wqd

using namespace wqd;

static int gemv_entry(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                      int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
                      int64_t n_out, uint32_t flags, const uint16_t* x, uint16_t* y,
                      const wq_variant* v, void* stream, const char* who) {
  if (int r = wq::check_shape(N, K, who)) return r;
  if (int r = wq::check_outlier_args(out_idx, out_w, n_out, K, who)) return r;
  if (!codes || !scales || !zeros || !x || !y)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(zeros) || !aligned16(x) ||
      !aligned16(y) || (n_out > 0 && (!aligned16(out_idx) || !aligned16(out_w))))
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: device pointers must be 16-byte aligned", who);
  GemvArgs a{};
  a.codes = codes;
  a.scales = scales;
  a.zeros = zeros;
  a.out_idx = out_idx;
  a.out_w = out_w;
  a.x = x;
  a.y = y;
  a.N = (int)N;
  a.K = (int)K;
  a.n_out = (int)n_out;
  a.fuse = (flags & WQ_FUSE_OUTLIERS) ? 1 : 0;
  hipStream_t s = (hipStream_t)stream;
  // the matrix-core kernel fuses the outlier pass; an unfused call with
  // outlier columns stays on the VALU kernels
  if (a.fuse || n_out == 0) {
    const int mode = variant_or(v, &wq_variant::gemv_kernel, 1);
    bool launched = false;
    const int r = wqd_gemv_mma(fmt, false, codes, scales, zeros, N, K, out_idx, out_w,
                               a.fuse ? n_out : 0, x, y, s, who, mode, &launched);
    if (r != WQ_OK || launched) return r;
  }
  return fmt == 4 ? launch_gemv<4>(a, s, who, v)
                  : fmt == 5 ? launch_gemv<5>(a, s, who, v) : launch_gemv<2>(a, s, who, v);
}

extern "C" int wq_gemv_v(int fmt, const uint8_t* codes, const uint16_t* scales,
                         const uint16_t* zeros, int64_t N, int64_t K, const int32_t* out_idx,
                         const uint16_t* out_w, int64_t n_out, uint32_t flags, const uint16_t* x,
                         uint16_t* y, const wq_variant* variant, void* stream) {
  if (fmt != WQ_FMT_W4 && fmt != WQ_FMT_W2 && fmt != WQ_FMT_W4P)
    return wq::fail(WQ_ERR_INVALID_ARG, "wq_gemv_v: fmt must be WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2");
  return gemv_entry(fmt, codes, scales, zeros, N, K, out_idx, out_w, n_out, flags, x, y, variant,
                    stream, "wq_gemv_v");
}

extern "C" int wq_gemv_w4(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                          int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
                          int64_t n_out, uint32_t flags, const uint16_t* x, uint16_t* y,
                          void* stream) {
  return gemv_entry(4, codes, scales, zeros, N, K, out_idx, out_w, n_out, flags, x, y, nullptr,
                    stream, "wq_gemv_w4");
}

extern "C" int wq_gemv_w4p(const uint8_t* codes, const uint16_t* scales,
                           const uint8_t* zeros_packed, int64_t N, int64_t K,
                           const int32_t* out_idx, const uint16_t* out_w, int64_t n_out,
                           uint32_t flags, const uint16_t* x, uint16_t* y, void* stream) {
  return gemv_entry(5, codes, scales, reinterpret_cast<const uint16_t*>(zeros_packed), N, K,
                    out_idx, out_w, n_out, flags, x, y, nullptr, stream, "wq_gemv_w4p");
}

extern "C" int wq_gemv_w2(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                          int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
                          int64_t n_out, uint32_t flags, const uint16_t* x, uint16_t* y,
                          void* stream) {
  return gemv_entry(2, codes, scales, zeros, N, K, out_idx, out_w, n_out, flags, x, y, nullptr,
                    stream, "wq_gemv_w2");
}

extern "C" int wq_gemm_tiled_v(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                               const int32_t* out_idx, int64_t n_out, const uint16_t* X, int64_t M,
                               uint16_t* Y, const wq_variant* variant, void* stream) {
  const char* who = "wq_gemm_tiled";
  if (fmt != WQ_FMT_W4 && fmt != WQ_FMT_W2 && fmt != WQ_FMT_W4P)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: fmt must be WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2", who);
  if (int r = wq::check_shape(N, K, who)) return r;
  if (n_out < 0 || n_out > K)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: n_out must be in [0, K] (got %lld)", who,
                    (long long)n_out);
  if (M < 1) return wq::fail(WQ_ERR_INVALID_ARG, "%s: M must be >= 1", who);
  if (M > WQ_GEMM_MAX_M)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: M above %d is not supported", who, WQ_GEMM_MAX_M);
  if (!tiled || !X || !Y || (n_out > 0 && !out_idx))
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(tiled) || !aligned16(X) || !aligned16(Y) || (n_out > 0 && !aligned16(out_idx)))
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: device pointers must be 16-byte aligned", who);
  bool launched = false;
  // up to four rows (W2: two): the M = 1 kernel with its group slots shared
  // by the rows; else the batched kernel on the same tiles
  if (M == 1 || variant_or(variant, &wq_variant::gemm_rows, 1) != 0) {
    const int r = wqd_mma_rows(fmt, true, tiled, nullptr, nullptr, N, K, out_idx, nullptr, n_out,
                               X, M, Y, (hipStream_t)stream, who, 2, &launched);
    if (r != WQ_OK || launched) return r;
  }
  if (M >= 2) {
    const int r = wqd_gemm_mma_tiled(fmt, tiled, N, K, out_idx, n_out, X, M, Y, variant,
                                     (hipStream_t)stream, who, &launched);
    if (r != WQ_OK || launched) return r;
  }
  return wq::fail(WQ_ERR_UNSUPPORTED,
                  "%s: shape not supported by the tiled kernels at M = %lld (K <= 32768, at most "
                  "32 outlier positions per 512-channel slice, at most 1024 outlier columns for "
                  "M > 1, partial sums within the LDS)", who, (long long)M);
}

extern "C" int wq_gemm_tiled(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                             const int32_t* out_idx, int64_t n_out, const uint16_t* X, int64_t M,
                             uint16_t* Y, void* stream) {
  return wq_gemm_tiled_v(fmt, tiled, N, K, out_idx, n_out, X, M, Y, nullptr, stream);
}

extern "C" int wq_gemv_tiled(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                             const int32_t* out_idx, int64_t n_out, const uint16_t* x,
                             uint16_t* y, void* stream) {
  const char* who = "wq_gemv_tiled";
  if (fmt != WQ_FMT_W4 && fmt != WQ_FMT_W2 && fmt != WQ_FMT_W4P)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: fmt must be WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2", who);
  if (int r = wq::check_shape(N, K, who)) return r;
  if (n_out < 0 || n_out > K)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: n_out must be in [0, K] (got %lld)", who,
                    (long long)n_out);
  if (!tiled || !x || !y || (n_out > 0 && !out_idx))
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(tiled) || !aligned16(x) || !aligned16(y) || (n_out > 0 && !aligned16(out_idx)))
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: device pointers must be 16-byte aligned", who);
  bool launched = false;
  const int r = wqd_gemv_mma(fmt, true, tiled, nullptr, nullptr, N, K, out_idx, nullptr, n_out, x,
                             y, (hipStream_t)stream, who, 2, &launched);
  if (r != WQ_OK) return r;
  if (!launched)
    return wq::fail(WQ_ERR_UNSUPPORTED,
                    "%s: shape not supported by the tiled kernel (K <= 32768 and at most 32 "
                    "outlier positions per 512-channel slice)", who);
  return WQ_OK;
}

extern "C" int wq_gemv_tiled_refine_v(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                                      const int32_t* out_idx, int64_t n_out, const uint16_t* x,
                                      uint16_t* y, const uint8_t* rcodes, const uint16_t* rscales,
                                      const uint16_t* rzeros, int64_t chunk, int64_t k,
                                      int32_t* sel_out, const wq_variant* variant, void* stream) {
  const char* who = "wq_gemv_tiled_refine";
  if (fmt != WQ_FMT_W4 && fmt != WQ_FMT_W2 && fmt != WQ_FMT_W4P)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: fmt must be WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2", who);
  if (int r = wq::check_shape(N, K, who)) return r;
  if (n_out < 0 || n_out > K)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: n_out must be in [0, K] (got %lld)", who,
                    (long long)n_out);
  if (N % 32) return wq::fail(WQ_ERR_UNSUPPORTED, "%s: N must be a multiple of 32", who);
  if (chunk < 64 || chunk > 1024 || chunk % 64)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: chunk must be a multiple of 64 in [64, 1024]", who);
  if (k < 0) return wq::fail(WQ_ERR_INVALID_ARG, "%s: k must be >= 0", who);
  if (k == 0) return wq_gemv_tiled(fmt, tiled, N, K, out_idx, n_out, x, y, stream);
  if (!tiled || !x || !y || (n_out > 0 && !out_idx) || !rcodes || !rscales || !rzeros)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(tiled) || !aligned16(x) || !aligned16(y) || (n_out > 0 && !aligned16(out_idx)) ||
      !aligned16(rcodes))
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: device pointers must be 16-byte aligned", who);
  if ((uint64_t)K * (uint64_t)N / 2 > 0xFFFFE000ull)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: refinement larger than 4 GB", who);
  if (variant_or(variant, &wq_variant::refine_fuse, 1) != 0) {
    bool launched = false;
    const int r = wqd_gemv_refine_mma(fmt, tiled, N, K, out_idx, n_out, x, y, rcodes, rscales,
                                      rzeros, chunk, k, sel_out, variant, (hipStream_t)stream, who,
                                      &launched);
    if (r != WQ_OK || launched) return r;
  }
  // two launches: the product (rounded to FP16), then the selection and the add
  if (int r = wq_gemv_tiled(fmt, tiled, N, K, out_idx, n_out, x, y, stream)) return r;
  return wq_refine_topk_v(rcodes, rscales, rzeros, N, K, chunk, k, x, y, sel_out, variant, stream);
}

extern "C" int wq_gemv_tiled_refine(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                                    const int32_t* out_idx, int64_t n_out, const uint16_t* x,
                                    uint16_t* y, const uint8_t* rcodes, const uint16_t* rscales,
                                    const uint16_t* rzeros, int64_t chunk, int64_t k,
                                    int32_t* sel_out, void* stream) {
  return wq_gemv_tiled_refine_v(fmt, tiled, N, K, out_idx, n_out, x, y, rcodes, rscales, rzeros,
                                chunk, k, sel_out, nullptr, stream);
}
