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

#include <stdlib.h>

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
  if constexpr (FMT == 4) {
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

constexpr int kPrepSlots = 2;   // groups of activations each thread prepares in LDS

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

// XLDS: the workgroup prepares the masked, paired activations once in LDS
// and every wave reads its slice (otherwise each lane prepares its own).
template <int FMT, int GPL, bool HAS_OUT, bool XLDS>
__global__ void __launch_bounds__(512) gemv_kernel(GemvArgs a) {
  typedef Fmt<FMT> F;
  extern __shared__ __align__(16) unsigned char smem[];
  const int G = a.K / kGroup;
  const int RT = a.wr * a.rpw;
  // LDS: [mask / partial sums (aliased: the mask is dead before partials are
  // written)] [per-group activation sums] [paired activations, 64 B a group]
  const int head = max(4 * G, 16 * RT * a.wk);
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(smem);                 // [G] outlier bits
  float* s_part = reinterpret_cast<float*>(smem);                       // [RT][wk][4]
  float* s_sx = reinterpret_cast<float*>(smem + head);                  // [G]
  u4v* s_xp = reinterpret_cast<u4v*>(smem + ((head + 4 * G + 15) & ~15));   // [G][4]

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
  constexpr int XS = XLDS ? kPrepSlots : GPL;
  uint32_t xw[XS][16];
#pragma unroll
  for (int i = 0; i < XS; ++i) {
    const uint32_t g = XLDS ? (uint32_t)(tid + nthr * i) : (uint32_t)((kw * GPL + i) * kWave + lane);
    load_group_x(xrs, g < (uint32_t)G ? g * 64u : kOob, xw[i]);
  }
  const uint64_t row_bytes = (uint64_t)a.K / F::kRowBytesPerK;
  const __amdgpu_buffer_rsrc_t crs =
      make_rsrc(a.codes + (uint64_t)tile0 * row_bytes, clamp_bytes((uint64_t)rows_here * row_bytes));
  const __amdgpu_buffer_rsrc_t srs =
      make_rsrc(a.scales + (uint64_t)tile0 * G, clamp_bytes((uint64_t)rows_here * G * 2));
  const __amdgpu_buffer_rsrc_t zrs =
      make_rsrc(a.zeros + (uint64_t)tile0 * G, clamp_bytes((uint64_t)rows_here * G * 2));
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(
      do_out ? a.out_w + (uint64_t)tile0 * a.n_out : a.out_w,
      do_out ? clamp_bytes((uint64_t)rows_here * a.n_out * 2) : 0u);
  bool gvalid[GPL];
#pragma unroll
  for (int i = 0; i < GPL; ++i) gvalid[i] = (kw * GPL + i) * kWave + lane < G;

  RowBatch<FMT, GPL> b;
#pragma unroll
  for (int u = 0; u < kRowsPerStep; ++u) {
    const bool rv = r_first + u < r_end;
    const uint32_t rl = (uint32_t)(r_first + u);
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const uint32_t g = (uint32_t)((kw * GPL + i) * kWave + lane);
      const bool ok = rv && gvalid[i];
      const uint32_t co = ok ? rl * (uint32_t)row_bytes + g * F::kGroupBytes : kOob;
      const uint32_t mo = ok ? (rl * (uint32_t)G + g) * 2u : kOob;
      if constexpr (FMT == 4)
        b.cw[u][i] = ld128(crs, co);
      else
        b.cw[u][i] = ld64(crs, co);
      b.sv[u][i] = ld16(srs, mo);
      b.zv[u][i] = ld16(zrs, mo);
    }
    if constexpr (HAS_OUT) {
#pragma unroll
      for (int t = 0; t < kOutRegs; ++t) {
        const int j = (kw + a.wk * t) * kWave + lane;
        const bool ok = rv && oval[t];
        b.ow[u][t] = ld16(ors, ok ? (rl * (uint32_t)a.n_out + (uint32_t)j) * 2u : kOob);
      }
    }
  }

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
  if constexpr (XLDS) {
#pragma unroll
    for (int i = 0; i < XS; ++i) {
      const int g = tid + nthr * i;
      if (g < G) {
        uint32_t pr[16];
        float sum;
        pair_group<FMT>(xw[i], HAS_OUT ? s_mask[g] : 0u, pr, sum);
#pragma unroll
        for (int v = 0; v < 4; ++v) s_xp[g * 4 + v] = (u4v){pr[4 * v], pr[4 * v + 1], pr[4 * v + 2], pr[4 * v + 3]};
        s_sx[g] = sum;
      }
    }
    for (int g = tid + nthr * XS; g < G; g += nthr) {   // only when K > 64 * 512 * ...
      uint32_t w2[16], pr[16];
      float sum;
      load_group_x(xrs, (uint32_t)g * 64u, w2);
      pair_group<FMT>(w2, HAS_OUT ? s_mask[g] : 0u, pr, sum);
#pragma unroll
      for (int v = 0; v < 4; ++v) s_xp[g * 4 + v] = (u4v){pr[4 * v], pr[4 * v + 1], pr[4 * v + 2], pr[4 * v + 3]};
      s_sx[g] = sum;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int g = (kw * GPL + i) * kWave + lane;
      const int gg = gvalid[i] ? g : 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const u4v t = s_xp[gg * 4 + v];
        xr[i][4 * v + 0] = t.x;
        xr[i][4 * v + 1] = t.y;
        xr[i][4 * v + 2] = t.z;
        xr[i][4 * v + 3] = t.w;
      }
      sx[i] = s_sx[gg];
    }
  } else {
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int g = (kw * GPL + i) * kWave + lane;
      const uint32_t m = !gvalid[i] ? 0xFFFFFFFFu : (HAS_OUT ? s_mask[g] : 0u);
      pair_group<FMT>(xw[i], m, xr[i], sx[i]);
    }
  }

  // ---- (5) the rows (s_part aliases s_mask: wait until every wave has read its mask)
  if constexpr (HAS_OUT && !XLDS) lds_barrier();
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
        const float z = h2f(b.zv[u][i]);
        if constexpr (FMT == 4) {
          float alo = 0.f, ahi = 0.f;
          const uint32_t wv[4] = {b.cw[u][i].x, b.cw[u][i].y, b.cw[u][i].z, b.cw[u][i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t lo0, hi0, lo1, hi1;
            w4_word_sub(wv[j], lo0, hi0, lo1, hi1);
            alo = __builtin_amdgcn_fdot2(as_h2(lo0), as_h2(xr[i][4 * j + 0]), alo, false);
            ahi = __builtin_amdgcn_fdot2(as_h2(hi0), as_h2(xr[i][4 * j + 1]), ahi, false);
            alo = __builtin_amdgcn_fdot2(as_h2(lo1), as_h2(xr[i][4 * j + 2]), alo, false);
            ahi = __builtin_amdgcn_fdot2(as_h2(hi1), as_h2(xr[i][4 * j + 3]), ahi, false);
          }
          // sum q x = 2^24 (alo + ahi / 16); then (sum q x - z sum x) s
          float v = __builtin_fmaf(ahi, 0.0625f, alo) * 16777216.0f;
          v = __builtin_fmaf(-z, sx[i], v);
          acc = __builtin_fmaf(s, v, acc);
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
  int gpl, wk, wr, rpw, rt, blocks;
  size_t lds, lds_reg;
  bool xlds;
};

static GemvPlan plan_gemv(int64_t N, int64_t K, int64_t n_out) {
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
  // One batch of at most 4 rows per wave; fewer rows per wave when that is
  // what it takes to have ~1024 workgroups in flight.
  p.rpw = kRowsPerStep;
  while (p.rpw > 1 && (N + (int64_t)p.wr * p.rpw - 1) / ((int64_t)p.wr * p.rpw) < 1024) p.rpw /= 2;
  if (const char* e = getenv("WQ_GEMV_ROWS_PER_WAVE")) {
    const int v = atoi(e);
    if (v >= 1 && v <= kRowsPerStep) p.rpw = v;
  }
  p.rt = p.wr * p.rpw;
  p.blocks = (int)((N + p.rt - 1) / p.rt);
  const size_t head = std::max((size_t)4 * G, (size_t)16 * p.rt * p.wk);
  p.lds_reg = head;
  p.lds = ((head + (size_t)4 * G + 15) & ~(size_t)15) + (size_t)64 * G;
  p.xlds = p.lds <= kMaxLdsBytes;
  if (const char* e = getenv("WQ_GEMV_XLDS")) p.xlds = p.xlds && atoi(e) != 0;
  if (!p.xlds) p.lds = p.lds_reg;
  return p;
}

template <int FMT>
static int launch_gemv(const GemvArgs& a0, hipStream_t stream, const char* who) {
  GemvArgs a = a0;
  const GemvPlan p = plan_gemv(a.N, a.K, a.n_out);
  if (p.gpl == 0) return wq::fail(WQ_ERR_UNSUPPORTED, "%s: K=%d not supported", who, a.K);
  if (p.lds > kMaxLdsBytes)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: %zu bytes of LDS needed (n_out too large)", who, p.lds);
  a.wk = p.wk;
  a.wr = p.wr;
  a.rpw = p.rpw;
  const dim3 grid(p.blocks), block(p.wk * p.wr * kWave);
  const bool out = a.n_out > 0;
#define WQ_GEMV_CASE(G_, O_, X_)                                                           \
  if (p.gpl == G_ && out == O_ && p.xlds == X_) {                                          \
    hipLaunchKernelGGL((gemv_kernel<FMT, G_, O_, X_>), grid, block, p.lds, stream, a);     \
    return check_launch(who);                                                              \
  }
  WQ_GEMV_CASE(1, false, true) WQ_GEMV_CASE(1, true, true) WQ_GEMV_CASE(1, false, false)
  WQ_GEMV_CASE(1, true, false) WQ_GEMV_CASE(2, false, true) WQ_GEMV_CASE(2, true, true)
  WQ_GEMV_CASE(2, false, false) WQ_GEMV_CASE(2, true, false) WQ_GEMV_CASE(4, false, true)
  WQ_GEMV_CASE(4, true, true) WQ_GEMV_CASE(4, false, false) WQ_GEMV_CASE(4, true, false)
#undef WQ_GEMV_CASE
  return check_launch(who);
}

}  // namespace wqd

using namespace wqd;

static int gemv_entry(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                      int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
                      int64_t n_out, uint32_t flags, const uint16_t* x, uint16_t* y,
                      void* stream, const char* who) {
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
  return fmt == 4 ? launch_gemv<4>(a, s, who) : launch_gemv<2>(a, s, who);
}

extern "C" int wq_gemv_w4(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                          int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
                          int64_t n_out, uint32_t flags, const uint16_t* x, uint16_t* y,
                          void* stream) {
  return gemv_entry(4, codes, scales, zeros, N, K, out_idx, out_w, n_out, flags, x, y, stream,
                    "wq_gemv_w4");
}

extern "C" int wq_gemv_w2(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                          int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
                          int64_t n_out, uint32_t flags, const uint16_t* x, uint16_t* y,
                          void* stream) {
  return gemv_entry(2, codes, scales, zeros, N, K, out_idx, out_w, n_out, flags, x, y, stream,
                    "wq_gemv_w2");
}
