// Exact per-chunk top-k selection by |x| on one wave (StrataFlux page,
// section 3.2.1, "Channel selection"), shared by the refinement kernels and
// the GEMV that fuses the refinement add.
//
// Lane l holds channels 16l .. 16l + 15 of the chunk.  The k-th largest FP16
// magnitude T comes from two histogram passes in the wave's own LDS (the top 7
// bits of the 15-bit magnitude, then the low 8 bits inside the chosen bin);
// every channel above T is kept, and of those equal to T the lowest-indexed
// ones, counted by a wave prefix sum, fill the rest.  The picks are written in
// index order.  Only wave-level LDS ordering is used, no block barrier; the
// bin each pass finds is passed to the other lanes by ballot and readlane, not
// through LDS, and the histograms are cleared before the chunk's values are
// waited for.
#pragma once

#include "wq_common.cuh"

namespace wqd {

constexpr uint32_t kSelOob = 0xFFFFF000u;     // past every buffer: loads return 0
constexpr int kSelBins1 = 128;                // magnitude bits 14..8
constexpr int kSelBins2 = 256;                // magnitude bits 7..0
constexpr int kSelWords = kSelBins1 + kSelBins2;       // per wave: both histograms

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Per wave (all 64 lanes active): the sum of v over the lanes below this one,
// and over all lanes in `total`.  Inclusive scan with DPP: shifts by 1, 2, 4, 8
// inside each row of 16 lanes, then the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ uint32_t wave_excl_sum(uint32_t v, uint32_t& total) {
  const int lane = (int)__lane_id();
  const int rl = lane & 15;
  uint32_t r = v, t;
  t = dpp_mov<0x111>(r);   // row_shr:1
  if (rl >= 1) r += t;
  t = dpp_mov<0x112>(r);   // row_shr:2
  if (rl >= 2) r += t;
  t = dpp_mov<0x114>(r);   // row_shr:4
  if (rl >= 4) r += t;
  t = dpp_mov<0x118>(r);   // row_shr:8
  if (rl >= 8) r += t;
  t = dpp_mov<0x142>(r);   // row_bcast:15
  if ((lane & 31) >= 16) r += t;
  t = dpp_mov<0x143>(r);   // row_bcast:31
  if (lane >= 32) r += t;
  total = (uint32_t)__builtin_amdgcn_readlane((int)r, 63);
  return r - v;
}

// One wave: of the csize channels c0 .. c0 + csize - 1 (csize a multiple of 16,
// at most 1024), the kk of largest |x| with ties to the lower index, written
// ascending to out[0 .. kk), and with outx the picks' FP16 values beside them.
// Lane l holds channels c0 + 16 l .. c0 + 16 l + 15 in wv (two FP16 values per
// word, the lower channel in the low half); lanes past csize hold anything.
// hist: this wave's kSelWords words of LDS.
template <bool WITH_X>
__device__ __forceinline__ void wave_topk_regs(const uint32_t (&wv)[8], int c0, int csize, int kk,
                                               uint32_t* hist, int32_t* out, uint16_t* outx,
                                               int lane) {
  const bool valid = 16 * lane < csize;
  const bool all = kk >= csize;
  const bool part = !all && kk > 0;
  uint32_t* h1 = hist;
  uint32_t* h2 = hist + kSelBins1;
  if (part) {
    h1[lane] = 0u;
    h1[lane + kWave] = 0u;
#pragma unroll
    for (int i = 0; i < kSelBins2 / kWave; ++i) h2[lane + kWave * i] = 0u;
  }
  // the clearing stays ahead of the first use of wv (and of its wait)
  __builtin_amdgcn_sched_barrier(0);
  uint32_t m[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m[2 * i] = wv[i] & 0x7FFFu;
    m[2 * i + 1] = (wv[i] >> 16) & 0x7FFFu;
  }
  uint32_t T = 0u, keq = 0u;   // keep |x| > T, and the first keq channels with |x| == T
  if (part) {
    wave_lds_sync();
    if (valid) {
#pragma unroll
      for (int e = 0; e < 16; ++e) atomicAdd(&h1[m[e] >> 8], 1u);
    }
    wave_lds_sync();
    uint32_t b1, rem;
    {
      // lane l holds bins 2l (lower) and 2l + 1 (higher); exactly one bin holds
      // the kk-th largest (1 <= kk < number of valid channels), and the one
      // lane that holds it passes the bin and the rank inside it on
      const uint32_t rk = (uint32_t)kk;
      const uint32_t lo = h1[2 * lane], hi = h1[2 * lane + 1];
      uint32_t tot;
      const uint32_t below = wave_excl_sum(lo + hi, tot);
      const uint32_t suf = tot - below;                     // bins >= 2l
      const uint32_t above = suf - lo - hi;                 // bins >= 2l + 2
      const bool in_hi = above < rk && rk <= above + hi;
      const bool in_lo = above + hi < rk && rk <= suf;
      const uint32_t bin = in_hi ? 2u * lane + 1u : 2u * lane;
      const uint32_t r1 = in_hi ? rk - above : rk - above - hi;
      const int src = (int)__builtin_ctzll(__ballot(in_hi || in_lo) | (1ull << 63));
      b1 = (uint32_t)__builtin_amdgcn_readlane((int)bin, src);
      rem = (uint32_t)__builtin_amdgcn_readlane((int)r1, src);
    }
    if (valid) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if ((m[e] >> 8) == b1) atomicAdd(&h2[m[e] & 0xFFu], 1u);
    }
    wave_lds_sync();
    {
      uint32_t hb[4], sum = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hb[i] = h2[4 * lane + i];
        sum += hb[i];
      }
      uint32_t tot;
      const uint32_t below = wave_excl_sum(sum, tot);
      uint32_t cum = tot - below - sum;                     // bins >= 4l + 4
      uint32_t tv = 0u, qv = 0u;
      bool found = false;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (cum < rem && rem <= cum + hb[i]) {
          tv = (b1 << 8) | (uint32_t)(4 * lane + i);
          qv = rem - cum;
          found = true;
        }
        cum += hb[i];
      }
      const int src = (int)__builtin_ctzll(__ballot(found) | (1ull << 63));
      T = (uint32_t)__builtin_amdgcn_readlane((int)tv, src);
      keq = (uint32_t)__builtin_amdgcn_readlane((int)qv, src);
    }
  }
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const bool g = valid && (all || (kk > 0 && m[e] > T));
    const bool q = valid && !all && kk > 0 && m[e] == T;
    gt |= (uint32_t)g << e;
    eq |= (uint32_t)q << e;
  }
  const uint32_t neq = (uint32_t)__builtin_popcount(eq);
  uint32_t tot;
  const uint32_t eq_before = wave_excl_sum(neq, tot);
  uint32_t keep = gt;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t rank = eq_before + (uint32_t)__builtin_popcount(eq & ((1u << e) - 1u));
    if (((eq >> e) & 1u) && rank < keq) keep |= 1u << e;
  }
  const uint32_t cnt = (uint32_t)__builtin_popcount(keep);
  uint32_t pos = wave_excl_sum(cnt, tot);
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if ((keep >> e) & 1u) {
      if (pos < (uint32_t)kk) {   // never past the chunk's picks
        out[pos] = c0 + 16 * lane + e;
        if constexpr (WITH_X) outx[pos] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
      }
      ++pos;
    }
}


// The same, reading the chunk from x through a buffer resource.
__device__ __forceinline__ void wave_chunk_topk(__amdgpu_buffer_rsrc_t xrs, int c0, int csize, int kk,
                                uint32_t* hist, int32_t* out, int lane) {
  const uint32_t off = 16 * lane < csize ? (uint32_t)(c0 + 16 * lane) * 2u : kSelOob;
  const u4v a = ld128(xrs, off), b = ld128(xrs, off + 16u);
  const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  wave_topk_regs<false>(wv, c0, csize, kk, hist, out, nullptr, lane);
}

}  // namespace wqd
