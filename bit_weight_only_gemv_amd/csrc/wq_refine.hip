// Runtime top-k refinement (StrataFlux page, section 3.2.1, "Channel
// selection" and Eq. 2), for gfx950:
//
//   S(x) = in each chunk of `chunk` input channels, the k channels of largest
//          |x_i| (ties to the lower index, each chunk's picks ascending);
//   y'   = y + sum_{i in S(x)} x_i C[:, i],
//
// where C holds 4-bit refinement columns: the residual of the resident layer
// stored per input channel (C transposed, [K][N]) in the W4 format along N
// (groups of 32 output rows, FP16 scale and zero, in-group nibble interleave).
//
// topk_kernel: one workgroup per chunk.  The selection is an exact radix
// select on 26-bit keys ((|x| bits << 10 | 1023 - local index) + 1, unique
// per chunk, so ties go to the lower index); the kept channels are then
// written in index order through a block-wide prefix count.
//
// refine_kernel: a workgroup owns 64 output rows (2 groups of 32) and splits
// the selected columns over 32 slots of 8 threads; thread (slot, group,
// quarter) decodes 4 code bytes, 8 rows, of columns j = slot, slot + 32, ...
// with four columns' loads in flight at a time.  The slots' partial sums are
// added in a fixed order and added once into the FP16 output.

#include "wq_common.cuh"
#include "wq_device.h"

namespace wqd {

constexpr int kTopkThreads = 256;
constexpr int kRadixBits = 7;
constexpr int kRadixBins = 1 << kRadixBits;   // 128
constexpr int kRefineThreads = 256;
constexpr int kRefineRows = 64;               // 2 groups of 32 rows per workgroup
constexpr int kRefineSlots = kRefineThreads / 8;   // columns in flight per workgroup
constexpr int kRefineUnroll = 4;              // columns per slot with loads in flight
constexpr uint32_t kOobR = 0xFFFFF000u;       // past every buffer: loads return 0

// Per wave: inclusive suffix sums over lanes (lane l gets the sum of lanes >= l).
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t t = __shfl_down(v, d);
    if (lane + d < kWave) v += t;
  }
  return v;
}

// Per wave: inclusive prefix sums over lanes.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const uint16_t* __restrict__ x,
                                                           int K, int chunk, int k,
                                                           int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[kRadixBins];
  __shared__ uint32_t s_state[2];            // [0] key prefix, [1] rank still wanted
  __shared__ uint32_t s_wave[kTopkThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int c = blockIdx.x;
  const int c0 = c * chunk;
  const int csize = min(chunk, K - c0);
  const int kk = min(k, csize);

  // four consecutive channels per thread; past the chunk or K: key 0
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (uint32_t)K * 2u);
  const int j0 = 4 * tid;
  const u2 xv = ld64(xrs, j0 < csize ? (uint32_t)(c0 + j0) * 2u : kOobR);
  const uint32_t h[4] = {xv.x & 0xFFFFu, xv.x >> 16, xv.y & 0xFFFFu, xv.y >> 16};
  uint32_t key[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = j0 + e;
    key[e] = j < csize ? (((h[e] & 0x7FFFu) << 10) | (uint32_t)(1023 - j)) + 1u : 0u;
  }

  // ---- radix select of the kk-th largest key: 4 passes of 7 bits (bits 27..0)
  uint32_t thr = 1u;   // kk == csize: every valid key (>= 1) is kept
  if (kk > 0 && kk < csize) {
    if (tid == 0) {
      s_state[0] = 0u;
      s_state[1] = (uint32_t)kk;
    }
    uint32_t pmask = 0u;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 21 - kRadixBits * pass;
      if (tid < kRadixBins) hist[tid] = 0u;
      __syncthreads();
      const uint32_t prefix = s_state[0];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (key[e] != 0u && (key[e] & pmask) == prefix)
          atomicAdd(&hist[(key[e] >> shift) & (kRadixBins - 1)], 1u);
      __syncthreads();
      if (wave == 0) {
        // lane l holds bins 2l (lower) and 2l + 1 (higher); find the bin that
        // holds the wanted rank counting from the largest key
        const uint32_t rem = s_state[1];
        const uint32_t lo = hist[2 * lane], hi = hist[2 * lane + 1];
        const uint32_t suf = wave_suffix_sum(lo + hi, lane);   // bins >= 2l
        const uint32_t above = suf - lo - hi;                 // bins >= 2l + 2
        int bin = -1;
        uint32_t left = 0u;
        if (above < rem && rem <= above + hi) {
          bin = 2 * lane + 1;
          left = rem - above;
        } else if (above + hi < rem && rem <= suf) {
          bin = 2 * lane;
          left = rem - above - hi;
        }
        if (bin >= 0) {
          s_state[0] = prefix | ((uint32_t)bin << shift);
          s_state[1] = left;
        }
      }
      __syncthreads();
      pmask |= (uint32_t)(kRadixBins - 1) << shift;
    }
    thr = s_state[0];   // keys are unique: exactly kk keys are >= thr
  }

  // ---- keep key >= thr (and k > 0), written in index order
  uint32_t keep[4], cnt = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    keep[e] = (kk > 0 && key[e] != 0u && key[e] >= thr) ? 1u : 0u;
    cnt += keep[e];
  }
  const uint32_t incl = wave_prefix_sum(cnt, lane);
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  uint32_t base = 0u;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  uint32_t pos = base + incl - cnt;
  int32_t* out = sel + (size_t)c * (size_t)k;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (keep[e]) out[pos++] = c0 + j0 + e;
}

__global__ void __launch_bounds__(kRefineThreads) refine_kernel(
    const uint8_t* __restrict__ rcodes, const uint16_t* __restrict__ rscales,
    const uint16_t* __restrict__ rzeros, int N, int K, const int32_t* __restrict__ sel, int n_sel,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ y) {
  __shared__ float s_part[kRefineSlots][kRefineRows];
  const int tid = threadIdx.x;
  const int p = tid & 7, slot = tid >> 3;             // part of the row block, column slot
  const int q = p & 3;                                // quarter of the group
  const int Gn = N / kGroup;                          // groups along N
  const int g = blockIdx.x * (kRefineRows / kGroup) + (p >> 2);
  const bool gv = g < Gn;
  const uint32_t row_bytes = (uint32_t)N / 2u;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(rcodes, clamp_bytes((uint64_t)K * row_bytes));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(rscales, clamp_bytes((uint64_t)K * Gn * 2));
  const __amdgpu_buffer_rsrc_t zrs = make_rsrc(rzeros, clamp_bytes((uint64_t)K * Gn * 2));
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (uint32_t)K * 2u);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int kStep = kRefineSlots * kRefineUnroll;
  for (int j0 = slot; j0 < n_sel; j0 += kStep) {
    // kRefineUnroll columns of this slot, all loads issued before any use; a
    // column past n_sel or out of [0, K) reads zeros everywhere and adds 0
    uint32_t co[kRefineUnroll], mo[kRefineUnroll], xo[kRefineUnroll];
#pragma unroll
    for (int u = 0; u < kRefineUnroll; ++u) {
      const int j = j0 + u * kRefineSlots;
      const int ch = j < n_sel ? sel[j] : -1;
      const bool cv = ch >= 0 && ch < K;
      xo[u] = cv ? (uint32_t)ch * 2u : kOobR;
      co[u] = cv && gv ? (uint32_t)ch * row_bytes + (uint32_t)g * 16u + 4u * (uint32_t)q : kOobR;
      mo[u] = cv && gv ? ((uint32_t)ch * (uint32_t)Gn + (uint32_t)g) * 2u : kOobR;
    }
    uint32_t w[kRefineUnroll];
    uint16_t sv[kRefineUnroll], zv[kRefineUnroll], xv[kRefineUnroll];
#pragma unroll
    for (int u = 0; u < kRefineUnroll; ++u) {
      w[u] = ld32(crs, co[u]);
      sv[u] = ld16(srs, mo[u]);
      zv[u] = ld16(zrs, mo[u]);
      xv[u] = ld16(xrs, xo[u]);
    }
#pragma unroll
    for (int u = 0; u < kRefineUnroll; ++u) {
      const float z = h2f(zv[u]);
      const float xsv = h2f(xv[u]) * h2f(sv[u]);
      // byte b of the quarter: rows 4q + b (low nibble) and 4q + b + 16 (high nibble)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float lo = (float)((w[u] >> (8 * b)) & 0x0Fu) - z;
        const float hi = (float)((w[u] >> (8 * b + 4)) & 0x0Fu) - z;
        acc[b] = __builtin_fmaf(lo, xsv, acc[b]);
        acc[4 + b] = __builtin_fmaf(hi, xsv, acc[4 + b]);
      }
    }
  }
  const int rb = (p >> 2) * kGroup + 4 * q;           // first row of this thread in the block
#pragma unroll
  for (int i = 0; i < 8; ++i) s_part[slot][rb + (i & 3) + (i >= 4 ? 16 : 0)] = acc[i];
  __syncthreads();
  if (tid < kRefineRows) {
    const int row = blockIdx.x * kRefineRows + tid;
    if (row < N) {
      float t = s_part[0][tid];
#pragma unroll
      for (int s = 1; s < kRefineSlots; ++s) t += s_part[s][tid];   // fixed order
      y[row] = f2h(h2f(y[row]) + t);
    }
  }
}

}  // namespace wqd

using namespace wqd;

extern "C" int64_t wq_topk_count(int64_t K, int64_t chunk, int64_t k) {
  if (K < 0 || chunk < 1 || k < 0) return wq::fail(WQ_ERR_INVALID_ARG, "wq_topk_count: bad sizes");
  const int64_t full = K / chunk, rest = K % chunk;
  wq::ok();
  return full * std::min(k, chunk) + std::min(k, rest);
}

extern "C" int wq_topk_chunks(const uint16_t* x, int64_t K, int64_t chunk, int64_t k,
                              int32_t* sel, void* stream) {
  const char* who = "wq_topk_chunks";
  if (K < 32 || K % 32 || K > WQ_MAX_K)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: K must be a multiple of 32 in [32, %d]", who,
                    WQ_MAX_K);
  if (chunk < 64 || chunk > 1024 || chunk % 64)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: chunk must be a multiple of 64 in [64, 1024]", who);
  if (k < 0) return wq::fail(WQ_ERR_INVALID_ARG, "%s: k must be >= 0", who);
  if (k == 0) return wq::ok();
  if (!x || !sel) return wq::fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(x)) return wq::fail(WQ_ERR_INVALID_ARG, "%s: x must be 16-byte aligned", who);
  const int nch = (int)((K + chunk - 1) / chunk);
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)nch), dim3(kTopkThreads), 0, (hipStream_t)stream,
                     x, (int)K, (int)chunk, (int)std::min<int64_t>(k, chunk), sel);
  return check_launch(who);
}

extern "C" int wq_refine_add(const uint8_t* rcodes, const uint16_t* rscales,
                             const uint16_t* rzeros, int64_t N, int64_t K, const int32_t* sel,
                             int64_t n_sel, const uint16_t* x, uint16_t* y, void* stream) {
  const char* who = "wq_refine_add";
  if (int r = wq::check_shape(N, K, who)) return r;
  if (N % 32) return wq::fail(WQ_ERR_UNSUPPORTED, "%s: N must be a multiple of 32", who);
  if (n_sel < 0 || n_sel > K) return wq::fail(WQ_ERR_INVALID_ARG, "%s: n_sel must be in [0, K]", who);
  if (n_sel == 0) return wq::ok();
  if (!rcodes || !rscales || !rzeros || !sel || !x || !y)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if ((uint64_t)K * (uint64_t)N / 2 > 0xFFFFE000ull)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: refinement larger than 4 GB", who);
  const int blocks = (int)((N + kRefineRows - 1) / kRefineRows);
  hipLaunchKernelGGL(refine_kernel, dim3((unsigned)blocks), dim3(kRefineThreads), 0,
                     (hipStream_t)stream, rcodes, rscales, rzeros, (int)N, (int)K, sel, (int)n_sel,
                     x, y);
  return check_launch(who);
}
