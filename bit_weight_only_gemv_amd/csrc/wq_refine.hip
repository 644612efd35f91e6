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
// Selection (wave_chunk_topk, wq_select.cuh): one wave per chunk, lane l
// holding channels 16l .. 16l + 15; the k-th largest FP16 magnitude comes from
// two histogram passes in the wave's own LDS.  No block barrier is needed.
//
// Refinement add (refine_groups): a workgroup of 512 threads owns GPW groups of
// 32 output rows and splits the selected columns over 128 slots of 4 threads;
// thread (slot, quarter) decodes 4 code bytes, 8 rows, of each of its groups
// for columns j = slot, slot + 128, ... with four columns' loads in flight at
// a time.  The slots' partial sums are added in a fixed order and added once
// into the FP16 output.
//
// topk_kernel runs the selection alone (one wave per chunk), refine_kernel the
// add alone from a given selection, and topk_refine_kernel both in one launch:
// each workgroup selects for every chunk into LDS (8 waves, chunks w, w + 8,
// ...) and then adds for its own group.  The two paths sum in the same order,
// so their outputs agree bit for bit.

#include "wq_common.cuh"
#include "wq_device.h"
#include "wq_select.cuh"

namespace wqd {

constexpr uint32_t kOobR = 0xFFFFF000u;       // past every buffer: loads return 0
constexpr int kRefineThreads = 512;
constexpr int kRefineSlots = kRefineThreads / 4;       // column slots per workgroup
constexpr int kRefineUnroll = 4;              // columns per slot with loads in flight
constexpr int kRefineRuns = kRefineThreads / kGroup;   // 16 runs of 8 slots in the sum
constexpr int kFusedMaxSel = 4096;            // selections the fused kernel holds in LDS

// One chunk per workgroup of one wave.
__global__ void __launch_bounds__(kWave) topk_kernel(const uint16_t* __restrict__ x, int K,
                                                    int chunk, int k, int32_t* __restrict__ sel) {
  __shared__ uint32_t hist[kSelWords];
  const int c = blockIdx.x;
  const int c0 = c * chunk;
  const int csize = min(chunk, K - c0);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (uint32_t)K * 2u);
  wave_chunk_topk(xrs, c0, csize, min(k, csize), hist, sel + (size_t)c * (size_t)k,
                  (int)threadIdx.x);
}

// y[32 g .. 32 g + 31] += sum_{j < n_sel} x[sel[j]] C[rows][sel[j]] for the
// workgroup's GPW groups g = g0 .. g0 + GPW - 1 (those below Gn), 512 threads.
// Every group is summed in the same order whatever GPW is.  sel may sit in LDS
// or global memory; s_part holds GPW * 128 * 32 floats, s_red GPW * 16 * 32.
template <int GPW>
__device__ __forceinline__ void refine_groups(const __amdgpu_buffer_rsrc_t& crs,
                                              const __amdgpu_buffer_rsrc_t& srs,
                                              const __amdgpu_buffer_rsrc_t& zrs,
                                              const __amdgpu_buffer_rsrc_t& xrs, uint32_t row_bytes,
                                              int Gn, int K, int g0, const int32_t* sel, int n_sel,
                                              uint16_t y0, uint16_t* __restrict__ y, float* s_part,
                                              float* s_red) {
  const int tid = threadIdx.x;
  const int q = tid & 3, slot = tid >> 2;             // quarter of a group, column slot
  float acc[GPW][8];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[gi][i] = 0.f;
  constexpr int kStep = kRefineSlots * kRefineUnroll;
  for (int j0 = slot; j0 < n_sel; j0 += kStep) {
    // kRefineUnroll columns of this slot, all loads issued before any use; a
    // column past n_sel or out of [0, K), or a group past Gn, reads zeros
    // everywhere and adds 0
    int ch[kRefineUnroll];
#pragma unroll
    for (int u = 0; u < kRefineUnroll; ++u) {
      const int j = j0 + u * kRefineSlots;
      const int c = j < n_sel ? sel[j] : -1;
      ch[u] = c >= 0 && c < K ? c : -1;
    }
    uint32_t w[kRefineUnroll][GPW];
    uint16_t sv[kRefineUnroll][GPW], zv[kRefineUnroll][GPW], xv[kRefineUnroll];
#pragma unroll
    for (int u = 0; u < kRefineUnroll; ++u) {
      const bool cv = ch[u] >= 0;
      xv[u] = ld16(xrs, cv ? (uint32_t)ch[u] * 2u : kOobR);
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const int g = g0 + gi;
        const bool ok = cv && g < Gn;
        w[u][gi] = ld32(crs, ok ? (uint32_t)ch[u] * row_bytes + (uint32_t)g * 16u + 4u * (uint32_t)q
                                : kOobR);
        const uint32_t mo = ok ? ((uint32_t)ch[u] * (uint32_t)Gn + (uint32_t)g) * 2u : kOobR;
        sv[u][gi] = ld16(srs, mo);
        zv[u][gi] = ld16(zrs, mo);
      }
    }
#pragma unroll
    for (int u = 0; u < kRefineUnroll; ++u) {
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const float z = h2f(zv[u][gi]);
        const float xsv = h2f(xv[u]) * h2f(sv[u][gi]);
        // byte b of the quarter: rows 4q + b (low nibble) and 4q + b + 16 (high nibble)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float lo = (float)((w[u][gi] >> (8 * b)) & 0x0Fu) - z;
          const float hi = (float)((w[u][gi] >> (8 * b + 4)) & 0x0Fu) - z;
          acc[gi][b] = __builtin_fmaf(lo, xsv, acc[gi][b]);
          acc[gi][4 + b] = __builtin_fmaf(hi, xsv, acc[gi][4 + b]);
        }
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      s_part[(gi * kRefineSlots + slot) * kGroup + 4 * q + (i & 3) + (i >= 4 ? 16 : 0)] =
          acc[gi][i];
  __syncthreads();
  // fixed-order sums per group: 16 runs of 8 slots, then the 16 run sums
  {
    const int r = tid & (kGroup - 1), run = tid >> 5;
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const float* p = s_part + (gi * kRefineSlots + run * 8) * kGroup + r;
      float t = p[0];
#pragma unroll
      for (int s = 1; s < 8; ++s) t += p[s * kGroup];
      s_red[(gi * kRefineRuns + run) * kGroup + r] = t;
    }
  }
  __syncthreads();
  if (tid < GPW * kGroup && g0 + tid / kGroup < Gn) {
    const int gi = tid / kGroup, r = tid & (kGroup - 1);
    const float* p = s_red + gi * kRefineRuns * kGroup + r;
    float t = p[0];
#pragma unroll
    for (int s = 1; s < kRefineRuns; ++s) t += p[s * kGroup];
    y[g0 * kGroup + tid] = f2h(h2f(y0) + t);
  }
}

struct RefineArgs {
  const uint8_t* rcodes;
  const uint16_t* rscales;
  const uint16_t* rzeros;
  const uint16_t* x;
  uint16_t* y;
  const int32_t* sel;   // refine_kernel: the selection; topk_refine_kernel: unused
  int32_t* sel_out;     // topk_refine_kernel: optional copy of the selection
  int N, K, n_sel, chunk, k;
};

template <int GPW>
__global__ void __launch_bounds__(kRefineThreads) refine_kernel(RefineArgs a) {
  __shared__ float s_part[GPW * kRefineSlots * kGroup];
  __shared__ float s_red[GPW * kRefineRuns * kGroup];
  const int Gn = a.N / kGroup;
  const int g0 = blockIdx.x * GPW;
  const uint32_t row_bytes = (uint32_t)a.N / 2u;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(a.rcodes, clamp_bytes((uint64_t)a.K * row_bytes));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.rscales, clamp_bytes((uint64_t)a.K * Gn * 2));
  const __amdgpu_buffer_rsrc_t zrs = make_rsrc(a.rzeros, clamp_bytes((uint64_t)a.K * Gn * 2));
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x, (uint32_t)a.K * 2u);
  // the output rows are read up front, off the selection's critical path
  const int tid = threadIdx.x;
  const uint16_t y0 =
      tid < GPW * kGroup && g0 + tid / kGroup < Gn ? a.y[g0 * kGroup + tid] : (uint16_t)0;
  refine_groups<GPW>(crs, srs, zrs, xrs, row_bytes, Gn, a.K, g0, a.sel, a.n_sel, y0, a.y, s_part,
                     s_red);
}

template <int GPW>
__global__ void __launch_bounds__(kRefineThreads) topk_refine_kernel(RefineArgs a) {
  constexpr int kWaves = kRefineThreads / kWave;
  // the selection's histograms live in the partial-sum area until it is used
  constexpr int kPartFloats = GPW * kRefineSlots * kGroup;
  static_assert(kPartFloats >= kWaves * kSelWords, "histograms must fit the partial sums");
  __shared__ int32_t s_sel[kFusedMaxSel];
  __shared__ float s_part[kPartFloats];
  __shared__ float s_red[GPW * kRefineRuns * kGroup];
  uint32_t* s_hist = reinterpret_cast<uint32_t*>(s_part);
  const int Gn = a.N / kGroup;
  const int g0 = blockIdx.x * GPW;
  const uint32_t row_bytes = (uint32_t)a.N / 2u;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(a.rcodes, clamp_bytes((uint64_t)a.K * row_bytes));
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.rscales, clamp_bytes((uint64_t)a.K * Gn * 2));
  const __amdgpu_buffer_rsrc_t zrs = make_rsrc(a.rzeros, clamp_bytes((uint64_t)a.K * Gn * 2));
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x, (uint32_t)a.K * 2u);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const uint16_t y0 =
      tid < GPW * kGroup && g0 + tid / kGroup < Gn ? a.y[g0 * kGroup + tid] : (uint16_t)0;
  const int nch = (a.K + a.chunk - 1) / a.chunk;
  for (int c = wave; c < nch; c += kWaves) {
    const int c0 = c * a.chunk;
    const int csize = min(a.chunk, a.K - c0);
    wave_chunk_topk(xrs, c0, csize, min(a.k, csize), s_hist + wave * kSelWords, s_sel + c * a.k,
                    lane);
  }
  __syncthreads();
  if (a.sel_out != nullptr && blockIdx.x == 0)
    for (int j = tid; j < a.n_sel; j += kRefineThreads) a.sel_out[j] = s_sel[j];
  refine_groups<GPW>(crs, srs, zrs, xrs, row_bytes, Gn, a.K, g0, s_sel, a.n_sel, y0, a.y, s_part,
                     s_red);
}

// Groups per workgroup: enough workgroups to spread the loads, few enough that
// the fused kernel's per-workgroup selection is not repeated far beyond one
// workgroup per compute unit.
// An explicit variant may choose 1, 2 or 4 groups per workgroup instead.
static int refine_gpw(int Gn, bool fused, const wq_variant* v) {
  int gpw = 1;
  if (fused) {
    const int cus = device_cus() > 0 ? device_cus() : 256;
    while (gpw < 4 && (Gn + gpw - 1) / gpw > cus) gpw *= 2;
  }
  const int e = variant_or(v, &wq_variant::refine_groups, gpw);
  if (e == 1 || e == 2 || e == 4) gpw = e;
  return gpw;
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
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)nch), dim3(kWave), 0, (hipStream_t)stream, x,
                     (int)K, (int)chunk, (int)std::min<int64_t>(k, chunk), sel);
  return check_launch(who);
}

extern "C" int wq_refine_add_v(const uint8_t* rcodes, const uint16_t* rscales,
                               const uint16_t* rzeros, int64_t N, int64_t K, const int32_t* sel,
                               int64_t n_sel, const uint16_t* x, uint16_t* y,
                               const wq_variant* variant, void* stream) {
  const char* who = "wq_refine_add";
  if (int r = wq::check_shape(N, K, who)) return r;
  if (N % 32) return wq::fail(WQ_ERR_UNSUPPORTED, "%s: N must be a multiple of 32", who);
  if (n_sel < 0 || n_sel > K) return wq::fail(WQ_ERR_INVALID_ARG, "%s: n_sel must be in [0, K]", who);
  if (n_sel == 0) return wq::ok();
  if (!rcodes || !rscales || !rzeros || !sel || !x || !y)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if ((uint64_t)K * (uint64_t)N / 2 > 0xFFFFE000ull)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: refinement larger than 4 GB", who);
  RefineArgs a{};
  a.rcodes = rcodes;
  a.rscales = rscales;
  a.rzeros = rzeros;
  a.x = x;
  a.y = y;
  a.sel = sel;
  a.N = (int)N;
  a.K = (int)K;
  a.n_sel = (int)n_sel;
  const int Gn = (int)(N / kGroup), gpw = refine_gpw(Gn, false, variant);
  const dim3 grid((unsigned)((Gn + gpw - 1) / gpw)), block(kRefineThreads);
  if (gpw == 1)
    hipLaunchKernelGGL(refine_kernel<1>, grid, block, 0, (hipStream_t)stream, a);
  else if (gpw == 2)
    hipLaunchKernelGGL(refine_kernel<2>, grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(refine_kernel<4>, grid, block, 0, (hipStream_t)stream, a);
  return check_launch(who);
}

extern "C" int wq_refine_topk_v(const uint8_t* rcodes, const uint16_t* rscales,
                                const uint16_t* rzeros, int64_t N, int64_t K, int64_t chunk,
                                int64_t k, const uint16_t* x, uint16_t* y, int32_t* sel_out,
                                const wq_variant* variant, void* stream) {
  const char* who = "wq_refine_topk";
  if (int r = wq::check_shape(N, K, who)) return r;
  if (N % 32) return wq::fail(WQ_ERR_UNSUPPORTED, "%s: N must be a multiple of 32", who);
  if (chunk < 64 || chunk > 1024 || chunk % 64)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: chunk must be a multiple of 64 in [64, 1024]", who);
  if (k < 0) return wq::fail(WQ_ERR_INVALID_ARG, "%s: k must be >= 0", who);
  if (k == 0) return wq::ok();
  const int64_t kk = std::min(k, chunk);
  const int64_t n_sel = (K / chunk) * kk + std::min(kk, K % chunk);
  if (!rcodes || !rscales || !rzeros || !x || !y)
    return wq::fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(x)) return wq::fail(WQ_ERR_INVALID_ARG, "%s: x must be 16-byte aligned", who);
  if ((uint64_t)K * (uint64_t)N / 2 > 0xFFFFE000ull)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: refinement larger than 4 GB", who);
  // Past 8 chunks each of the one-launch kernel's 8 waves selects several
  // chunks in turn; with a buffer for the selection, the two-kernel path is
  // faster there (and holds any number of selections), and it sums in the
  // same order (identical y).
  const int64_t nch = (K + chunk - 1) / chunk;
  if (sel_out != nullptr && (nch > kRefineThreads / kWave || n_sel > kFusedMaxSel)) {
    if (int r = wq_topk_chunks(x, K, chunk, k, sel_out, stream)) return r;
    return wq_refine_add_v(rcodes, rscales, rzeros, N, K, sel_out, n_sel, x, y, variant, stream);
  }
  if (n_sel > kFusedMaxSel)
    return wq::fail(WQ_ERR_UNSUPPORTED, "%s: %lld selected channels exceed %d without sel_out "
                    "(pass sel_out, or call wq_topk_chunks + wq_refine_add)", who,
                    (long long)n_sel, kFusedMaxSel);
  RefineArgs a{};
  a.rcodes = rcodes;
  a.rscales = rscales;
  a.rzeros = rzeros;
  a.x = x;
  a.y = y;
  a.sel_out = sel_out;
  a.N = (int)N;
  a.K = (int)K;
  a.n_sel = (int)n_sel;
  a.chunk = (int)chunk;
  a.k = (int)kk;
  const int Gn = (int)(N / kGroup), gpw = refine_gpw(Gn, true, variant);
  const dim3 grid((unsigned)((Gn + gpw - 1) / gpw)), block(kRefineThreads);
  if (gpw == 1)
    hipLaunchKernelGGL(topk_refine_kernel<1>, grid, block, 0, (hipStream_t)stream, a);
  else if (gpw == 2)
    hipLaunchKernelGGL(topk_refine_kernel<2>, grid, block, 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(topk_refine_kernel<4>, grid, block, 0, (hipStream_t)stream, a);
  return check_launch(who);
}

extern "C" int wq_refine_add(const uint8_t* rcodes, const uint16_t* rscales,
                             const uint16_t* rzeros, int64_t N, int64_t K, const int32_t* sel,
                             int64_t n_sel, const uint16_t* x, uint16_t* y, void* stream) {
  return wq_refine_add_v(rcodes, rscales, rzeros, N, K, sel, n_sel, x, y, nullptr, stream);
}

extern "C" int wq_refine_topk(const uint8_t* rcodes, const uint16_t* rscales,
                              const uint16_t* rzeros, int64_t N, int64_t K, int64_t chunk,
                              int64_t k, const uint16_t* x, uint16_t* y, int32_t* sel_out,
                              void* stream) {
  return wq_refine_topk_v(rcodes, rscales, rzeros, N, K, chunk, k, x, y, sel_out, nullptr, stream);
}
