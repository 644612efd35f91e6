// M = 1 .. 4 dequantize-and-multiply on the matrix cores of gfx950
// (v_mfma_f32_16x16x32_f16), persistent over row blocks.
//
// What is computed is the same as the VALU kernels of wq_gemv.hip (SPECTRA
// page, section 4.1; OTF-LLM v4.0 page, section 5):
//   y[n] = FP16( sum_{k not in outliers} w_hat[n][k] x[k]
//                + sum_j out_w[n][j] x[out_idx[j]] ),   FP32 accumulation.
//
// Layout of the work:
//  * A workgroup owns row blocks of 16 rows (blockIdx.x, + gridDim.x, ...) and
//    has nw waves; wave w owns the K-slices of 512 channels w, w + nw, ...
//    Each wave keeps its slices' x in an LDS region of its own (masked at the
//    outlier columns, with per-group sums of x and the slice's outlier
//    activations).  The set-up (W2 centroid table, x, outlier gather) runs
//    while the first row blocks are in flight; its two workgroup barriers wait
//    for LDS traffic only, never for the weight stream.
//  * One MFMA multiplies a 16 x 32 A block by a 32 x 16 B block.  B holds
//    decoded weights: lane (n, r) = (lane % 16, lane / 16) gives 8 weights of
//    row n from its own 16-byte load (W4: one group; W2: two groups).  The
//    four lane quarters read different groups, so a plain product would mix
//    groups that carry different scales.  The 16 rows of A keep them apart:
//    A row m ("slot") holds x only in the k-quarter and step that belong to
//    group m of the slice, zero elsewhere, so D[m][n] = sum over group m of
//    x * code value.  After the 16 steps of a row block, lane (n, r) holds
//    D[4r + j][n], the sums of the 4 consecutive groups 4r .. 4r + 3, and
//    applies their scales and zeros:
//      W4: s (sum q x - z sum x), codes entering as FP16 subnormals q 2^-24;
//      W2: S sum C[q] x + Z sum x, centroids from an LDS table.
//  * W2 table: 256 entries (one code byte -> its four FP16 centroids), 32
//    copies, copy c at byte 8c of each 256-byte entry row, lane l reading copy
//    l % 32.  Every lane thus reads its own bank pair (no bank conflicts), and
//    the address (entry << 8 | 8 (l % 32)) is one byte permute of the code word.
//  * Outlier columns: the slab positions are cut into chunks of 8, and slice
//    ks owns chunks C(ks) .. C(ks + 1) - 1, C(ks) = floor(ks nch / nks), at
//    most 4 of them; lane quarter r takes chunk C(ks) + r.  The positions, not
//    the columns they name, are split, so every slab load address is known at
//    entry and the slab streams with the codes.  At set-up the lanes gather
//    the outlier activations of their share from the workgroup's copy of x and
//    zero those columns there; per row block the slab values are dotted with
//    them (v_dot2).
//  * Two layouts of the packed arrays: the row-major one of the C ABI, and the
//    tiled one (TILED), in which every load of a wave is one contiguous 1 KB
//    block: codes and scale/zero tiles per (row block, slice), slab chunks of
//    16 rows x 8 positions.
//  * Row-block loads go through a ring of DEPTH register buffers, so that
//    while one row block is multiplied, the next ones are in flight.
//  * Per row block each wave reduces its 4 lane quarters and adds its row
//    sums into an LDS slot of its own; the slots are summed in a fixed order
//    at the end (deterministic, no atomics).
//  * Several activation rows (MS = 2 or 4) share the 16 slots: each slice is
//    taken in MS windows of 16 / MS groups, and slot R stands for row R / WG,
//    group WG w + R % WG of window w (WG = 16 / MS).  Window w is multiplied
//    in the 16 / MS steps whose B fragments hold its groups, so a row block
//    still takes 16 MFMAs and one pass over the weights whatever MS is: the
//    slots a single row leaves empty in a step carry the other rows.  The
//    lane that holds a slot's sum is not the lane that loaded its scale and
//    zero; they come from the loading lane quarter by a cross-lane move.  W2
//    stops at MS = 2: its loads put two groups of different windows into the
//    same MFMA step.

#include "wq_common.cuh"
#include "wq_device.h"
#include "wq_mma.h"
#include "wq_select.cuh"


#include <algorithm>

namespace wqd {

constexpr int kSliceCh = 512;      // channels per K-slice
constexpr int kSliceGroups = 16;   // groups per K-slice = MFMA slots
constexpr int kLutRow = 256;       // bytes per W2 table entry (32 copies x 8 bytes)
constexpr int kMaxWaves = 8;
// Buffer offset past every range the kernels read (the plans keep each
// array below kMaxArrayBytes, and instruction offsets of up to 3 KB cannot
// wrap it): loads from it return 0.
constexpr uint32_t kOob = 0xFFFFF000u;
constexpr int64_t kMaxArrayBytes = 0xFFFFE000ll;

struct MmaArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* zeros;
  const int32_t* out_idx;
  const uint16_t* out_w;
  const uint16_t* x;   // [M][K]
  uint16_t* y;         // [M][N]
  int N, K, n_out;   // n_out = 0 when there are no outlier columns
  int M;             // activation rows (at most the kernel's MS)
  int nw;            // waves per workgroup
  int nks;           // K-slices
  int nsw;           // K-slices per wave, at most
  int nrb;           // row blocks (16 rows)
  int rbl;           // row blocks per workgroup, at most
  int nch;           // outlier chunks of 8 slab positions, ceil(n_out / 8)
  // Runtime top-k refinement (kernels with REF only): the refinement columns
  // in the W4 format along N ([K][N / 2] codes, [K][N / 32] scales and zeros),
  // the selection (optional copy, written by workgroup 0), chunk size, picks
  // per chunk (at most the chunk), chunks, helper waves, and the helpers'
  // shares: chunks per helper, 32-pick groups per chunk, row blocks per lane
  // half.
  const uint8_t* rcodes;
  const uint16_t* rscales;
  const uint16_t* rzeros;
  int32_t* sel_out;
  int rchunk, rk, rnch, nh;
  int rc, rp, rh;
};

// Refinement units (chunk, 32-pick group, row block) one helper lane holds, at
// most, and the workgroup size with the helper waves.
constexpr int kRefUnits = 4;
constexpr int kRefMaxThreads = 768;
// The W4 / W4P kernels without outliers fit 128 VGPRs, and so 16 waves.
constexpr int kRefWideThreads = 1024;

// Per-wave LDS region: for each of its slices and each activation row, x
// (1 KB, masked at the outlier columns), the 16 group sums of x (64 B) and the
// 32 outlier activations of the slice's share of the slab (64 B, zero past the
// share).
constexpr uint32_t kSliceLds = 1024u + 64u + 64u;
constexpr int kShareMax = 32;   // slab positions per slice, at most

// LDS layout (byte offsets), identical on host and device.
// With the refinement also: per helper wave the selection histograms, the
// picks of every chunk (rnch x rk channel indices and their FP16
// activations), and the refinement's row sums [row blocks][helpers][16].
struct MmaLds {
  uint32_t lut, wave, part, hist, sel, selx, rpart, total;
};
__host__ __device__ inline MmaLds mma_lds_layout(int fmt, int nw, int nsw, int rbl, int ms,
                                                 int rnch = 0, int rk = 0, int nh = 0) {
  MmaLds L{};
  uint32_t off = 0;
  L.lut = off;
  if (fmt == 2) off += 256u * kLutRow;
  L.wave = off;
  off += (uint32_t)nw * (uint32_t)nsw * (uint32_t)ms * kSliceLds;
  L.part = off;
  off += (uint32_t)rbl * (uint32_t)nw * (uint32_t)ms * 64u;
  L.hist = L.sel = L.selx = L.rpart = off;
  if (rnch > 0) {
    off += (uint32_t)nh * (uint32_t)kSelWords * 4u;
    L.sel = off;
    off += ((uint32_t)rnch * (uint32_t)rk * 4u + 15u) & ~15u;
    L.selx = off;
    off += ((uint32_t)rnch * (uint32_t)rk * 2u + 15u) & ~15u;
    L.rpart = off;
    off += (uint32_t)rbl * (uint32_t)nh * 64u;
  }
  L.total = off;
  return L;
}

template <int FMT>
struct MmaFmt;
template <>
struct MmaFmt<4> {
  static constexpr int kLoads = 4;       // 16-byte code loads per lane per row block
  static constexpr int kSliceBytes = 256;
  static constexpr int kRowBytesDiv = 2;
};
template <>
struct MmaFmt<5> : MmaFmt<4> {};   // W4P: W4 codes, packed zero points
template <>
struct MmaFmt<2> {
  static constexpr int kLoads = 2;
  static constexpr int kSliceBytes = 128;
  static constexpr int kRowBytesDiv = 4;
};

// 8-byte LDS load at a byte address of the kernel's LDS (the kernel declares
// no static LDS, so its dynamic LDS window starts at address 0).
__device__ __forceinline__ u2 lds_ld64(uint32_t addr) {
  return *(const __attribute__((address_space(3))) u2*)(size_t)addr;
}

// Loads of one row block of one K-slice: codes, scales, zeros, and the
// slice's share of the outlier slab (5 dwords per lane: the 8 FP16 values of
// the lane's positions, which may start at an odd index).
template <int FMT, bool OUT>
struct Item {
  u4v cw[MmaFmt<FMT>::kLoads];
  u2 sv, zv;
  uint32_t od[OUT ? 5 : 1];
};

// Dots 8 FP16 slab values (5 dwords starting at an even or odd FP16 index,
// sh = 0 or 16) with 4 pairs of FP16 activations; keep clears the values past
// the lane's share (they belong to other positions or rows, and an infinite
// one must not meet a zero activation).
__device__ __forceinline__ float slab_dot(const uint32_t (&od)[5], const uint32_t (&xw)[4],
                                          const uint32_t (&keep)[4], uint32_t sh, float v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wv = __builtin_amdgcn_alignbit(od[i + 1], od[i], sh) & keep[i];
    v = __builtin_amdgcn_fdot2(as_h2(wv), as_h2(xw[i]), v, false);
  }
  return v;
}

template <int FMT, bool OUT, bool TILED, int NSW, int MS, bool REF, bool WIDE = false>
__global__ void __launch_bounds__(WIDE ? kRefWideThreads : REF ? kRefMaxThreads : 512)
    mma1d_kernel(MmaArgs a) {
  typedef MmaFmt<FMT> F;
  constexpr int DEPTH = 2;
  static_assert(MS == 1 || MS == 2 || (MS == 4 && FMT != 2), "1, 2 or (W4) 4 activation rows");
  static_assert(!REF || MS == 1, "the refinement runs with one activation row");
  constexpr int WG = 16 / MS;   // groups per window: each slice is taken in MS windows
  extern __shared__ __align__(16) unsigned char smem[];
  const int n_out = OUT ? a.n_out : 0;
  const MmaLds L =
      mma_lds_layout(FMT, a.nw, a.nsw, a.rbl, MS, REF ? a.rnch : 0, REF ? a.rk : 0, REF ? a.nh : 0);
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n16 = lane & 15;
  const int r = lane >> 4;
  const int G = a.K >> 5;
  const uint32_t row_bytes = (uint32_t)a.K / F::kRowBytesDiv;
  const int nrb_wg = (a.nrb - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  // With the refinement, waves nw .. nw + nh - 1 are helpers: they take part
  // in the workgroup's set-up and barriers but own no slices (no items).
  const bool helper = REF && w >= a.nw;
  const int hw = w - a.nw;                           // helper index
  const int ns_w = helper ? 0 : (a.nks - w + a.nw - 1) / a.nw;   // 1 .. NSW (nw <= nks)
  const int T = ns_w * nrb_wg;                       // items of this wave
  const uint32_t wave_bytes = (uint32_t)a.nsw * MS * kSliceLds;
  const uint32_t wreg = L.wave + (uint32_t)w * wave_bytes;
  // slice s, activation row m: 1 KB of x, then the group sums and the outlier
  // activations
  auto slice_x = [&](int s, int m) { return wreg + (uint32_t)(s * MS + m) * kSliceLds; };
  auto slice_sx = [&](int s, int m) { return slice_x(s, m) + 1024u; };
  auto slice_xo = [&](int s, int m) { return slice_x(s, m) + 1088u; };
  // first outlier chunk of slice ks (ks nch < 2^31: the plan bounds both),
  // and the slice's share of slab positions, 8 C(ks) .. min(8 C(ks + 1), n_out)
  auto chunk_lo = [&](int ks) { return (uint32_t)(ks * a.nch) / (uint32_t)a.nks; };
  auto share_end = [&](int ks) { return min(8u * chunk_lo(ks + 1), (uint32_t)n_out); };

  // Row-major: codes [N][K/div], scales / zeros [N][G], slab [N][n_out].
  // Tiled: codes tiles of 16 kSliceBytes and scale/zero tiles of 1 KB per
  // (row block, slice), slab chunks of 256 bytes per (row block, chunk); the
  // arrays are padded to whole tiles, so the record counts cover them.
  const uint64_t tiles = (uint64_t)a.nrb * a.nks;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(
      a.codes, clamp_bytes(TILED ? tiles * 16 * F::kSliceBytes : (uint64_t)a.N * row_bytes));
  const uint64_t meta = TILED ? tiles * (FMT == 5 ? 640 : 1024) : (uint64_t)a.N * G * 2;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.scales, clamp_bytes(meta));
  const __amdgpu_buffer_rsrc_t zrs =
      make_rsrc(TILED ? a.scales : a.zeros,
                clamp_bytes(TILED ? meta : FMT == 5 ? (uint64_t)a.N * (G / 2) : meta));
  // The row-major slab is read with 4-byte loads at 4-byte-aligned offsets;
  // its record count is rounded up to that size, which stays inside the
  // 16-byte block (and page) of the last element.
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(
      a.out_w, clamp_bytes(TILED ? (uint64_t)a.nrb * a.nch * 256
                                 : ((uint64_t)a.N * n_out * 2 + 3) & ~(uint64_t)3));
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(a.out_idx, (uint32_t)n_out * 4u);
  const __amdgpu_buffer_rsrc_t xrs =
      make_rsrc(a.x, (MS == 1 ? 1u : (uint32_t)a.M) * (uint32_t)a.K * 2u);

  // ---- (0) x of every slice of this wave and the outlier indices of its
  //      slices' shares (lane l: slice 2p + l / 32, position l % 32 of the
  //      share), issued before the weight stream so that waiting for them
  //      never waits for weights
  u4v xr[MS][NSW];
  const __amdgpu_buffer_rsrc_t xnul = make_rsrc(a.x, 0u);
#pragma unroll
  for (int m = 0; m < MS; ++m)
#pragma unroll
    for (int s = 0; s < NSW; ++s) {   // lane l: channels 512 ks + 8 l .. + 8 (past K: 0)
      const uint32_t c = (uint32_t)((w + a.nw * s) * kSliceCh + 8 * lane);
      // with two rows, row 0's channels past K would read row 1: send them past
      // the buffer (the row-major codes there belong to the next weight row)
      const uint32_t off = MS == 1 ? c * 2u
                           : c < (uint32_t)a.K ? ((uint32_t)m * (uint32_t)a.K + c) * 2u : kOob;
      xr[m][s] = ld128(s < ns_w ? xrs : xnul, off);
    }
  constexpr int NIP = OUT ? (NSW + 1) / 2 : 1;
  uint32_t oi[NIP];
  bool oval[NIP];
  if constexpr (OUT) {
#pragma unroll
    for (int p = 0; p < NIP; ++p) {
      const int s = 2 * p + (lane >> 5);
      const int ks = w + a.nw * s;
      const uint32_t j = 8u * chunk_lo(ks) + (uint32_t)(lane & 31);
      oval[p] = s < ns_w && j < share_end(ks);
      oi[p] = ld32(irs, oval[p] ? j * 4u : kOob);
    }
  }
  asm volatile("" ::: "memory");   // these loads stay ahead of the weight stream

  // ---- (1) loads of one row block of one slice (every load is issued
  //      unconditionally; an item past the end reads nothing)
  // Offsets need no per-lane checks: rows past N and the bytes past the end
  // of a short last slice lie past the arrays (the loads return 0) or, in the
  // row-major layout, in the next row, where the activations are zero; an
  // item past the end of the wave's list reads through descriptors of zero
  // records.  A lane quarter past its slice's chunks reads at kOob (zero).
  const __amdgpu_buffer_rsrc_t nul = make_rsrc(a.codes, 0u);
  auto load_item = [&](Item<FMT, OUT>& it, bool valid, int ks, int rb) {
    const __amdgpu_buffer_rsrc_t c_ = valid ? crs : nul;
    const __amdgpu_buffer_rsrc_t s_ = valid ? srs : nul;
    const __amdgpu_buffer_rsrc_t z_ = valid ? zrs : nul;
    const uint32_t row = (uint32_t)(rb * 16 + n16);
    if constexpr (TILED) {
      const uint32_t tile = (uint32_t)(rb * a.nks + ks);
      const uint32_t cbase = tile * (16u * F::kSliceBytes) + 16u * (uint32_t)lane;
#pragma unroll
      for (int u = 0; u < F::kLoads; ++u) it.cw[u] = ld128(c_, cbase + 1024u * u);
      if constexpr (FMT == 5) {   // 640-byte tile: 4 scales per lane, then 4 packed zeros
        it.sv = ld64(s_, tile * 640u + 8u * (uint32_t)lane);
        it.zv = (u2){ld16(s_, tile * 640u + 512u + 2u * (uint32_t)lane), 0u};
      } else {
        const u4v m = ld128(s_, tile * 1024u + 16u * (uint32_t)lane);
        it.sv = (u2){m.x, m.y};
        it.zv = (u2){m.z, m.w};
      }
    } else {
      const uint32_t rbase = row * row_bytes + (uint32_t)(ks * F::kSliceBytes + 16 * r);
#pragma unroll
      for (int u = 0; u < F::kLoads; ++u) it.cw[u] = ld128(c_, rbase + 64u * u);
      const uint32_t mo = (row * (uint32_t)G + (uint32_t)(ks * kSliceGroups + 4 * r)) * 2u;
      it.sv = ld64(s_, mo);
      if constexpr (FMT == 5)   // groups 16 ks + 4 r .. + 3: two bytes of the packed row
        it.zv = (u2){ld16(z_, row * (uint32_t)(G / 2) + (uint32_t)(8 * ks + 2 * r)), 0u};
      else
        it.zv = ld64(z_, mo);
    }
    if constexpr (OUT) {
      const __amdgpu_buffer_rsrc_t o_ = valid ? ors : nul;
      const uint32_t c0 = chunk_lo(ks);
      const bool on = (uint32_t)r < chunk_lo(ks + 1) - c0;
      if constexpr (TILED) {
        const uint32_t off = ((uint32_t)rb * (uint32_t)a.nch + c0) * 256u + 16u * (uint32_t)lane;
        const u4v t = ld128(o_, on ? off : kOob);
        it.od[0] = t.x;
        it.od[1] = t.y;
        it.od[2] = t.z;
        it.od[3] = t.w;
      } else {
        const uint32_t e0 = row * (uint32_t)n_out + 8u * (c0 + (uint32_t)r);
        const uint32_t b0 = on ? (e0 * 2u) & ~3u : kOob;
#pragma unroll
        for (int i = 0; i < 5; ++i) it.od[i] = ld32(o_, b0 + 4u * i);
      }
    }
  };
  int ls = 0, lr = 0;   // slice / row-block counters of the next item to load
  auto advance = [&](int& s_, int& q_) {
    if (++q_ == nrb_wg) {
      q_ = 0;
      ++s_;
    }
  };
  // W2 centroid table: entry e (a code byte) -> its four FP16 centroids, 32
  // copies in a 256-byte row; 16-byte chunk ch holds copies 2 (ch % 16) and
  // 2 (ch % 16) + 1 of entry ch / 16, and consecutive lanes write consecutive
  // chunks.
  auto build_lut = [&]() {
    if constexpr (FMT == 2) {
      u4v* lut = reinterpret_cast<u4v*>(smem + L.lut);
      for (int ch = tid; ch < 256 * 16; ch += nthr) {
        const uint32_t e = (uint32_t)ch >> 4;
        const uint32_t lo = w2_centroid_pair((e & 3u) | (((e >> 2) & 3u) << 16));
        const uint32_t hi = w2_centroid_pair(((e >> 4) & 3u) | ((e >> 6) << 16));
        lut[ch] = (u4v){lo, hi, lo, hi};
      }
    }
  };

  // ---- (2) set-up: every wave stores x of its slices; after a barrier each
  //      lane gathers the activations of its outlier positions (from whichever
  //      wave holds the column) and zeroes the column there; after a second
  //      barrier each wave sums the groups of its masked slices (W4: scaled by
  //      2^-24 like the code values)
  auto setup = [&]() {
#pragma unroll
    for (int m = 0; m < MS; ++m)
#pragma unroll
      for (int s = 0; s < NSW; ++s)
        if (s < ns_w) reinterpret_cast<u4v*>(smem + slice_x(s, m))[lane] = xr[m][s];
    lds_barrier();   // x of every wave, and the W2 table, visible
    if constexpr (OUT) {
#pragma unroll
      for (int p = 0; p < NIP; ++p) {
        const int s = 2 * p + (lane >> 5);
        const uint32_t c = oi[p];
        const bool v = oval[p] && c < (uint32_t)a.K;
#pragma unroll
        for (int m = 0; m < MS; ++m) {
          uint16_t xv = 0;
          if (v) {   // column c: slice c / 512, held by wave (c / 512) % nw as its slice (c / 512) / nw
            const uint32_t kc = c >> 9;
            const uint32_t wc = kc % (uint32_t)a.nw, sc = kc / (uint32_t)a.nw;
            uint16_t* xp = reinterpret_cast<uint16_t*>(
                smem + L.wave + wc * wave_bytes + (sc * MS + (uint32_t)m) * kSliceLds +
                (c & 511u) * 2u);
            xv = *xp;
            *xp = 0;
          }
          if (s < ns_w) reinterpret_cast<uint16_t*>(smem + slice_xo(s, m))[lane & 31] = xv;
        }
      }
      lds_barrier();   // every outlier column of x zeroed
    }
    // lane l sums group l % 16 of the (row, slice) pair p0 + l / 16 (pair p:
    // row p / NSW, slice p % NSW), four pairs per pass; each group's sum is
    // the same chain of dot products in every variant.  (Measured on MI355X,
    // against one pair per pass on lanes 0..15: W4 4096 x 14336 at M = 1
    // 10.01 -> 9.61 us, at M = 4 14.17 -> 13.0 us; W2 8192 x 28672 with 1003
    // outliers 22.97 -> 22.5 us; the same bits.)
#pragma unroll
    for (int p0 = 0; p0 < MS * NSW; p0 += 4) {
      const int pp = p0 + (lane >> 4);
      const int m = pp / NSW, s = pp % NSW;
      if (m < MS && s < ns_w) {
        const int gl = lane & (kSliceGroups - 1);
        float sum = 0.f;
        const u4v* src = reinterpret_cast<const u4v*>(smem + slice_x(s, m) + (uint32_t)gl * 64u);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u4v t = src[v];
          const uint32_t tw[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sum = __builtin_amdgcn_fdot2(as_h2(tw[i]), as_h2(0x3C003C00u), sum, false);
        }
        reinterpret_cast<float*>(smem + slice_sx(s, m))[gl] =
            FMT != 2 ? sum * 5.9604644775390625e-8f : sum;
      }
    }
  };

  // ---- (3) the prologue: the first row block's loads go out, the table is
  //      written and the set-up runs while they are in flight, and only then
  //      is the rest of the ring issued (measured on MI355X: issuing the
  //      whole ring at entry delays the first row block behind the others
  //      and costs more than the overlap gains)
  // A helper's chunks of x (refinement only): chunk hw + nh cw, lane l holds
  // channels 16 l .. 16 l + 15.  The first is requested here, beside the
  // first row block, so that it does not queue behind the ring.
  u4v xc0, xc1;
  auto chunk_x = [&](int cw, u4v& t0, u4v& t1) {
    const int cc = hw + a.nh * cw;
    const int c0 = cc * a.rchunk;
    const bool on = cw < a.rc && cc < a.rnch && 16 * lane < min(a.rchunk, a.K - c0);
    const uint32_t off = on ? (uint32_t)(c0 + 16 * lane) * 2u : kOob;
    t0 = ld128(xrs, off);
    t1 = ld128(xrs, off + 16u);
  };
  if constexpr (REF) {
    if (helper && hw < min(a.nh, a.rnch)) chunk_x(0, xc0, xc1);
  }
  Item<FMT, OUT> buf[DEPTH];
  load_item(buf[0], 0 < T, w + a.nw * ls, blockIdx.x + lr * gridDim.x);
  advance(ls, lr);
  build_lut();
  setup();
#pragma unroll
  for (int d = 1; d < DEPTH; ++d) {
    load_item(buf[d], d < T, w + a.nw * ls, blockIdx.x + lr * gridDim.x);
    advance(ls, lr);
  }

  // ---- (3b) refinement (StrataFlux page, section 3.2.1 and Eq. 2), on the
  //      helper waves while the others stream the weights: helper hw selects
  //      the k largest |x| of its chunks (hw, hw + nh, ...) into LDS, then
  //      loads, for each of its units, the 16 code bytes of one picked column
  //      over the 32-row group of one of the workgroup's row blocks, with the
  //      group's scale and zero.  Lane l takes pick 32 p + l % 32 of the unit's
  //      chunk and row block (l / 32) rh + h.
  const int nselh = REF ? min(a.nh, a.rnch) : 0;   // helpers with one chunk or more
  const int nunits = REF ? a.rc * a.rp * a.rh : 0;
  u4v rcw[REF ? kRefUnits : 1];
  uint16_t rsv[REF ? kRefUnits : 1], rzv[REF ? kRefUnits : 1];   // FP16 scale, zero
  uint32_t rxv[REF ? kRefUnits : 1];   // the pick's FP16 activation; 0 when the unit is empty
  // The products of the units: per unit, pick x (q - z) s for the 16 rows of
  // its row block (the row block's half of the group: low nibbles for an even
  // one, high for an odd one), summed over the 32 picks of the lane half by a
  // butterfly that leaves row ((l % 32) >> 1) on lane l; units of the same row
  // block are added in unit order, and lane pairs store their row's sum.
  float* s_rpart = reinterpret_cast<float*>(smem + L.rpart);
  auto refine_units = [&]() {
    if constexpr (REF) {
      float red[kRefUnits];
#pragma unroll
      for (int hh = 0; hh < kRefUnits; ++hh) red[hh] = 0.f;
#pragma unroll
      for (int u = 0; u < kRefUnits; ++u) {
        if (u < nunits) {
          const int h = u % a.rh;
          const int ri = (lane >> 5) * a.rh + h;
          // an empty unit holds zeros everywhere and adds 0
          const float xs = h2f((uint16_t)rxv[u]) * h2f(rsv[u]);
          const float z = h2f(rzv[u]);
          const uint32_t sh = 4u * ((blockIdx.x + (uint32_t)ri * gridDim.x) & 1u);
          const uint32_t dw[4] = {rcw[u].x, rcw[u].y, rcw[u].z, rcw[u].w};
          float v[16];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float q = (float)((dw[i] >> (8 * j + sh)) & 0x0Fu);
              v[4 * i + j] = (q - z) * xs;
            }
          // reduce-scatter over the 32 lanes of the half: rows by lane bits 4..1
#pragma unroll
          for (int st = 8; st >= 1; st >>= 1) {
            const bool upper = (lane & (2 * st)) != 0;
#pragma unroll
            for (int j = 0; j < st; ++j) {
              const float send = upper ? v[j] : v[j + st];
              const float keep = upper ? v[j + st] : v[j];
              v[j] = keep + __shfl_xor(send, 2 * st);
            }
          }
          v[0] += __shfl_xor(v[0], 1);
#pragma unroll
          for (int hh = 0; hh < kRefUnits; ++hh) red[hh] += hh == h ? v[0] : 0.f;
        }
      }
      if ((lane & 1) == 0) {
#pragma unroll
        for (int hh = 0; hh < kRefUnits; ++hh) {
          const int ri = (lane >> 5) * a.rh + hh;
          if (hh < a.rh && ri < nrb_wg)
            s_rpart[((uint32_t)ri * (uint32_t)a.nh + (uint32_t)hw) * 16u +
                    (uint32_t)((lane & 31) >> 1)] = red[hh];
        }
      }
    }
  };
  if (REF && helper && hw < nselh) {
    // the helper's work is short and latency-bound: it issues ahead of the
    // waves that stream the weights
    __builtin_amdgcn_s_setprio(3);
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + L.hist) + hw * kSelWords;
    int32_t* s_sel = reinterpret_cast<int32_t*>(smem + L.sel);
    uint16_t* s_selx = reinterpret_cast<uint16_t*>(smem + L.selx);
    // chunks hw, hw + nh, ...: the first was requested at entry, and the next
    // chunk's activations are in flight while this one is selected
#pragma unroll
    for (int cw = 0; cw < kRefUnits; ++cw) {
      const int cc = hw + a.nh * cw;
      if (cw < a.rc && cc < a.rnch) {
        const int c0 = cc * a.rchunk;
        const int csize = min(a.rchunk, a.K - c0);
        const int kk = min(a.rk, csize);
        const uint32_t xsel[8] = {xc0.x, xc0.y, xc0.z, xc0.w, xc1.x, xc1.y, xc1.z, xc1.w};
        if (cw + 1 < kRefUnits) chunk_x(cw + 1, xc0, xc1);
        wave_topk_regs<true>(xsel, c0, csize, kk, hist, s_sel + cc * a.rk, s_selx + cc * a.rk,
                             lane);
        if (a.sel_out != nullptr && blockIdx.x == 0) {
          wave_lds_sync();
          for (int j = lane; j < kk; j += kWave) a.sel_out[cc * a.rk + j] = s_sel[cc * a.rk + j];
        }
      }
    }
    wave_lds_sync();
    const __amdgpu_buffer_rsrc_t rcrs =
        make_rsrc(a.rcodes, clamp_bytes((uint64_t)a.K * (uint64_t)(a.N / 2)));
    const uint64_t rmeta = (uint64_t)a.K * (uint64_t)(a.N / 32) * 2u;
    const __amdgpu_buffer_rsrc_t rsrs = make_rsrc(a.rscales, clamp_bytes(rmeta));
    const __amdgpu_buffer_rsrc_t rzrs = make_rsrc(a.rzeros, clamp_bytes(rmeta));
#pragma unroll
    for (int u = 0; u < kRefUnits; ++u) {
      const int h = u % a.rh, pg = (u / a.rh) % a.rp, cw = u / (a.rh * a.rp);
      const int cc = hw + a.nh * cw;
      const int ri = (lane >> 5) * a.rh + h;
      const int pos = 32 * pg + (lane & 31);
      const int kk = cc < a.rnch ? min(a.rk, a.K - cc * a.rchunk) : 0;
      const bool on = u < nunits && cc < a.rnch && pos < kk && ri < nrb_wg;
      const uint32_t ch = on ? (uint32_t)s_sel[cc * a.rk + pos] : 0u;
      const uint32_t grp = (blockIdx.x + (uint32_t)ri * gridDim.x) >> 1;   // 32-row group
      rcw[u] = ld128(rcrs, on ? ch * (uint32_t)(a.N / 2) + grp * 16u : kOob);
      const uint32_t mo = on ? (ch * (uint32_t)(a.N / 32) + grp) * 2u : kOob;
      rsv[u] = ld16(rsrs, mo);
      rzv[u] = ld16(rzrs, mo);
      rxv[u] = on ? (uint32_t)s_selx[cc * a.rk + pos] : 0u;
    }
    refine_units();
    __builtin_amdgcn_s_setprio(0);
  }

  // ---- A fragments, group sums and outlier activations of slice s.  The 16
  //      A rows are group slots: with one activation row, slot g carries group
  //      g; with MS rows the slice is taken in MS windows of WG = 16 / MS
  //      groups, and slot WG m + g' carries group WG w + g' of row m in window w.
  h8 afr[16];
  f4 sxw[MS];
  uint32_t xo0[MS][4];
  uint32_t keep[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    sxw[m] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) xo0[m][i] = 0u;
  }
  auto enter_slice = [&](int s) {
    const int ks = w + a.nw * s;
    if constexpr (OUT) {
      // valid positions of the lane's chunk (row-major slab: the values past
      // them are other positions or rows, and are masked off)
      const int cnt = (int)share_end(ks) - (int)(8u * (chunk_lo(ks) + (uint32_t)r));
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        const u4v v = *reinterpret_cast<const u4v*>(smem + slice_xo(s, m) + (uint32_t)r * 16u);
        xo0[m][0] = v.x;
        xo0[m][1] = v.y;
        xo0[m][2] = v.z;
        xo0[m][3] = v.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        keep[i] = 2 * i + 1 < cnt ? 0xFFFFFFFFu : 2 * i < cnt ? 0x0000FFFFu : 0u;
    }
    // group sums of this lane's output slots in each window: C rows 4r .. 4r + 3
    // are the groups WG w + 4 (r % (WG / 4)) + j of row r / (WG / 4)
#pragma unroll
    for (int wdw = 0; wdw < MS; ++wdw) {
      const int mc = r / (WG / 4);
      const int gb = WG * wdw + 4 * (r % (WG / 4));
      sxw[wdw] = *reinterpret_cast<const f4*>(smem + slice_sx(s, mc) + (uint32_t)gb * 4u);
    }
    // A: the lane of a slot whose k-quarter holds the slot's group carries that
    // group's 32 activations in the 4 steps of the group; all else is 0
#pragma unroll
    for (int wdw = 0; wdw < MS; ++wdw) {
      const int R = n16;
      const int mi = R / WG;
      const int g = WG * wdw + R % WG;
      bool act;
      int u_m, t0;
      if constexpr (FMT == 2) {   // group g: load g / 8, quarter (g / 2) % 4, half g % 2
        act = r == ((g >> 1) & 3);
        u_m = g >> 3;
        t0 = 4 * (g & 1);
      } else {                    // group g: load g / 4, quarter g % 4
        act = r == (g & 3);
        u_m = g >> 2;
        t0 = 0;
      }
      uint32_t gv[16];
      {
        const u4v* src = reinterpret_cast<const u4v*>(smem + slice_x(s, mi) + (uint32_t)g * 64u);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u4v t = src[v];
          gv[4 * v + 0] = act ? t.x : 0u;
          gv[4 * v + 1] = act ? t.y : 0u;
          gv[4 * v + 2] = act ? t.z : 0u;
          gv[4 * v + 3] = act ? t.w : 0u;
        }
      }
      uint32_t fr[4][4];   // the group's 4 fragments (W4: in decode order)
      if constexpr (FMT == 2) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) fr[t][i] = gv[4 * t + i];
      } else {
        // step t, word i: codes k0 = 16 (t & 1) + 4 i + (t >> 1) and k0 + 2
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k0 = 16 * (t & 1) + 4 * i;
            fr[t][i] = __builtin_amdgcn_perm(gv[k0 / 2 + 1], gv[k0 / 2],
                                             (t >> 1) ? 0x07060302u : 0x05040100u);
          }
      }
      // the window's fragments: 16 / MS of the 16 steps
#pragma unroll
      for (int f = wdw * (16 / MS); f < (wdw + 1) * (16 / MS); ++f) {
        const int u = FMT == 2 ? (f >> 3) : (f >> 2);
        const int t = FMT == 2 ? (f & 7) : (f & 3);
        const int tt = FMT == 2 ? (t & 3) : t;
        const bool on = u == u_m && (FMT == 2 ? (t & 4) == t0 : true);
        const u4v v = on ? (u4v){fr[tt][0], fr[tt][1], fr[tt][2], fr[tt][3]}
                         : (u4v){0u, 0u, 0u, 0u};
        afr[f] = __builtin_bit_cast(h8, v);
      }
    }
  };

  // ---- one row block of one slice: products, slot scales, the slice's share
  //      of the outlier slab, reduction of the lane quarters
  float* s_part = reinterpret_cast<float*>(smem + L.part);
  const uint32_t lut_lane = (uint32_t)(lane & 31) * 8u;
  auto compute = [&](const Item<FMT, OUT>& it, int ri, int si) {
    const int row = (int)(blockIdx.x + (unsigned)ri * gridDim.x) * 16 + n16;
    float v = 0.f;   // this lane's slots: row r / (WG / 4)
#pragma unroll
    for (int wdw = 0; wdw < MS; ++wdw) {
      f4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FMT != 2) {
        // c0: low-nibble steps (values q 2^-24), c1: high-nibble steps (16 q 2^-24)
#pragma unroll
        for (int u = wdw * (4 / MS); u < (wdw + 1) * (4 / MS); ++u) {
          const uint32_t d[4] = {it.cw[u].x, it.cw[u].y, it.cw[u].z, it.cw[u].w};
          uint32_t d8[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) d8[i] = d[i] >> 8;
          const u4v b0 = {d[0] & 0x000F000Fu, d[1] & 0x000F000Fu, d[2] & 0x000F000Fu,
                          d[3] & 0x000F000Fu};
          const u4v b1 = {d[0] & 0x00F000F0u, d[1] & 0x00F000F0u, d[2] & 0x00F000F0u,
                          d[3] & 0x00F000F0u};
          const u4v b2 = {d8[0] & 0x000F000Fu, d8[1] & 0x000F000Fu, d8[2] & 0x000F000Fu,
                          d8[3] & 0x000F000Fu};
          const u4v b3 = {d8[0] & 0x00F000F0u, d8[1] & 0x00F000F0u, d8[2] & 0x00F000F0u,
                          d8[3] & 0x00F000F0u};
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[4 * u + 0], __builtin_bit_cast(h8, b0),
                                                      c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[4 * u + 1], __builtin_bit_cast(h8, b1),
                                                      c1, 0, 0, 0);
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[4 * u + 2], __builtin_bit_cast(h8, b2),
                                                      c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[4 * u + 3], __builtin_bit_cast(h8, b3),
                                                      c1, 0, 0, 0);
        }
      } else {
        // byte b of a code word -> LDS address (b << 8) | 8 (lane % 32); the 16
        // table reads of a load are issued before its 8 products
#pragma unroll
        for (int u = wdw * (2 / MS); u < (wdw + 1) * (2 / MS); ++u) {
          const uint32_t d[4] = {it.cw[u].x, it.cw[u].y, it.cw[u].z, it.cw[u].w};
          u2 lv[16];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const uint32_t word = d[t >> 1];
            const uint32_t bsel = (uint32_t)(2 * (t & 1));
            lv[2 * t] =
                lds_ld64(L.lut + __builtin_amdgcn_perm(word, lut_lane, 0x0C0C0400u + (bsel << 8)));
            lv[2 * t + 1] =
                lds_ld64(L.lut + __builtin_amdgcn_perm(word, lut_lane, 0x0C0C0500u + (bsel << 8)));
          }
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const u4v bv = {lv[2 * t].x, lv[2 * t].y, lv[2 * t + 1].x, lv[2 * t + 1].y};
            if (t & 1)
              c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[8 * u + t],
                                                          __builtin_bit_cast(h8, bv), c1, 0, 0, 0);
            else
              c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr[8 * u + t],
                                                          __builtin_bit_cast(h8, bv), c0, 0, 0, 0);
          }
        }
      }
      // slots 4r + j: groups ks*16 + WG w + 4 (r % (WG / 4)) + j, whose scales and
      // zeros the lane quarter w (WG / 4) + r % (WG / 4) of the same weight row
      // loaded (one row: this lane; two: this one or the one 32 lanes away)
      uint32_t sw[2] = {it.sv.x, it.sv.y};
      uint32_t zw[2] = {it.zv.x, it.zv.y};
      if constexpr (MS == 2) {
        const bool own = (r >> 1) == wdw;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t os = (uint32_t)__shfl_xor((int)sw[i], 32);
          const uint32_t oz = (uint32_t)__shfl_xor((int)zw[i], 32);
          sw[i] = own ? sw[i] : os;
          zw[i] = own ? zw[i] : oz;
        }
      } else if constexpr (MS == 4) {
        const int src = n16 + 16 * wdw;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          sw[i] = (uint32_t)__shfl((int)sw[i], src);
          zw[i] = (uint32_t)__shfl((int)zw[i], src);
        }
      }
      const f4 sx4 = sxw[wdw];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float s = h2f((uint16_t)(sw[j >> 1] >> (16 * (j & 1))));
        const float z = FMT == 5 ? (float)((zw[0] >> (4 * j)) & 0x0Fu)
                                 : h2f((uint16_t)(zw[j >> 1] >> (16 * (j & 1))));
        if constexpr (FMT != 2) {
          float t = __builtin_fmaf(c1[j], 0.0625f, c0[j]);
          t = __builtin_fmaf(-z, sx4[j], t);
          v = __builtin_fmaf(s, t, v);
        } else {
          v = __builtin_fmaf(s, c0[j] + c1[j], v);
          v = __builtin_fmaf(z, sx4[j], v);
        }
      }
    }
    if constexpr (FMT != 2) v *= 16777216.0f;
    float vv[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      vv[m] = (MS == 1 || m == r / (WG / 4)) ? v : 0.f;
      if constexpr (OUT) {
        if constexpr (TILED) {   // zero-padded chunks: no alignment, no mask
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vv[m] = __builtin_amdgcn_fdot2(as_h2(it.od[i]), as_h2(xo0[m][i]), vv[m], false);
        } else {
          const uint32_t sh = (((uint32_t)row * (uint32_t)n_out) & 1u) * 16u;
          vv[m] = slab_dot(it.od, xo0[m], keep, sh, vv[m]);
        }
      }
      // the four lane quarters hold parts of the same row's sum: add them
      vv[m] += __shfl_xor(vv[m], 16);
      vv[m] += __shfl_xor(vv[m], 32);
    }
    if (r == 0) {
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        float* p = s_part + (((uint32_t)ri * (uint32_t)a.nw + (uint32_t)w) * MS + (uint32_t)m) * 16u +
                   (uint32_t)n16;
        *p = si == 0 ? vv[m] : *p + vv[m];
      }
    }
  };

  // ---- (4) the items: compute one, refill its buffer with the one DEPTH
  //      ahead.  Only the ring's loads are in this loop.
  int si = 0, ri = 0;   // slice / row-block counters of the item being computed
  for (int base = 0; base < T; base += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (base + d < T) {
        if (ri == 0) enter_slice(si);
        compute(buf[d], ri, si);
        advance(si, ri);
      }
      load_item(buf[d], base + d + DEPTH < T, w + a.nw * ls, blockIdx.x + lr * gridDim.x);
      advance(ls, lr);
    }
  }

  // ---- (5) fixed-order sum of the waves' row sums
  __syncthreads();
  if constexpr (MS == 1) {
    for (int t = tid; t < nrb_wg * 16; t += nthr) {
      const int ri2 = t >> 4, n = t & 15;
      const int row = (int)(blockIdx.x + (unsigned)ri2 * gridDim.x) * 16 + n;
      if (row >= a.N) continue;
      float s = 0.f;
      for (int k = 0; k < a.nw; ++k) s += s_part[((uint32_t)ri2 * a.nw + k) * 16u + n];
      if constexpr (REF)
        for (int k = 0; k < nselh; ++k) s += s_rpart[((uint32_t)ri2 * a.nh + k) * 16u + n];
      a.y[row] = f2h(s);
    }
  } else {
    for (int t = tid; t < nrb_wg * 16 * MS; t += nthr) {
      const int n = t & 15, m = (t >> 4) % MS, ri2 = (t >> 4) / MS;
      const int row = (int)(blockIdx.x + (unsigned)ri2 * gridDim.x) * 16 + n;
      if (row >= a.N || m >= a.M) continue;
      float s = 0.f;
      for (int k = 0; k < a.nw; ++k)
        s += s_part[(((uint32_t)ri2 * a.nw + k) * MS + (uint32_t)m) * 16u + (uint32_t)n];
      a.y[(size_t)m * a.N + row] = f2h(s);
    }
  }
}

// ====================================================== batched (2 <= M <= 16)
//
// Same persistent layout (waves own K-slices, here of 256 or 512 channels;
// the workgroup's row blocks stream through a ring), but A holds the M activation
// rows (rows M..15 zero) and B holds the dequantized weights themselves, so
// each MFMA adds 16 rows x M activation rows x 32 channels into one tile:
//   W4: w_hat = (q - z) s exactly: (1024 + q) - (1024 + z) in FP16 is the
//       exact integer q - z, and its product with the FP16 scale rounds once,
//       to the dequantized weight itself;
//   W2: w_hat = S C[q] + Z as one FP16 fused multiply-add of the table's
//       centroids (one rounding).
// Lane (n, q) reads the QG consecutive groups QG q .. QG q + QG - 1 of row n's
// slice (W4: 16 QG bytes, W2: 8 QG bytes), whose scales and zeros are one
// 2 QG-byte load each.  The activation rows of the
// next slice are loaded one slice ahead.  W2 zeroes the outlier columns in the
// activation fragments (W4 needs no mask: a column zeroed before
// quantization decodes to exactly 0); the slice's run of the outlier slab is
// one more MFMA per row block, against the gathered outlier activations.

// Slice geometry: QG groups of 32 channels per lane quarter, so a slice is
// 128 QG channels (QG = 2: 256, QG = 4: 512).  W4 (and W4P) lanes read one
// 16-byte load per group, W2 lanes one per two groups.
template <int FMT, int QG>
struct MmbFmt {
  static constexpr int kSliceCh = 128 * QG;
  static constexpr int kSliceGroups = 4 * QG;
  static constexpr int kLoads = FMT == 2 ? QG / 2 : QG;
  static constexpr int kSliceBytes = FMT == 2 ? 32 * QG : 64 * QG;
  static constexpr int kRowBytesDiv = FMT == 2 ? 4 : 2;
  static constexpr int kSteps = 4 * QG;   // MFMA steps (and x loads) per lane per slice
};

struct MmbArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* zeros;
  const int32_t* out_idx;
  const uint16_t* out_w;
  const uint16_t* X;
  uint16_t* Y;
  int N, K, M, n_out;
  int nw, nks, nrb, rbl;
  int nch;   // tiled layout: outlier chunks of 8 slab positions, ceil(n_out / 8)
};

// LDS: W2 table; with outliers per wave two slice areas (outlier-column mask,
// one bit per channel of the slice, and, on the row-major layout, the run's
// column offsets, up to one per channel); partial tiles [rbl][nw][Mp][16]
// with Mp = M rounded up to the lane quarter's 4 rows (rows M..Mp-1 stay
// unread).
__host__ __device__ constexpr uint32_t mmb_wave_area(int qg, bool tiled) {
  return tiled ? 16u * qg : 16u * qg + 512u * qg;
}
struct MmbLds {
  uint32_t lut, wave, runs, idx, part, xt, total;
};
// Transpose area of the activation rows (XT kernels): per wave Mp rows of one
// slice, each padded by 16 bytes against bank conflicts.  xh (the tiled layout
// at M > 8): an area of 8 rows that the rows pass through in two rounds, where
// 16 rows would not fit (beside the W2 centroid table, or the LDS partial
// tiles of several row blocks).
__host__ __device__ constexpr uint32_t mmb_xt_stride(int qg) { return 256u * qg + 16u; }
__host__ __device__ constexpr uint32_t mmb_xt_rows(int M, bool xh) {
  return xh ? 8u : (uint32_t)((M + 3) & ~3);
}
// With outliers also: the run table (slice ks's run of the sorted indices
// starts at runs[ks], nks + 1 words) and a copy of the indices (256 iv words).
// preg: the partial tiles are kept in registers while the weights stream and
// written at the end into the staged-rows area (free by then), so the layout
// has no separate region for them.
__host__ __device__ inline MmbLds mmb_lds_layout(int fmt, int M, int nw, int rbl, int qg, int nks,
                                                 int iv, bool xt = false, bool tiled = false,
                                                 bool preg = false, bool xh = false) {
  MmbLds L{};
  uint32_t off = 0;
  L.lut = off;
  if (fmt == 2) off += 256u * kLutRow;
  L.wave = off;
  if (iv > 0) off += (uint32_t)nw * 2u * mmb_wave_area(qg, tiled);
  L.runs = off;
  if (iv > 0) off += ((uint32_t)(nks + 1) * 4u + 15u) & ~15u;
  L.idx = off;
  off += (uint32_t)iv * 1024u;
  L.part = off;
  if (!preg) off += (uint32_t)rbl * (uint32_t)nw * (uint32_t)((M + 3) & ~3) * 64u;
  L.xt = off;
  if (xt) {
    uint32_t area = (uint32_t)nw * mmb_xt_rows(M, xh) * mmb_xt_stride(qg);
    if (preg) {   // the partial tiles land here at the end
      const uint32_t tiles = (uint32_t)rbl * (uint32_t)nw * (uint32_t)((M + 3) & ~3) * 64u;
      area = area > tiles ? area : tiles;
    }
    off += area;
  }
  if (preg) L.part = L.xt;
  L.total = off;
  return L;
}

template <int FMT, bool OUT, int QG>
struct ItemB {
  u4v cw[MmbFmt<FMT, QG>::kLoads];
  u2 sv, zv;   // QG FP16 scales / zeros (W4P: QG packed nibbles in zv.x)
  uint32_t od[OUT ? 5 : 1];
};

__device__ __forceinline__ uint32_t splat_lo(uint32_t v) { return __builtin_amdgcn_perm(v, v, 0x01000100u); }
__device__ __forceinline__ uint32_t splat_hi(uint32_t v) { return __builtin_amdgcn_perm(v, v, 0x03020302u); }

// TILED: the layer in the tiled layout of the M = 1 kernel (512-channel slices,
// QG = 4).  Lane (n, q) reads its groups 4q .. 4q + 3 of a tile as 256-byte
// runs: each load of a wave is 4 contiguous runs instead of 64 row segments.
// The scale/zero tile gives lane (n, q) exactly those groups' scales and zeros.
// The outlier slab is split by position, as in the M = 1 kernel: slice ks owns
// chunks C(ks) .. C(ks + 1) - 1 of 8 positions (at most 4), lane quarter q
// takes chunk C(ks) + q, and its activations are gathered per slice through
// the index copy in LDS; the chunks are zero-padded, so no alignment or mask.
// PREG: each wave's partial tiles in registers (at most kPregMax row blocks
// per workgroup), added in the same order as the LDS tiles would be, so the
// results are the same bits; they reach LDS once, at the end.
// R8 (with XT): at most 8 activation rows, so staged rows 8..15 are neither
// loaded nor held in registers (they would be zeros).
// XH (tiled, with XT, M > 8): the rows pass through an 8-row LDS area in two
// rounds, rows 0..7 and then 8..15, where 16 rows would not fit.
constexpr int kPregMax = 8;
template <int FMT, int IV, int DEPTH, int QG, bool XT, bool TILED = false, bool PREG = false,
          bool R8 = false, bool XH = false>
__global__ void __launch_bounds__(512) mmb_kernel(MmbArgs a) {
  typedef MmbFmt<FMT, QG> F;
  static_assert(!TILED || QG == 4, "the tiled layout has 512-channel slices");
  static_assert(!PREG || XT, "register partials reuse the staged-rows area at the end");
  static_assert(!R8 || XT, "R8 limits the staged rows");
  constexpr int kSliceChB = F::kSliceCh;
  constexpr int kSliceGroupsB = F::kSliceGroups;
  constexpr int XS = F::kSteps;
  constexpr uint32_t kMmbWaveArea = mmb_wave_area(QG, TILED);
  constexpr bool OUT = IV > 0;
  extern __shared__ __align__(16) unsigned char smem[];
  const int n_out = OUT ? a.n_out : 0;
  static_assert(!XH || (XT && !R8 && TILED), "two rounds: whole rows of 512-channel slices, M > 8");
  const MmbLds L = mmb_lds_layout(FMT, a.M, a.nw, a.rbl, QG, a.nks, IV, XT, TILED, PREG, XH);
  uint32_t* s_runs = reinterpret_cast<uint32_t*>(smem + L.runs);
  const int32_t* s_idx = reinterpret_cast<const int32_t*>(smem + L.idx);
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15;   // weight row of B / activation row of A
  const int q = lane >> 4;     // k-quarter
  const int G = a.K >> 5;
  const uint32_t row_bytes = (uint32_t)a.K / F::kRowBytesDiv;
  const int nrb_wg = (a.nrb - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int ns_w = (a.nks - w + a.nw - 1) / a.nw;
  const int T = ns_w * nrb_wg;

  const uint64_t tiles = (uint64_t)a.nrb * a.nks;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(
      a.codes, clamp_bytes(TILED ? tiles * 16 * F::kSliceBytes : (uint64_t)a.N * row_bytes));
  const uint64_t meta = TILED ? tiles * (FMT == 5 ? 640 : 1024) : (uint64_t)a.N * G * 2;
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.scales, clamp_bytes(meta));
  // W4P: zero points packed two per byte, (G / 2) bytes per row (G is even here)
  const __amdgpu_buffer_rsrc_t zrs =
      make_rsrc(TILED ? a.scales : a.zeros,
                clamp_bytes(TILED ? meta : FMT == 5 ? (uint64_t)a.N * (G / 2) : meta));
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(
      a.out_w, clamp_bytes(TILED ? (uint64_t)a.nrb * a.nch * 256
                                 : ((uint64_t)a.N * n_out * 2 + 3) & ~(uint64_t)3));
  // tiled slab: slice ks owns chunks chunk_lo(ks) .. chunk_lo(ks + 1) - 1
  auto chunk_lo = [&](int ks) { return (uint32_t)(ks * a.nch) / (uint32_t)a.nks; };
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(a.out_idx, ((uint32_t)n_out * 4u + 15u) & ~15u);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.X, clamp_bytes((uint64_t)a.M * a.K * 2));
  const __amdgpu_buffer_rsrc_t nul = make_rsrc(a.codes, 0u);

  // ---- (0) outlier indices (wave 0: lane l holds idx[256 v + 4 l + k]; they
  //      become the run table below), then the activation rows of this
  //      wave's first slice
  int32_t oidx[IV > 0 ? IV : 1][4];
  if constexpr (OUT) {
#pragma unroll
    for (int v = 0; v < IV; ++v) {
      const u4v t = ld128(w == 0 ? irs : nul, (uint32_t)(256 * v + 4 * lane) * 4u);
      oidx[v][0] = (int32_t)t.x;
      oidx[v][1] = (int32_t)t.y;
      oidx[v][2] = (int32_t)t.z;
      oidx[v][3] = (int32_t)t.w;
    }
  }
  // lane (m, q) of slice ks: channels 128 QG ks + 32 QG q + 8 t (t < 4 QG),
  // i.e. the QG groups 4 QG ks + QG q + u, 32 channels each; past K they read
  // 0 (fixed up when the fragments are built)
  // XT: load t covers whole rows instead (4 / QG rows of the slice, lane l
  // at row t (4 / QG) + l / (16 QG), channels 8 (l % (16 QG)) .. + 7), so each
  // load is contiguous; the rows reach the lane layout above through LDS when
  // the slice is entered.
  constexpr int kXLanesPerRow = 16 * QG;
  constexpr int kXRowsPerLoad = kWave / kXLanesPerRow;
  // loads (and registers) of a slice's activation rows: R8 stages rows 0..7
  constexpr int XL = (XT && R8) ? 8 / kXRowsPerLoad : XS;
  static_assert(!XH || kXRowsPerLoad == 1, "two rounds of whole rows");
  auto x_load = [&](int ks, u4v (&xv)[XL]) {
    if constexpr (XT) {
      const uint32_t c = (uint32_t)(ks * kSliceChB + 8 * (lane % kXLanesPerRow));
#pragma unroll
      for (int t = 0; t < XL; ++t) {
        const uint32_t row = (uint32_t)(t * kXRowsPerLoad + lane / kXLanesPerRow);
        xv[t] = ld128(xrs, (row * (uint32_t)a.K + c) * 2u);
      }
    } else {
      const uint32_t rowoff = (uint32_t)n16 * (uint32_t)a.K;
#pragma unroll
      for (int t = 0; t < XS; ++t) {
        const uint32_t c = (uint32_t)(ks * kSliceChB + 32 * QG * q + 8 * t);
        xv[t] = ld128(xrs, (rowoff + c) * 2u);
      }
    }
  };
  // XT with outliers: two slices of rows in flight (even slices in xpre, odd
  // ones in xpre2), as the weights are two items ahead (measured: the W2
  // 8192 x 28672 layer at M = 8 gains 8%; without outliers the registers cost
  // more than the earlier loads gain, and on the tiled layout, even with R8's
  // eight rows, that layer at M = 8 goes from 33.3 to 36.7 us)
  constexpr bool X2 = XT && OUT && !TILED;
  u4v xpre[XL];
  u4v xpre2[X2 ? XL : 1];
  x_load(w, xpre);
  if constexpr (X2)
    if (1 < ns_w) x_load(w + a.nw, xpre2);
  asm volatile("" ::: "memory");   // these loads stay ahead of the weight stream

  // slice ks's run of the sorted indices: positions j_lo .. j_lo + nin - 1
  auto jrange = [&](int ks, int& j_lo, int& nin) {
    j_lo = 0;
    nin = 0;
    if constexpr (OUT) {
      j_lo = (int)s_runs[ks];
      nin = (int)s_runs[ks + 1] - j_lo;
    }
  };

  // ---- (1) the ring
  auto load_main = [&](ItemB<FMT, OUT, QG>& it, bool valid, int ks, int rb) {
    const __amdgpu_buffer_rsrc_t c_ = valid ? crs : nul;
    const __amdgpu_buffer_rsrc_t s_ = valid ? srs : nul;
    const __amdgpu_buffer_rsrc_t z_ = valid ? zrs : nul;
    const uint32_t row = (uint32_t)(rb * 16 + n16);
    if constexpr (TILED) {
      // tile (rb, ks); lane (n, q): W4 load u = group 4q + u, at 1024 q + 16 (n + 16 u);
      // W2 load v = groups 4q + 2v, + 1, at 1024 (q / 2) + 16 (n + 16 (2 (q % 2) + v))
      const uint32_t tile = (uint32_t)(rb * a.nks + ks);
      const uint32_t cb = tile * (16u * F::kSliceBytes) +
                          (FMT == 2 ? 1024u * (uint32_t)(q >> 1) + 16u * (uint32_t)(n16 + 32 * (q & 1))
                                    : 1024u * (uint32_t)q + 16u * (uint32_t)n16);
#pragma unroll
      for (int u = 0; u < F::kLoads; ++u) it.cw[u] = ld128(c_, cb + 256u * u);
      if constexpr (FMT == 5) {   // 640-byte tile: 4 scales per lane, then 4 packed zeros
        it.sv = ld64(s_, tile * 640u + 8u * (uint32_t)lane);
        it.zv = (u2){(uint32_t)ld16(s_, tile * 640u + 512u + 2u * (uint32_t)lane), 0u};
      } else {
        const u4v m = ld128(s_, tile * 1024u + 16u * (uint32_t)lane);
        it.sv = (u2){m.x, m.y};
        it.zv = (u2){m.z, m.w};
      }
      return;
    }
    const uint32_t rbase = row * row_bytes + (uint32_t)(ks * F::kSliceBytes + 16 * F::kLoads * q);
#pragma unroll
    for (int u = 0; u < F::kLoads; ++u) it.cw[u] = ld128(c_, rbase + 16u * u);
    const uint32_t mo = (row * (uint32_t)G + (uint32_t)(ks * kSliceGroupsB + QG * q)) * 2u;
    if constexpr (QG == 4)
      it.sv = ld64(s_, mo);
    else
      it.sv = (u2){ld32(s_, mo), 0u};
    if constexpr (FMT == 5) {   // the QG groups' nibbles: QG / 2 bytes of the packed row
      const uint32_t zo = row * (uint32_t)(G / 2) + (uint32_t)((kSliceGroupsB * ks + QG * q) / 2);
      it.zv = (u2){QG == 4 ? (uint32_t)ld16(z_, zo) : (uint32_t)ld8(z_, zo), 0u};
    } else if constexpr (QG == 4) {
      it.zv = ld64(z_, mo);
    } else {
      it.zv = (u2){ld32(z_, mo), 0u};
    }
  };
  auto load_slab = [&](ItemB<FMT, OUT, QG>& it, bool valid, int ks, int rb) {
    if constexpr (OUT && TILED) {
      const uint32_t c0 = chunk_lo(ks);
      const bool on = valid && (uint32_t)q < chunk_lo(ks + 1) - c0;
      const uint32_t off = ((uint32_t)rb * (uint32_t)a.nch + c0) * 256u + 16u * (uint32_t)lane;
      const u4v t = ld128(ors, on ? off : kOob);
      it.od[0] = t.x;
      it.od[1] = t.y;
      it.od[2] = t.z;
      it.od[3] = t.w;
    } else if constexpr (OUT) {
      int j_lo, nin;
      jrange(ks, j_lo, nin);
      const __amdgpu_buffer_rsrc_t o_ = valid ? ors : nul;
      const uint32_t row = (uint32_t)(rb * 16 + n16);
      const uint32_t e0 = row * (uint32_t)n_out + (uint32_t)(j_lo + 8 * q);
      const uint32_t b0 = (e0 * 2u) & ~3u;
#pragma unroll
      for (int i = 0; i < 5; ++i) it.od[i] = ld32(o_, b0 + 4u * i);
    }
  };
  int ls = 0, lr = 0;
  auto advance = [&](int& s_, int& q_) {
    if (++q_ == nrb_wg) {
      q_ = 0;
      ++s_;
    }
  };
  ItemB<FMT, OUT, QG> buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    load_main(buf[d], d < T, w + a.nw * ls, blockIdx.x + lr * gridDim.x);
    advance(ls, lr);
    if (d == 0 && FMT == 2) {   // W2 centroid table (as in the M = 1 kernel)
      // 16-byte chunk ch: copies 2 (ch % 16) and 2 (ch % 16) + 1 of entry ch / 16
      u4v* lut = reinterpret_cast<u4v*>(smem + L.lut);
      for (int ch = tid; ch < 256 * 16; ch += nthr) {
        const uint32_t e = (uint32_t)ch >> 4;
        const uint32_t lo = w2_centroid_pair((e & 3u) | (((e >> 2) & 3u) << 16));
        const uint32_t hi = w2_centroid_pair(((e >> 4) & 3u) | ((e >> 6) << 16));
        lut[ch] = (u4v){lo, hi, lo, hi};
      }
      // with outliers the run table's barrier below covers the table too
      // (one wait for the slowest wave instead of two)
      if constexpr (!OUT) lds_barrier();
    }
  }
  if constexpr (OUT) {
    // the run table, built once per workgroup by wave 0: counts per slice,
    // then their prefix sums (the indices are sorted, so slice ks's run starts
    // at the number of indices below 128 QG ks); and the indices into LDS
    if (w == 0) {
      for (int t = lane; t <= a.nks; t += kWave) s_runs[t] = 0u;
      wave_lds_sync();
#pragma unroll
      for (int v = 0; v < IV; ++v) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t j = (uint32_t)(256 * v + 4 * lane + k);
          const int c = oidx[v][k];
          if (j < (uint32_t)n_out && c >= 0 && c < a.K) atomicAdd(&s_runs[c / kSliceChB + 1], 1u);
        }
        reinterpret_cast<u4v*>(smem + L.idx)[64 * v + lane] =
            (u4v){(uint32_t)oidx[v][0], (uint32_t)oidx[v][1], (uint32_t)oidx[v][2],
                  (uint32_t)oidx[v][3]};
      }
      wave_lds_sync();
      // inclusive prefix sums over runs[0 .. nks] (at most 257 words): lane l
      // takes words 5l .. 5l + 4, then the lanes' totals are scanned
      uint32_t v5[5], tot = 0u;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int t = 5 * lane + i;
        v5[i] = t <= a.nks ? s_runs[t] : 0u;
        tot += v5[i];
        v5[i] = tot;
      }
      uint32_t incl = tot;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t u = __shfl_up(incl, d);
        if (lane >= d) incl += u;
      }
      const uint32_t before = incl - tot;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int t = 5 * lane + i;
        if (t <= a.nks) s_runs[t] = before + v5[i];
      }
    }
    lds_barrier();   // the run table, the index copy and the W2 table, visible to every wave
  }
  {
    int s2 = 0, r2 = 0;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      load_slab(buf[d], d < T, w + a.nw * s2, blockIdx.x + r2 * gridDim.x);
      advance(s2, r2);
    }
  }

  // ---- per-slice activation work: outlier-column mask and run list in this
  //      wave's LDS area (parity p), then the run's outlier activations
  const uint32_t warea0 = L.wave + (uint32_t)w * 2u * kMmbWaveArea;
  // The next slice's outlier activations: per position the aligned 4-byte
  // word that holds the FP16 value, and in bit e of xhalf which half of word
  // e it is.  A global gather is issued when the previous slice is entered
  // and its words are first read when their slice is entered: as whole
  // loaded registers (no 16-bit zero extension, no copy into the loop's
  // registers) they make the wave wait neither for them nor, as loads
  // complete in order, for every load issued before them.
  uint32_t xopre[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  uint32_t xhalf = 0u;
  auto prep_slice = [&](int ks, int p) {
    if constexpr (OUT) {
      uint32_t* mask = reinterpret_cast<uint32_t*>(smem + warea0 + (uint32_t)p * kMmbWaveArea);
      // (the tiled layout keeps no run list: its slab is split by position)
      int32_t* list =
          reinterpret_cast<int32_t*>(smem + warea0 + (uint32_t)p * kMmbWaveArea + 16u * QG);
      int j_lo, nin;
      jrange(ks, j_lo, nin);
      const int lo = ks * kSliceChB;
      // the bit mask serves W2 fragments loaded in the lane layout only: W4
      // needs none (its zeroed columns reconstruct to 0), and rows staged
      // through LDS have their outlier columns zeroed there
      constexpr bool kMaskBits = FMT == 2 && !XT;
      if constexpr (kMaskBits || !TILED) {
        if (kMaskBits && lane < 4 * QG) mask[lane] = 0u;
        if constexpr (!TILED)
          for (int j = lane; j < 32; j += kWave) list[j] = -1;   // first run step padded
        wave_lds_sync();
        for (int j = lane; j < nin; j += kWave) {
          const int c = s_idx[j_lo + j] - lo;   // in [0, slice) for sorted indices
          if ((unsigned)c < (unsigned)kSliceChB) {
            if constexpr (kMaskBits)
              __hip_atomic_fetch_or(&mask[c >> 5], 1u << (c & 31), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_WORKGROUP);
            if constexpr (!TILED) list[j] = c;
          }
        }
      }
      // tiled: the activations of the slice's share of slab positions, lane
      // quarter q: positions 8 (C(ks) + q) .. + 7 (past the share: 0)
      if constexpr (TILED) {
        const uint32_t c0 = chunk_lo(ks);
        const uint32_t send = min(8u * chunk_lo(ks + 1), (uint32_t)n_out);
        const uint32_t jmax = (uint32_t)IV * 256u - 1u;   // the LDS copy's last entry
        xhalf = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {   // past the share: read at kOob, which gives 0
          const uint32_t j = 8u * (c0 + (uint32_t)q) + (uint32_t)e;
          const bool ok = j < send;
          const uint32_t col = (uint32_t)s_idx[min(j, jmax)];
          const uint32_t off = ((uint32_t)n16 * (uint32_t)a.K + col) * 2u;
          xopre[e] = ld32(xrs, ok ? (off & ~3u) : kOob);
          xhalf |= ((off >> 1) & 1u) << e;
        }
      }
      // outlier activations of the first 32 columns of the run: X[m][lo + c]
      // (XT: read from the slice's rows in LDS when the slice is entered)
      if constexpr (!XT && !TILED) {
        const int4 l0 = *reinterpret_cast<const int4*>(list + 8 * q);
        const int4 l1 = *reinterpret_cast<const int4*>(list + 8 * q + 4);
        const int cl[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        xhalf = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {   // an idle position reads at kOob, which gives 0
          const bool ok = 8 * q + e < nin && cl[e] >= 0;
          const uint32_t col =
              (uint32_t)(lo + __builtin_amdgcn_ubfe(ok ? cl[e] : 0, 0, QG == 4 ? 9 : 8));
          const uint32_t off = ((uint32_t)n16 * (uint32_t)a.K + col) * 2u;
          xopre[e] = ld32(xrs, ok ? (off & ~3u) : kOob);
          xhalf |= ((off >> 1) & 1u) << e;
        }
      }
    }
  };
  prep_slice(w, 0);

  h8 afr[XS];
  uint32_t xo[4] = {0u, 0u, 0u, 0u};
  int cur_jlo = 0, cur_nin = 0;
  auto enter_slice_rows = [&](int s, auto& xbuf) {
    const int ks = w + a.nw * s;
    const int p = s & 1;
    // the slice's activations in the lane layout of the fragments: read back
    // from LDS when the rows were loaded whole, else the loaded registers
    u4v fv[XT ? XS : 1];
    auto xf = [&](int t) -> u4v {
      if constexpr (XT)
        return fv[t];
      else
        return xbuf[t];
    };
    if constexpr (XT) {
      // the slice's rows, loaded whole, into this wave's LDS area and back in
      // the lane layout of the fragments (lane (m, q): channels 32 QG q + 8 t
      // of row m); rows past M are zero.  NR = 2 (XH): through the 8-row
      // area, rows 0..7 and then 8..15
      const uint32_t mpx = (uint32_t)((a.M + 3) & ~3);
      {
        constexpr int NR = XH ? 2 : 1;
        const uint32_t arows = NR == 2 ? 8u : mpx;
        const uint32_t xbase = L.xt + (uint32_t)w * arows * mmb_xt_stride(QG);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const uint32_t r0 = 8u * (uint32_t)r;   // the round's first row
          if (r > 0) wave_lds_sync();             // after the first round's reads
#pragma unroll
          for (int t = 0; t < XL; ++t) {
            if (NR == 2 && t / 8 != r) continue;   // a constant once unrolled
            const uint32_t row = (uint32_t)(t * kXRowsPerLoad + lane / kXLanesPerRow);
            if (row < mpx)
              *reinterpret_cast<u4v*>(smem + xbase + (row - r0) * mmb_xt_stride(QG) +
                                      16u * (uint32_t)(lane % kXLanesPerRow)) = xbuf[t];
          }
          wave_lds_sync();
          if constexpr (OUT && !TILED) {
            // the run's first 32 outlier activations from the same rows (the
            // slice's column list was written when the previous slice was entered)
            const int32_t* list = reinterpret_cast<const int32_t*>(
                smem + warea0 + (uint32_t)p * kMmbWaveArea + 16u * QG);
            int j_lo, nin;
            jrange(ks, j_lo, nin);
            const int4 l0 = *reinterpret_cast<const int4*>(list + 8 * q);
            const int4 l1 = *reinterpret_cast<const int4*>(list + 8 * q + 4);
            const int cl[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
            xhalf = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const bool ok =
                  8 * q + e < nin && cl[e] >= 0 && cl[e] < kSliceChB && (uint32_t)n16 < mpx;
              xopre[e] = ok ? (uint32_t)*reinterpret_cast<const uint16_t*>(
                                  smem + xbase + (uint32_t)n16 * mmb_xt_stride(QG) + (uint32_t)cl[e] * 2u)
                            : 0u;
            }
          }
          if constexpr (FMT == 2 && OUT) {
            // W2 outlier columns of the slice: zero in every staged row (after
            // the run's activations above were read from them)
            int j_lo, nin;
            jrange(ks, j_lo, nin);
            const int lo = ks * kSliceChB;
            wave_lds_sync();
            const uint32_t mr = mpx - r0 < arows ? mpx - r0 : arows;
            for (int j = lane; j < nin; j += kWave) {
              const int c = s_idx[j_lo + j] - lo;
              if ((unsigned)c < (unsigned)kSliceChB)
                for (uint32_t m = 0; m < mr; ++m)
                  *reinterpret_cast<uint16_t*>(smem + xbase + m * mmb_xt_stride(QG) + (uint32_t)c * 2u) = 0;
            }
            wave_lds_sync();
          }
          if (NR == 1 || (uint32_t)n16 / 8u == (uint32_t)r) {
#pragma unroll
            for (int t = 0; t < XS; ++t)
              fv[t] = (uint32_t)n16 < mpx
                          ? *reinterpret_cast<const u4v*>(smem + xbase + ((uint32_t)n16 - r0) * mmb_xt_stride(QG) +
                                                           (uint32_t)(32 * QG * q + 8 * t) * 2u)
                          : (u4v){0u, 0u, 0u, 0u};
          }
        }
      }
    }
    // fragments of this slice from the prefetched rows (channels past K: 0)
    uint32_t fr[XS][4];
    // a slice inside K needs no selects (uniform: every lane's channels lie
    // below (ks + 1) * slice)
    const bool inside = (ks + 1) * kSliceChB <= a.K;
    if constexpr (FMT == 2) {
      if (inside) {
#pragma unroll
        for (int t = 0; t < XS; ++t) {
          fr[t][0] = xf(t).x;
          fr[t][1] = xf(t).y;
          fr[t][2] = xf(t).z;
          fr[t][3] = xf(t).w;
        }
      } else {
#pragma unroll
        for (int t = 0; t < XS; ++t) {
          const bool ok = ks * kSliceChB + 32 * QG * q + 8 * t < a.K;
          fr[t][0] = ok ? xf(t).x : 0u;
          fr[t][1] = ok ? xf(t).y : 0u;
          fr[t][2] = ok ? xf(t).z : 0u;
          fr[t][3] = ok ? xf(t).w : 0u;
        }
      }
      if constexpr (OUT && !XT) {
        // zero the outlier columns: bits 2i, 2i + 1 of step t's byte
        const uint32_t* mask =
            reinterpret_cast<const uint32_t*>(smem + warea0 + (uint32_t)p * kMmbWaveArea);
        uint32_t mw[QG];
#pragma unroll
        for (int i = 0; i < QG; ++i) mw[i] = mask[QG * q + i];
#pragma unroll
        for (int t = 0; t < XS; ++t) {
          const uint32_t byte = (mw[t >> 2] >> (8 * (t & 3))) & 0xFFu;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t b2 = (byte >> (2 * i)) & 3u;
            const uint32_t keep = (b2 & 1u ? 0u : 0x0000FFFFu) | (b2 & 2u ? 0u : 0xFFFF0000u);
            fr[t][i] &= keep;
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < QG; ++u) {
        const bool ok = inside || ks * kSliceGroupsB + QG * q + u < G;
        uint32_t gv[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u4v t = xf(4 * u + v);
          gv[4 * v + 0] = ok ? t.x : 0u;
          gv[4 * v + 1] = ok ? t.y : 0u;
          gv[4 * v + 2] = ok ? t.z : 0u;
          gv[4 * v + 3] = ok ? t.w : 0u;
        }
        // step t, word i: codes k0 = 16 (t & 1) + 4 i + (t >> 1) and k0 + 2
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k0 = 16 * (t & 1) + 4 * i;
            fr[4 * u + t][i] = __builtin_amdgcn_perm(gv[k0 / 2 + 1], gv[k0 / 2],
                                                     (t >> 1) ? 0x07060302u : 0x05040100u);
          }
      }
    }
#pragma unroll
    for (int f = 0; f < XS; ++f)
      afr[f] = __builtin_bit_cast(h8, (u4v){fr[f][0], fr[f][1], fr[f][2], fr[f][3]});
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (xhalf >> (2 * i)) & 1u ? xopre[2 * i] >> 16 : xopre[2 * i] & 0xFFFFu;
      const uint32_t hi =
          (xhalf >> (2 * i + 1)) & 1u ? xopre[2 * i + 1] >> 16 : xopre[2 * i + 1] & 0xFFFFu;
      xo[i] = lo | (hi << 16);
    }
    // the words are consumed here, before the next slice's gather reuses
    // their registers (without this point the combine sinks below the new
    // loads, the old and new words overlap, and the loaded values are copied)
    asm volatile("" : "+v"(xo[0]), "+v"(xo[1]), "+v"(xo[2]), "+v"(xo[3])::"memory");
    jrange(ks, cur_jlo, cur_nin);
    // the next rows into the buffer just read (X2: two slices ahead, the
    // buffers alternate; else the next slice) and the next slice's outlier
    // activations
    if constexpr (X2) {
      if (s + 2 < ns_w) x_load(ks + 2 * a.nw, xbuf);
    } else {
      if (s + 1 < ns_w) x_load(ks + a.nw, xbuf);
    }
    if (s + 1 < ns_w) prep_slice(ks + a.nw, p ^ 1);
  };
  auto enter_slice = [&](int s) {
    if constexpr (X2) {
      if (s & 1)
        enter_slice_rows(s, xpre2);
      else
        enter_slice_rows(s, xpre);
    } else {
      enter_slice_rows(s, xpre);
    }
  };

  // Each lane owns its entries of the partial tiles: they start at 0 and each
  // slice's tile is added in program order (a fixed summation order); the four
  // reads go out together, so an item waits for LDS once.
  float* s_part = reinterpret_cast<float*>(smem + L.part);
  const uint32_t lut_lane = (uint32_t)(lane & 31) * 8u;
  const uint32_t Mp = (uint32_t)((a.M + 3) & ~3);
  const bool qrows = 4 * q < a.M;   // this lane quarter holds activation rows
  auto part_at = [&](int ri, int jj) {
    return s_part + (((uint32_t)ri * (uint32_t)a.nw + (uint32_t)w) * Mp + (uint32_t)(4 * q + jj)) *
                        16u + (uint32_t)n16;
  };
  f4 pacc[PREG ? kPregMax : 1];
#pragma unroll
  for (int r = 0; r < (PREG ? kPregMax : 1); ++r) pacc[r] = (f4){0.f, 0.f, 0.f, 0.f};
  if (!PREG && qrows)
    for (int ri = 0; ri < nrb_wg; ++ri)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) *part_at(ri, jj) = 0.f;
  auto add_tile = [&](const f4& c, int ri, int si) {
    (void)si;
    if constexpr (PREG) {   // ri is wave-uniform: one of these adds runs
#pragma unroll
      for (int r = 0; r < kPregMax; ++r)
        if (r == ri) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) pacc[r][jj] += c[jj];
        }
    } else if (qrows) {
      float old[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) old[jj] = *part_at(ri, jj);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) *part_at(ri, jj) = old[jj] + c[jj];
    }
  };
  auto compute = [&](const ItemB<FMT, OUT, QG>& it, int ri, int si) {
    f4 c = {0.f, 0.f, 0.f, 0.f};
    const uint32_t svw[2] = {it.sv.x, it.sv.y}, zvw[2] = {it.zv.x, it.zv.y};
    if constexpr (FMT != 2) {
#pragma unroll
      for (int u = 0; u < QG; ++u) {
        const uint32_t sp = (u & 1) ? splat_hi(svw[u >> 1]) : splat_lo(svw[u >> 1]);
        // -(1024 + z) and -(64 + z) in both halves: exact in FP16
        uint32_t nz, nz64;
        if constexpr (FMT == 5) {   // FP16 -(1024 + z) = 0xE400 | z, -(64 + z) = 0xD400 | 16 z
          const uint32_t z = (zvw[0] >> (4 * u)) & 0x0Fu;
          nz = splat_lo(0xE400u | z);
          nz64 = splat_lo(0xD400u | (z << 4));
        } else {
          const _Float16 zf = __builtin_bit_cast(_Float16, (uint16_t)(zvw[u >> 1] >> (16 * (u & 1))));
          nz = splat_lo((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(-1024.0f16 - zf)));
          nz64 = splat_lo((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(-64.0f16 - zf)));
        }
        const h2 sixteenth = {0.0625f16, 0.0625f16};
        const uint32_t d[4] = {it.cw[u].x, it.cw[u].y, it.cw[u].z, it.cw[u].w};
        uint32_t b[4][4];
        // the FP16 exponent of 1024 held in a register, so that mask and OR
        // fuse into one v_and_or_b32 (a VOP3 instruction takes no literal here)
        uint32_t magic = 0x64006400u;
        asm volatile("" : "+v"(magic));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // low nibbles: 1024 + q; high nibbles masked in place: 1024 + 16 q
          // (exact below 2048), which saves their shifts
          const uint32_t d8 = d[i] >> 8;
          const uint32_t v0 = (d[i] & 0x000F000Fu) | magic;
          const uint32_t v1 = (d[i] & 0x00F000F0u) | magic;
          const uint32_t v2 = (d8 & 0x000F000Fu) | magic;
          const uint32_t v3 = (d8 & 0x00F000F0u) | magic;
          const uint32_t vv[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            // exact q - z: (1024 + q) - (1024 + z), or for the high nibbles
            // (1024 + 16 q) / 16 - (64 + z) in one fused step (the product is
            // exact, and so is the sum); then one rounding: w_hat
            const h2 qz = (t & 1) ? __builtin_elementwise_fma(as_h2(vv[t]), sixteenth, as_h2(nz64))
                                  : as_h2(vv[t]) + as_h2(nz);
            b[t][i] = as_u32(qz * as_h2(sp));
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              afr[4 * u + t], __builtin_bit_cast(h8, (u4v){b[t][0], b[t][1], b[t][2], b[t][3]}), c,
              0, 0, 0);
      }
    } else {
#pragma unroll
      for (int uu = 0; uu < F::kLoads; ++uu) {   // one load: 64 codes, two groups
        const uint32_t sp[2] = {splat_lo(svw[uu]), splat_hi(svw[uu])};
        const uint32_t zp[2] = {splat_lo(zvw[uu]), splat_hi(zvw[uu])};
        const uint32_t d[4] = {it.cw[uu].x, it.cw[uu].y, it.cw[uu].z, it.cw[uu].w};
        u2 lv[16];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t word = d[t >> 1];
          const uint32_t bsel = (uint32_t)(2 * (t & 1));
          lv[2 * t] =
              lds_ld64(L.lut + __builtin_amdgcn_perm(word, lut_lane, 0x0C0C0400u + (bsel << 8)));
          lv[2 * t + 1] =
              lds_ld64(L.lut + __builtin_amdgcn_perm(word, lut_lane, 0x0C0C0500u + (bsel << 8)));
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int g = t >> 2;
          const uint32_t cv[4] = {lv[2 * t].x, lv[2 * t].y, lv[2 * t + 1].x, lv[2 * t + 1].y};
          uint32_t b[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            b[i] = as_u32(__builtin_elementwise_fma(as_h2(cv[i]), as_h2(sp[g]), as_h2(zp[g])));
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              afr[8 * uu + t], __builtin_bit_cast(h8, (u4v){b[0], b[1], b[2], b[3]}), c, 0, 0, 0);
        }
      }
    }
    if constexpr (OUT && TILED) {   // zero-padded chunks: no alignment, no mask
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          __builtin_bit_cast(h8, (u4v){xo[0], xo[1], xo[2], xo[3]}),
          __builtin_bit_cast(h8, (u4v){it.od[0], it.od[1], it.od[2], it.od[3]}), c, 0, 0, 0);
    } else if constexpr (OUT) {
      const uint32_t row = (uint32_t)(((int)blockIdx.x + ri * (int)gridDim.x) * 16 + n16);
      const uint32_t sh = ((row * (uint32_t)n_out + (uint32_t)cur_jlo) & 1u) * 16u;
      // the slab values past the run belong to other positions or rows (or
      // lie past the array): cleared, so that an infinite one never meets a
      // zero activation
      const int cnt = cur_nin - 8 * q;
      uint32_t bw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bw[i] = __builtin_amdgcn_alignbit(it.od[i + 1], it.od[i], sh) &
                (2 * i + 1 < cnt ? 0xFFFFFFFFu : 2 * i < cnt ? 0x0000FFFFu : 0u);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          __builtin_bit_cast(h8, (u4v){xo[0], xo[1], xo[2], xo[3]}),
          __builtin_bit_cast(h8, (u4v){bw[0], bw[1], bw[2], bw[3]}), c, 0, 0, 0);
    }
    add_tile(c, ri, si);
  };

  int si = 0, ri = 0;
  for (int base = 0; base < T; base += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (base + d < T) {
        if (ri == 0) enter_slice(si);
        compute(buf[d], ri, si);
        advance(si, ri);
      }
      load_main(buf[d], base + d + DEPTH < T, w + a.nw * ls, blockIdx.x + lr * gridDim.x);
      load_slab(buf[d], base + d + DEPTH < T, w + a.nw * ls, blockIdx.x + lr * gridDim.x);
      advance(ls, lr);
    }
  }

  // ---- outlier runs longer than 32 columns, after the weight stream (the
  //      tiled layout splits positions, at most 32 per slice)
  if constexpr (OUT && !TILED) {
    for (int s = 0; s < ns_w; ++s) {
      const int ks = w + a.nw * s;
      int j_lo, nin;
      jrange(ks, j_lo, nin);
      for (int c0 = 32; c0 < nin; c0 += 32) {
        // activations of columns j_lo + c0 + 8q + e
        uint32_t hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j_lo + c0 + 8 * q + e;
          const bool ok = c0 + 8 * q + e < nin;
          const int col = ok ? s_idx[j] : 0;
          hv[e] = ok ? (uint32_t)ld16(xrs, ((uint32_t)n16 * (uint32_t)a.K + (uint32_t)col) * 2u) : 0u;
        }
        const u4v xv = {hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                        hv[6] | (hv[7] << 16)};
        for (int r2 = 0; r2 < nrb_wg; ++r2) {
          const uint32_t row = (uint32_t)(((int)blockIdx.x + r2 * (int)gridDim.x) * 16 + n16);
          const uint32_t e0 = row * (uint32_t)n_out + (uint32_t)(j_lo + c0 + 8 * q);
          const uint32_t b0 = (e0 * 2u) & ~3u;
          uint32_t od[5];
#pragma unroll
          for (int i = 0; i < 5; ++i) od[i] = ld32(ors, b0 + 4u * i);
          const int cnt = nin - c0 - 8 * q;   // as in the run's first 32 positions
          uint32_t bw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            bw[i] = __builtin_amdgcn_alignbit(od[i + 1], od[i], (e0 & 1u) * 16u) &
                    (2 * i + 1 < cnt ? 0xFFFFFFFFu : 2 * i < cnt ? 0x0000FFFFu : 0u);
          f4 c = {0.f, 0.f, 0.f, 0.f};
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(h8, xv), __builtin_bit_cast(h8, (u4v){bw[0], bw[1], bw[2], bw[3]}), c,
              0, 0, 0);
          add_tile(c, r2, 1);
        }
      }
    }
  }

  // ---- fixed-order sum of the waves' tiles (register partials: written
  //      into the staged-rows area once every wave is done with it)
  if constexpr (PREG) {
    __syncthreads();
    if (qrows) {
#pragma unroll
      for (int r = 0; r < kPregMax; ++r)
        if (r < nrb_wg) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) *part_at(r, jj) = pacc[r][jj];
        }
    }
  }
  __syncthreads();
  for (int t = tid; t < nrb_wg * a.M * 16; t += nthr) {
    const int n = t & 15, m = (t >> 4) % a.M, ri2 = (t >> 4) / a.M;
    const int row = ((int)blockIdx.x + ri2 * (int)gridDim.x) * 16 + n;
    if (row >= a.N) continue;
    float s = 0.f;
    for (int k = 0; k < a.nw; ++k)
      s += s_part[(((uint32_t)ri2 * a.nw + k) * Mp + (uint32_t)m) * 16u + (uint32_t)n];
    a.Y[(size_t)m * a.N + row] = f2h(s);
  }
}

// ------------------------------------------------------------- launch plan

struct MmaPlan {
  bool ok, preferred;
  int nw, nks, nsw, nswt, nrb, nch, grid, rbl;
  size_t lds;
};

// Waves per workgroup for nks slices: one per slice up to 8, else 8 with the
// leftover slices on waves 0, 1, ...  The first wave on each SIMD (waves 0..3)
// gets its first data well before the second, so a split that gives the early
// waves more slices evens out the finish.  Measured on MI355X (per-wave
// timestamps): W4 4096 x 14336 (28 slices) at M = 8 on 7 waves of 4 slices,
// waves 4..6 entered their first slice 1.8 us after waves 0..3 and finished
// 2.5 us after them.  With 8 waves (4, 4, 4, 4, 3, 3, 3, 3): that layer at
// M = 1 / 4 / 8 / 16 9.69 / 13.03 / 14.35 / 16.35 -> 9.45 / 12.39 / 13.65 /
// 15.60 us; W4 4096 x 6144 (12 slices, 6 waves before) 6.60 / 9.31 ->
// 6.13 / 8.35 us at M = 1 / 8; W2 4096 x 14336 + outliers 9.49 -> 8.69 us.
static int mma_waves(int nks) { return nks <= kMaxWaves ? nks : kMaxWaves; }
// The fused refinement's streaming waves: the fewest wasted slices (28 slices:
// 7 waves), which leaves one more wave for the helpers (W4 4096 x 14336: 9
// helpers, 14.8 us; 8 streaming waves and 8 helpers, 15.1 us).
static int mma_waves_even(int nks) {
  if (nks <= kMaxWaves) return nks;
  int best = -1, nw_best = kMaxWaves;
  for (int nw = kMaxWaves; nw >= 4; --nw) {
    const int waste = ((nks + nw - 1) / nw) * nw - nks;
    if (best < 0 || waste < best) {
      best = waste;
      nw_best = nw;
    }
  }
  return nw_best;
}

static MmaPlan plan_mma1(int fmt, bool tiled, int64_t N, int64_t K, int64_t n_out, int ms,
                         bool refine = false) {
  MmaPlan p{};
  // the row-major layout reads whole 128-channel quarters of a slice from
  // each row; the tiled one is padded to whole slices
  if (K % (tiled ? 32 : 128) != 0 || K > 65536) return p;
  p.nks = (int)((K + kSliceCh - 1) / kSliceCh);
  p.nch = (int)((n_out + 7) / 8);
  p.nrb = (int)((N + 15) / 16);
  // every slice's share of the outlier slab fits the four lane quarters
  if (p.nch > 4 * p.nks) return p;
  if (tiled) {
    const wq::TiledGeometry g = wq::tiled_geometry(fmt, N, K, n_out);
    if (g.meta_off > kMaxArrayBytes || g.slab_off - g.meta_off > kMaxArrayBytes ||
        g.total - g.slab_off > kMaxArrayBytes)
      return p;
  } else {
    const int64_t row_bytes = fmt == 2 ? K / 4 : K / 2;
    if (N * row_bytes > kMaxArrayBytes || N * (K / 32) * 2 > kMaxArrayBytes ||
        N * n_out * 2 > kMaxArrayBytes)
      return p;
  }
  p.nw = refine ? mma_waves_even(p.nks) : mma_waves(p.nks);
  p.nsw = (p.nks + p.nw - 1) / p.nw;
  if (p.nsw > 8) return p;
  p.nswt = p.nsw <= 1 ? 1 : p.nsw <= 2 ? 2 : p.nsw <= 4 ? 4 : 8;
  const int cus = device_cus();
  if (cus <= 0) return p;
  p.grid = std::min(p.nrb, cus);
  p.rbl = (p.nrb + p.grid - 1) / p.grid;
  const MmaLds L = mma_lds_layout(fmt, p.nw, p.nsw, p.rbl, ms);
  p.lds = L.total;
  if (p.lds > kMaxLdsBytes) return p;
  p.ok = true;
  // One workgroup per compute unit: worth it once every unit has a row block.
  // Measured on MI355X: ahead of the VALU kernels for W2 (the centroid table
  // and the v_dot2 work leave the VALU path compute-bound); behind them for
  // W4, whose VALU decode is cheap and whose loads are fully contiguous.
  p.preferred = fmt == 2 && p.nrb >= cus;
  return p;
}


struct MmbPlan {
  bool ok, xt, preg, xh;
  int nw, nks, nrb, grid, rbl, iv, depth, qg;
  size_t lds;
};

static MmbPlan plan_mmb(int fmt, int64_t N, int64_t K, int64_t n_out, int64_t M,
                        const wq_variant* v, bool tiled = false) {
  MmbPlan p{};
  if (K % (tiled ? 32 : 128) != 0 || K > 65536 || n_out > 1024 || M < 2 || M > 16) return p;
  const int64_t row_bytes = fmt == 2 ? K / 4 : K / 2;
  if (tiled) {
    const wq::TiledGeometry g = wq::tiled_geometry(fmt, N, K, n_out);
    if (g.meta_off > kMaxArrayBytes || g.slab_off - g.meta_off > kMaxArrayBytes ||
        g.total - g.slab_off > kMaxArrayBytes || M * K * 2 > 0xFFFFFFF0ll)
      return p;
    // every slice's share of the slab fits the four lane quarters
    if (g.nch > 4 * g.nks) return p;
  } else if (N * row_bytes > 0xFFFFFFF0ll || N * (K / 32) * 2 > 0xFFFFFFF0ll ||
             N * n_out * 2 > 0xFFFFFFF0ll || M * K * 2 > 0xFFFFFFF0ll) {
    return p;
  }
  // 512-channel slices (QG = 4) halve the items and slice changes of layers up
  // to K = 8192 without outliers (measured faster there up to M = 8); longer
  // rows, the outlier variants (whose registers would spill at QG = 4) and
  // more rows keep 256, whose activation rows load whole (measured at M = 16
  // on 14336 x 4096: 14.6 us against 15.8).  An explicit variant may choose
  // either for the kernels without outliers.
  p.qg = n_out == 0 && K <= 8192 && M <= 8 ? 4 : 2;
  if (tiled) {
    p.qg = 4;
  } else if (n_out == 0) {
    const int qg = variant_or(v, &wq_variant::batch_slice_groups, p.qg);
    if (qg == 2 || qg == 4) p.qg = qg;
  }
  const int slice_ch = 128 * p.qg;
  p.nks = (int)((K + slice_ch - 1) / slice_ch);
  p.nw = mma_waves(p.nks);
  p.nrb = (int)((N + 15) / 16);
  const int cus = device_cus();
  if (cus <= 0) return p;
  p.grid = std::min(p.nrb, cus);
  p.rbl = (p.nrb + p.grid - 1) / p.grid;
  p.iv = n_out == 0 ? 0 : n_out <= 256 ? 1 : n_out <= 512 ? 2 : 4;
  p.lds = mmb_lds_layout(fmt, (int)M, p.nw, p.rbl, p.qg, p.nks, p.iv, false, tiled).total;
  if (p.lds > kMaxLdsBytes) return p;
  // The activation rows are loaded whole and transposed in LDS where it fits
  // (an explicit variant may turn it off).  (Measured on MI355X: taking fewer
  // waves per workgroup so that the transpose fits is slower than loading the
  // rows in the fragment layout at 8 waves.)
  const bool want_xt = variant_or(v, &wq_variant::batch_row_transpose, 1) != 0;
  const size_t lds_xt =
      mmb_lds_layout(fmt, (int)M, p.nw, p.rbl, p.qg, p.nks, p.iv, true, tiled).total;
  p.xt = lds_xt <= kMaxLdsBytes && want_xt;
  if (p.xt) p.lds = lds_xt;
  // On the tiled layout at M > 8 the rows may pass through an 8-row area in
  // two rounds where all of them do not fit.  Measured on MI355X: W2 8192 x
  // 28672 + 1003 outliers at M = 16 70.4 -> 46.0 us (rows in the lane layout
  // before), W4 14336 x 4096 at M = 16 14.1 -> 13.2 us (register partials
  // before); where 16 rows fit, two rounds per slice are slower (W4 4096 x
  // 14336 at M = 16 16.9 -> 17.7 us), so only then.
  const bool can_xh = tiled && M > 8;
  if (want_xt && !p.xt && can_xh) {
    const size_t lds_xh =
        mmb_lds_layout(fmt, (int)M, p.nw, p.rbl, p.qg, p.nks, p.iv, true, tiled, false, true).total;
    if (lds_xh <= kMaxLdsBytes) {
      p.xt = p.xh = true;
      p.lds = lds_xh;
    }
  }
  // Partial tiles in registers (a workgroup with at most kPregMax row blocks)
  // leave room for the staged rows where the LDS tiles would not.  Measured on
  // MI355X, the library takes them only then: W2 28672 x 8192 at M = 8 33.2 ->
  // 27.4 us, W4 14336 x 4096 at M = 16 14.1 -> 13.6 us; where the rows fit
  // anyway the per-item register select is slower (W4 14336 x 4096 at M = 8,
  // 11.8 -> 12.7 us).  An explicit variant may ask for them wherever they fit.
  const int preg = variant_or(v, &wq_variant::batch_register_partials, -1);
  if (want_xt && preg != 0 && (preg == 1 || !p.xt) && p.rbl <= kPregMax) {
    // the staging area chosen above, else 16 rows, else (tiled, M > 8) 8
    bool xh = p.xt && p.xh;
    size_t lds_preg =
        mmb_lds_layout(fmt, (int)M, p.nw, p.rbl, p.qg, p.nks, p.iv, true, tiled, true, xh).total;
    if (lds_preg > kMaxLdsBytes && !xh && can_xh) {
      xh = true;
      lds_preg =
          mmb_lds_layout(fmt, (int)M, p.nw, p.rbl, p.qg, p.nks, p.iv, true, tiled, true, true).total;
    }
    if (lds_preg <= kMaxLdsBytes) {
      p.xt = p.preg = true;
      p.xh = xh;
      p.lds = lds_preg;
    }
  }
  // Items in flight per wave: 2, or 1 on the tiled layout without outliers
  // where a workgroup has one row block (every item then starts a new slice).
  // Measured on MI355X (same bits): W4 4096 x 14336 at M = 5 / 8 / 16
  // 13.24 / 13.59 / 15.55 -> 12.02 / 12.63 / 14.68 us; with 3 or more row
  // blocks one item is slower (W4 14336 x 4096 at M = 8 11.1 -> 11.6 us, W2
  // 28672 x 8192 + 286 24.1 -> 26.4 us), and so are 3 items everywhere.
  p.depth = tiled && n_out == 0 && p.rbl == 1 ? 1 : 2;
  p.ok = true;
  return p;
}

}  // namespace wqd

using namespace wqd;

int wqd_gemv_mma(int fmt, bool tiled, const uint8_t* codes, const uint16_t* scales,
                 const uint16_t* zeros, int64_t N, int64_t K, const int32_t* out_idx,
                 const uint16_t* out_w, int64_t n_out, const uint16_t* x, uint16_t* y,
                 hipStream_t stream, const char* who, int mode, bool* launched) {
  return wqd_mma_rows(fmt, tiled, codes, scales, zeros, N, K, out_idx, out_w, n_out, x, 1, y,
                      stream, who, mode, launched);
}

// Kernel arguments of a plan (the tiled layout's three arrays sit at the
// offsets of its geometry inside one buffer).
static MmaArgs mma_args(const MmaPlan& p, int fmt, bool tiled, const uint8_t* codes,
                        const uint16_t* scales, const uint16_t* zeros, int64_t N, int64_t K,
                        const int32_t* out_idx, const uint16_t* out_w, int64_t n_out,
                        const uint16_t* X, int64_t M, uint16_t* Y) {
  MmaArgs a{};
  if (tiled) {
    const wq::TiledGeometry g = wq::tiled_geometry(fmt, N, K, n_out);
    a.codes = codes + g.codes_off;
    a.scales = reinterpret_cast<const uint16_t*>(codes + g.meta_off);
    a.zeros = a.scales;
    a.out_w = reinterpret_cast<const uint16_t*>(codes + g.slab_off);
  } else {
    a.codes = codes;
    a.scales = scales;
    a.zeros = zeros;
    a.out_w = out_w;
  }
  a.out_idx = out_idx;
  a.x = X;
  a.y = Y;
  a.N = (int)N;
  a.K = (int)K;
  a.n_out = (int)n_out;
  a.M = (int)M;
  a.nw = p.nw;
  a.nks = p.nks;
  a.nsw = p.nsw;
  a.nrb = p.nrb;
  a.rbl = p.rbl;
  a.nch = p.nch;
  return a;
}

int wqd_mma_rows(int fmt, bool tiled, const uint8_t* codes, const uint16_t* scales,
                 const uint16_t* zeros, int64_t N, int64_t K, const int32_t* out_idx,
                 const uint16_t* out_w, int64_t n_out, const uint16_t* X, int64_t M, uint16_t* Y,
                 hipStream_t stream, const char* who, int mode, bool* launched) {
  *launched = false;
  if (mode == 0 || M < 1 || M > 4 || (M > 2 && fmt == 2)) return WQ_OK;
  const int ms = M <= 2 ? (int)M : 4;   // three rows run as four, the last one empty
  const MmaPlan p = plan_mma1(fmt, tiled, N, K, n_out, ms);
  if (ms == 4 && p.nswt > 4) return WQ_OK;   // registers: four rows of x per slice
  if (!p.ok || (mode == 1 && !p.preferred)) return WQ_OK;
  const MmaArgs a = mma_args(p, fmt, tiled, codes, scales, zeros, N, K, out_idx, out_w, n_out, X,
                             M, Y);
  const dim3 grid(p.grid), block(p.nw * kWave);
#define WQ_MMA_LAUNCH_R(F_, O_, T_, S_, R_)                                                   \
  if (fmt == F_ && (n_out > 0) == O_ && tiled == T_ && p.nswt == S_ && ms == R_) {            \
    if (!allow_lds(reinterpret_cast<const void*>(&mma1d_kernel<F_, O_, T_, S_, R_, false>),   \
                   p.lds))                                                                    \
      return wq::fail(WQ_ERR_HIP, "%s: cannot raise the LDS limit to %zu bytes", who, p.lds);  \
    hipLaunchKernelGGL((mma1d_kernel<F_, O_, T_, S_, R_, false>), grid, block, p.lds, stream, a); \
    *launched = true;                                                                         \
    return check_launch(who);                                                                 \
  }
#define WQ_MMA_LAUNCH(F_, O_, T_, S_) WQ_MMA_LAUNCH_R(F_, O_, T_, S_, 1) WQ_MMA_LAUNCH_R(F_, O_, T_, S_, 2)
// four rows: W4 and W4P, at most 4 slices per wave
#define WQ_MMA_SLICES4(F_, O_, T_) \
  WQ_MMA_LAUNCH_R(F_, O_, T_, 1, 4) WQ_MMA_LAUNCH_R(F_, O_, T_, 2, 4) WQ_MMA_LAUNCH_R(F_, O_, T_, 4, 4)
#define WQ_MMA_LAYOUTS4(F_, O_) WQ_MMA_SLICES4(F_, O_, false) WQ_MMA_SLICES4(F_, O_, true)
#define WQ_MMA_SLICES(F_, O_, T_) \
  WQ_MMA_LAUNCH(F_, O_, T_, 1) WQ_MMA_LAUNCH(F_, O_, T_, 2) WQ_MMA_LAUNCH(F_, O_, T_, 4) \
  WQ_MMA_LAUNCH(F_, O_, T_, 8)
#define WQ_MMA_LAYOUTS(F_, O_) WQ_MMA_SLICES(F_, O_, false) WQ_MMA_SLICES(F_, O_, true)
  WQ_MMA_LAYOUTS(4, false) WQ_MMA_LAYOUTS(4, true) WQ_MMA_LAYOUTS(2, false) WQ_MMA_LAYOUTS(2, true)
  WQ_MMA_LAYOUTS(5, false) WQ_MMA_LAYOUTS(5, true)
  WQ_MMA_LAYOUTS4(4, false) WQ_MMA_LAYOUTS4(4, true) WQ_MMA_LAYOUTS4(5, false)
  WQ_MMA_LAYOUTS4(5, true)
#undef WQ_MMA_SLICES
#undef WQ_MMA_LAYOUTS
#undef WQ_MMA_LAUNCH
#undef WQ_MMA_LAUNCH_R
#undef WQ_MMA_SLICES4
#undef WQ_MMA_LAYOUTS4
  return WQ_OK;
}

int wqd_gemv_refine_mma(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                        const int32_t* out_idx, int64_t n_out, const uint16_t* x, uint16_t* y,
                        const uint8_t* rcodes, const uint16_t* rscales, const uint16_t* rzeros,
                        int64_t chunk, int64_t k, int32_t* sel_out, const wq_variant* v,
                        hipStream_t stream, const char* who, bool* launched) {
  *launched = false;
  MmaPlan p = plan_mma1(fmt, true, N, K, n_out, 1, true);
  if (!p.ok || chunk < 1 || k < 1) return WQ_OK;
  const int rk = (int)std::min(k, chunk);
  const int rnch = (int)((K + chunk - 1) / chunk);
  const int rp = (rk + 31) / 32;
  const int rh = (p.rbl + 1) / 2;
  // Helper waves, at most one per chunk: a 12-wave workgroup, or 16 waves for
  // the W4 / W4P kernels without outliers (they fit 128 VGPRs) where the extra
  // helpers take a chunk off every helper's share.  The wider plan is tried
  // first; if its units or LDS do not fit, the 12-wave plan is tried.
  const int nh12 = std::min(rnch, kRefMaxThreads / kWave - p.nw);
  int cand_nh[2] = {0, 0};
  bool cand_wide[2] = {false, false};
  int ncand = 0;
  if (fmt != 2 && n_out == 0 && variant_or(v, &wq_variant::refine_wide, 1) != 0) {
    const int nhw = std::min(rnch, kRefWideThreads / kWave - p.nw);
    if (nhw >= 1 && (nh12 < 1 || (rnch + nhw - 1) / nhw < (rnch + nh12 - 1) / nh12)) {
      cand_nh[ncand] = nhw;
      cand_wide[ncand++] = true;
    }
  }
  if (nh12 >= 1) {
    cand_nh[ncand] = nh12;
    cand_wide[ncand++] = false;
  }
  int nh = 0, rc = 0;
  bool wide = false;
  for (int c = 0; c < ncand && nh == 0; ++c) {
    const int rcc = (rnch + cand_nh[c] - 1) / cand_nh[c];
    if ((int64_t)rcc * rp * rh > kRefUnits) continue;   // registers: at most 4 units per lane
    const MmaLds Lc = mma_lds_layout(fmt, p.nw, p.nsw, p.rbl, 1, rnch, rk, cand_nh[c]);
    if (Lc.total > kMaxLdsBytes) continue;
    nh = cand_nh[c];
    rc = rcc;
    wide = cand_wide[c];
    p.lds = Lc.total;
  }
  if (nh == 0) return WQ_OK;
  MmaArgs a = mma_args(p, fmt, true, tiled, nullptr, nullptr, N, K, out_idx, nullptr, n_out, x,
                       1, y);
  a.rcodes = rcodes;
  a.rscales = rscales;
  a.rzeros = rzeros;
  a.sel_out = sel_out;
  a.rchunk = (int)chunk;
  a.rk = rk;
  a.rnch = rnch;
  a.nh = nh;
  a.rc = rc;
  a.rp = rp;
  a.rh = rh;
  const dim3 grid(p.grid), block((p.nw + nh) * kWave);
#define WQ_MMA_REF_WIDE(F_, S_)                                                               \
  if (wide && fmt == F_ && p.nswt == S_) {                                                     \
    if (!allow_lds(reinterpret_cast<const void*>(&mma1d_kernel<F_, false, true, S_, 1, true, true>), \
                   p.lds))                                                                     \
      return wq::fail(WQ_ERR_HIP, "%s: cannot raise the LDS limit to %zu bytes", who, p.lds);   \
    hipLaunchKernelGGL((mma1d_kernel<F_, false, true, S_, 1, true, true>), grid, block, p.lds,   \
                       stream, a);                                                             \
    *launched = true;                                                                          \
    return check_launch(who);                                                                  \
  }
  WQ_MMA_REF_WIDE(4, 1) WQ_MMA_REF_WIDE(4, 2) WQ_MMA_REF_WIDE(4, 4) WQ_MMA_REF_WIDE(4, 8)
  WQ_MMA_REF_WIDE(5, 1) WQ_MMA_REF_WIDE(5, 2) WQ_MMA_REF_WIDE(5, 4) WQ_MMA_REF_WIDE(5, 8)
#undef WQ_MMA_REF_WIDE
  if (wide) return WQ_OK;
#define WQ_MMA_REF(F_, O_, S_)                                                                \
  if (fmt == F_ && (n_out > 0) == O_ && p.nswt == S_) {                                        \
    if (!allow_lds(reinterpret_cast<const void*>(&mma1d_kernel<F_, O_, true, S_, 1, true>),    \
                   p.lds))                                                                     \
      return wq::fail(WQ_ERR_HIP, "%s: cannot raise the LDS limit to %zu bytes", who, p.lds);   \
    hipLaunchKernelGGL((mma1d_kernel<F_, O_, true, S_, 1, true>), grid, block, p.lds, stream, a); \
    *launched = true;                                                                          \
    return check_launch(who);                                                                  \
  }
#define WQ_MMA_REF_S(F_, O_) WQ_MMA_REF(F_, O_, 1) WQ_MMA_REF(F_, O_, 2) WQ_MMA_REF(F_, O_, 4) \
  WQ_MMA_REF(F_, O_, 8)
  WQ_MMA_REF_S(2, true) WQ_MMA_REF_S(2, false) WQ_MMA_REF_S(4, true) WQ_MMA_REF_S(4, false)
  WQ_MMA_REF_S(5, true) WQ_MMA_REF_S(5, false)
#undef WQ_MMA_REF_S
#undef WQ_MMA_REF
  return WQ_OK;
}

int wqd_gemm_mma(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                 int64_t N, int64_t K, const int32_t* out_idx, const uint16_t* out_w,
                 int64_t n_out, const uint16_t* X, int64_t M, uint16_t* Y, const wq_variant* v,
                 hipStream_t stream, const char* who, int mode, bool* launched) {
  *launched = false;
  if (mode == 0) return WQ_OK;
  const MmbPlan p = plan_mmb(fmt, N, K, n_out, M, v);
  if (!p.ok) return WQ_OK;
  MmbArgs a{};
  a.codes = codes;
  a.scales = scales;
  a.zeros = zeros;
  a.out_idx = out_idx;
  a.out_w = out_w;
  a.X = X;
  a.Y = Y;
  a.N = (int)N;
  a.K = (int)K;
  a.M = (int)M;
  a.n_out = (int)n_out;
  a.nw = p.nw;
  a.nks = p.nks;
  a.nrb = p.nrb;
  a.rbl = p.rbl;
  const dim3 grid(p.grid), block(p.nw * kWave);
  // staged rows: at most 8 for M <= 8
  const bool r8 = p.xt && M <= 8;
#define WQ_MMB_LAUNCH_XPR(F_, IV_, Q_, X_, P_, R_)                                               \
  if (fmt == F_ && p.iv == IV_ && p.qg == Q_ && p.xt == X_ && p.preg == P_ && r8 == R_) {     \
    if (!allow_lds(reinterpret_cast<const void*>(&mmb_kernel<F_, IV_, 2, Q_, X_, false, P_, R_>), \
                   p.lds))                                                                       \
      return wq::fail(WQ_ERR_HIP, "%s: cannot raise the LDS limit to %zu bytes", who, p.lds);    \
    hipLaunchKernelGGL((mmb_kernel<F_, IV_, 2, Q_, X_, false, P_, R_>), grid, block, p.lds, stream, \
                       a);                                                                       \
    *launched = true;                                                                           \
    return check_launch(who);                                                                   \
  }
#define WQ_MMB_LAUNCH_XP(F_, IV_, Q_, X_, P_) \
  WQ_MMB_LAUNCH_XPR(F_, IV_, Q_, X_, P_, false) WQ_MMB_LAUNCH_XPR(F_, IV_, Q_, X_, P_, X_)
#define WQ_MMB_LAUNCH_X(F_, IV_, Q_, X_) WQ_MMB_LAUNCH_XP(F_, IV_, Q_, X_, false) WQ_MMB_LAUNCH_XP(F_, IV_, Q_, X_, X_)
#define WQ_MMB_LAUNCH(F_, IV_) WQ_MMB_LAUNCH_X(F_, IV_, 2, false) WQ_MMB_LAUNCH_X(F_, IV_, 2, true)
  WQ_MMB_LAUNCH_X(4, 0, 4, false) WQ_MMB_LAUNCH_X(2, 0, 4, false) WQ_MMB_LAUNCH_X(5, 0, 4, false)
  WQ_MMB_LAUNCH_X(4, 0, 4, true) WQ_MMB_LAUNCH_X(2, 0, 4, true) WQ_MMB_LAUNCH_X(5, 0, 4, true)
  WQ_MMB_LAUNCH(4, 0) WQ_MMB_LAUNCH(4, 1) WQ_MMB_LAUNCH(4, 2) WQ_MMB_LAUNCH(4, 4)
  WQ_MMB_LAUNCH(2, 0) WQ_MMB_LAUNCH(2, 1) WQ_MMB_LAUNCH(2, 2) WQ_MMB_LAUNCH(2, 4)
  WQ_MMB_LAUNCH(5, 0) WQ_MMB_LAUNCH(5, 1) WQ_MMB_LAUNCH(5, 2) WQ_MMB_LAUNCH(5, 4)
#undef WQ_MMB_LAUNCH_X
#undef WQ_MMB_LAUNCH_XP
#undef WQ_MMB_LAUNCH_XPR
#undef WQ_MMB_LAUNCH
  return WQ_OK;
}

int wqd_gemm_mma_tiled(int fmt, const uint8_t* tiled, int64_t N, int64_t K,
                       const int32_t* out_idx, int64_t n_out, const uint16_t* X, int64_t M,
                       uint16_t* Y, const wq_variant* v, hipStream_t stream, const char* who,
                       bool* launched) {
  *launched = false;
  const MmbPlan p = plan_mmb(fmt, N, K, n_out, M, v, true);
  if (!p.ok) return WQ_OK;
  const wq::TiledGeometry g = wq::tiled_geometry(fmt, N, K, n_out);
  MmbArgs a{};
  a.codes = tiled + g.codes_off;
  a.scales = reinterpret_cast<const uint16_t*>(tiled + g.meta_off);
  a.zeros = a.scales;
  a.out_w = reinterpret_cast<const uint16_t*>(tiled + g.slab_off);
  a.out_idx = out_idx;
  a.X = X;
  a.Y = Y;
  a.N = (int)N;
  a.K = (int)K;
  a.M = (int)M;
  a.n_out = (int)n_out;
  a.nw = p.nw;
  a.nks = p.nks;
  a.nrb = p.nrb;
  a.rbl = p.rbl;
  a.nch = (int)g.nch;
  const dim3 grid(p.grid), block(p.nw * kWave);
  // staged rows: at most 8 for M <= 8 (measured on MI355X: W2 8192 x 28672 +
  // 1003 outliers at M = 8 38.0 -> 36.1 us, W4 14336 x 4096 11.86 -> 11.46 us;
  // with only those rows' registers held, 35.2 -> 33.3 us and W4 4096 x 14336
  // 15.2 -> 14.45 us)
  const bool r8 = p.xt && M <= 8;
#define WQ_MMT_LAUNCH_XPRHD(F_, IV_, X_, P_, R_, H_, D_)                                          \
  if (fmt == F_ && p.iv == IV_ && p.xt == X_ && p.preg == P_ && r8 == R_ && p.xh == H_ &&        \
      p.depth == D_) {                                                                           \
    if (!allow_lds(reinterpret_cast<const void*>(&mmb_kernel<F_, IV_, D_, 4, X_, true, P_, R_, H_>), \
                   p.lds))                                                                       \
      return wq::fail(WQ_ERR_HIP, "%s: cannot raise the LDS limit to %zu bytes", who, p.lds);    \
    hipLaunchKernelGGL((mmb_kernel<F_, IV_, D_, 4, X_, true, P_, R_, H_>), grid, block, p.lds,    \
                       stream, a);                                                               \
    *launched = true;                                                                           \
    return check_launch(who);                                                                   \
  }
#define WQ_MMT_LAUNCH_XPRH(F_, IV_, X_, P_, R_, H_) \
  WQ_MMT_LAUNCH_XPRHD(F_, IV_, X_, P_, R_, H_, 2) WQ_MMT_LAUNCH_XPRHD(F_, IV_, X_, P_, R_, H_, (IV_ == 0 ? 1 : 2))
#define WQ_MMT_LAUNCH_XPR(F_, IV_, X_, P_, R_) \
  WQ_MMT_LAUNCH_XPRH(F_, IV_, X_, P_, R_, false) WQ_MMT_LAUNCH_XPRH(F_, IV_, X_, P_, R_, (X_ && !R_))
#define WQ_MMT_LAUNCH_XP(F_, IV_, X_, P_) \
  WQ_MMT_LAUNCH_XPR(F_, IV_, X_, P_, false) WQ_MMT_LAUNCH_XPR(F_, IV_, X_, P_, X_)
#define WQ_MMT_LAUNCH_X(F_, IV_, X_) WQ_MMT_LAUNCH_XP(F_, IV_, X_, false) WQ_MMT_LAUNCH_XP(F_, IV_, X_, X_)
#define WQ_MMT_LAUNCH(F_, IV_) WQ_MMT_LAUNCH_X(F_, IV_, false) WQ_MMT_LAUNCH_X(F_, IV_, true)
  WQ_MMT_LAUNCH(4, 0) WQ_MMT_LAUNCH(4, 1) WQ_MMT_LAUNCH(4, 2) WQ_MMT_LAUNCH(4, 4)
  WQ_MMT_LAUNCH(2, 0) WQ_MMT_LAUNCH(2, 1) WQ_MMT_LAUNCH(2, 2) WQ_MMT_LAUNCH(2, 4)
  WQ_MMT_LAUNCH(5, 0) WQ_MMT_LAUNCH(5, 1) WQ_MMT_LAUNCH(5, 2) WQ_MMT_LAUNCH(5, 4)
#undef WQ_MMT_LAUNCH_X
#undef WQ_MMT_LAUNCH_XP
#undef WQ_MMT_LAUNCH_XPR
#undef WQ_MMT_LAUNCH_XPRH
#undef WQ_MMT_LAUNCH_XPRHD
#undef WQ_MMT_LAUNCH
  return WQ_OK;
}
