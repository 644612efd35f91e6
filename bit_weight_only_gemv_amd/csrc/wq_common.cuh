// Device-side building blocks shared by the gfx950 kernels: buffer
// resources, FP16 vector types, the W4 nibble and W2 codebook decoders, and
// wave-level reductions.  Written for CDNA (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wqd {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGroup = 32;

// ---------------------------------------------------------------- buffers
// Raw buffer resource (gfx9 descriptor, dword 3 = 0x00020000).  Loads beyond
// `bytes` return zero, so ragged tails never fault.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint32_t clamp_bytes(uint64_t b) {
  return b > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)b;
}

__device__ __forceinline__ u4v ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u2 ld64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint8_t ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// W4P: zero point of group g from the packed bytes of its row (group 2m in
// bits 3:0 of byte m, group 2m + 1 in bits 7:4), as a float (exact integer).
__device__ __forceinline__ float packed_zero(uint32_t byte, uint32_t g) {
  return (float)((byte >> (4u * (g & 1u))) & 0x0Fu);
}

__device__ __forceinline__ float h2f(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t f2h(float f) {   // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// ------------------------------------------------------------- W4 decoder
// A 32-bit word w of a W4 group holds bytes 4j..4j+3 (j = word index 0..3);
// byte k carries code k in its low nibble and code k+16 in its high nibble.
// Masking two nibbles into the two FP16 halves of a register yields FP16
// subnormals: bits 3:0 hold q * 2^-24 and bits 7:4 hold 16 q * 2^-24, exactly.
// gfx950's v_dot2 keeps FP16 subnormal inputs, so these feed the dot product
// directly and the 2^-24 (and 1/16) come back as one float scale per group:
//   lo0 = w      & 0x000F000F -> 2^-24 {q[4j],    q[4j+2]}
//   hi0 = w      & 0x00F000F0 -> 2^-20 {q[4j+16], q[4j+18]}
//   lo1 = w >> 8 & 0x000F000F -> 2^-24 {q[4j+1],  q[4j+3]}
//   hi1 = w >> 8 & 0x00F000F0 -> 2^-20 {q[4j+17], q[4j+19]}
__device__ __forceinline__ void w4_word_sub(uint32_t w, uint32_t& lo0, uint32_t& hi0,
                                            uint32_t& lo1, uint32_t& hi1) {
  const uint32_t w8 = w >> 8;
  lo0 = w & 0x000F000Fu;
  hi0 = w & 0x00F000F0u;
  lo1 = w8 & 0x000F000Fu;
  hi1 = w8 & 0x00F000F0u;
}
// The same four pairs as exact FP16 integers 1024 + q / 1024 + 16 q (the low
// nibble OR-ed into the mantissa of 1024.0 = 0x6400); used where a normal
// FP16 value is needed (device dequantization).
__device__ __forceinline__ void w4_word_magic(uint32_t w, uint32_t& lo0, uint32_t& hi0,
                                              uint32_t& lo1, uint32_t& hi1) {
  w4_word_sub(w, lo0, hi0, lo1, hi1);
  lo0 |= 0x64006400u;
  hi0 |= 0x64006400u;
  lo1 |= 0x64006400u;
  hi1 |= 0x64006400u;
}

// ------------------------------------------------------------- W2 decoder
// FP16 codebook {-1.52, -0.45, +0.45, +1.52} = {0xBE14, 0xB733, 0x3733, 0x3E14},
// split into a table of low bytes and a table of high bytes so that one byte
// permute turns two 2-bit codes into two FP16 centroids:
//   sel = q_a | (q_a + 4) << 8 | q_b << 16 | (q_b + 4) << 24
//   perm(kHiBytes, kLoBytes, sel) = C[q_a] | C[q_b] << 16
constexpr uint32_t kLoBytes = 0x14333314u;   // bytes {0x14, 0x33, 0x33, 0x14}
constexpr uint32_t kHiBytes = 0x3E37B7BEu;   // bytes {0xBE, 0xB7, 0x37, 0x3E}

// t holds two codes at bits 1:0 and 17:16 (everything else zero).
__device__ __forceinline__ uint32_t w2_centroid_pair(uint32_t t) {
  const uint32_t sel = t * 0x0101u + 0x04000400u;   // t < 2^18: one v_mad_u32_u24
  return __builtin_amdgcn_perm(kHiBytes, kLoBytes, sel);
}

// Workgroup barrier that only waits for this wave's LDS traffic (HIP's
// __syncthreads also waits for every outstanding global load, which would
// serialize a prologue behind the weight stream it is meant to overlap).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Orders one wave's own LDS traffic: a wave's LDS operations complete in
// order, and this keeps the compiler from moving them across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------ reductions
// Sum over each row of 16 lanes with DPP; every lane of the row ends up with
// the row's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov<0x124>(v);   // row_ror:4
  v += dpp_mov<0x128>(v);   // row_ror:8
  return v;
}

}  // namespace wqd
