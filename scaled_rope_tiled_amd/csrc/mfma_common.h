// Device helpers shared by the bf16 matrix-core attention kernels (forward
// and backward): bf16 packing, RoPE rotation of 16-byte bf16 chunks, LDS
// operand reads and lane-pair reductions for v_mfma_f32_32x32x16_bf16 tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "srt_internal.h"

namespace srt {
namespace mc {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline uint32_t pack2(float a, float b) {
  // one v_cvt_pk_bf16_f32: both values rounded to nearest even
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a, b}, b2_t));
}

// Rotate the 4 pairs of a 16-byte bf16 chunk with 4 (cos, sin) table entries.
__device__ inline uint4 rotate_chunk(uint4 w, float4 t0, float4 t1) {
  const uint32_t in[4] = {w.x, w.y, w.z, w.w};
  const float c[4] = {t0.x, t0.z, t1.x, t1.z};
  const float s[4] = {t0.y, t0.w, t1.y, t1.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = bf_lo(in[i]), x1 = bf_hi(in[i]);
    o[i] = pack2(x0 * c[i] - x1 * s[i], x0 * s[i] + x1 * c[i]);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Half-split pairs: chunk w1 holds dims i..i+7 of the first half, w2 the same
// dims of the second half; pair (w1[e], w2[e]) turns by table entry i + e.
__device__ inline void rotate_chunk_pair(uint4& w1, uint4& w2, const float4 (&t)[4]) {
  const uint32_t a[4] = {w1.x, w1.y, w1.z, w1.w};
  const uint32_t b[4] = {w2.x, w2.y, w2.z, w2.w};
  uint32_t o1[4], o2[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // elements 2q, 2q+1 of each chunk: pairs i+2q (t[q].x, t[q].y) and i+2q+1 (t[q].z, t[q].w)
    const float a0 = bf_lo(a[q]), a1 = bf_hi(a[q]), b0 = bf_lo(b[q]), b1 = bf_hi(b[q]);
    o1[q] = pack2(a0 * t[q].x - b0 * t[q].y, a1 * t[q].z - b1 * t[q].w);
    o2[q] = pack2(a0 * t[q].y + b0 * t[q].x, a1 * t[q].w + b1 * t[q].z);
  }
  w1 = make_uint4(o1[0], o1[1], o1[2], o1[3]);
  w2 = make_uint4(o2[0], o2[1], o2[2], o2[3]);
}

__device__ inline bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

// LDS operands are addressed with 32-bit LDS byte addresses.  `opaque` hides a
// step's base address from the loop optimisers, so every read of the step is
// that one base register plus an immediate offset (no per-read arithmetic).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4_t lds_u4;
__device__ inline uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}
__device__ inline uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ inline bf16x8 lds_read16(uint32_t addr) { return __builtin_bit_cast(bf16x8, *(lds_u4*)(uintptr_t)addr); }
// gfx950 transposing LDS read: each lane fetches 8 bytes at its address, then
// within every 16 lanes, lane i receives element (i & 3) of the values fetched
// by lanes 4t + (i >> 2), t = 0..3.
__device__ inline i16x4 lds_read_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)addr);
}

// Raw buffer descriptor over `bytes` bytes from `base`: 32-bit byte offsets,
// and loads at or past `bytes` return zero without touching memory.  The
// size is made wave-uniform (readfirstlane) so the descriptor stays scalar.
constexpr int kRawBufferWord3 = 0x00020000;   // descriptor word 3 for raw 32-bit loads (gfx9 family)
__device__ inline __amdgpu_buffer_rsrc_t raw_buffer(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, __builtin_amdgcn_readfirstlane(bytes),
                                           kRawBufferWord3);
}
__device__ inline uint4 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(w.x, w.y, w.z, w.w);
}

// Lanes l and l ^ 32 hold the same query (different keys).  v_permlane32_swap
// of a value with itself leaves the lower half's values in the first result and
// the upper half's in the second, in every lane, so their max / sum combines
// the pair without a trip through LDS.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mc
}  // namespace srt
