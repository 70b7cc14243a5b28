// device_common.h - small device helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i4d {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, f);
}

// nibble pairs (slot i, slot i+4) of a packed dword as bf16 (128 + u): the
// magic-exponent decode; value - 136 is the signed code.
__device__ __forceinline__ uint32_t nib_pair_bf16(uint32_t w, int i) {
  return ((w >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
}

// 8 codes of a dword as the bf16x8 MFMA operand (128 + u), k order e = 0..7
__device__ __forceinline__ bf16x8_t dword_to_bf16x8_biased(uint32_t w) {
  u32x4_t v;
  v.x = nib_pair_bf16(w, 0);
  v.y = nib_pair_bf16(w, 1);
  v.z = nib_pair_bf16(w, 2);
  v.w = nib_pair_bf16(w, 3);
  return bitcast<bf16x8_t>(v);
}

// 8 codes of a dword as exact signed fp16 (u - 8): (1024 + u) - 1032
__device__ __forceinline__ f16x8_t dword_to_f16x8_signed(uint32_t w) {
  const f16x2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  f16x2_t p0 = bitcast<f16x2_t>(((w >> 0) & 0x000F000Fu) | 0x64006400u) - off;
  f16x2_t p1 = bitcast<f16x2_t>(((w >> 4) & 0x000F000Fu) | 0x64006400u) - off;
  f16x2_t p2 = bitcast<f16x2_t>(((w >> 8) & 0x000F000Fu) | 0x64006400u) - off;
  f16x2_t p3 = bitcast<f16x2_t>(((w >> 12) & 0x000F000Fu) | 0x64006400u) - off;
  u32x4_t v;
  v.x = bitcast<uint32_t>(p0);
  v.y = bitcast<uint32_t>(p1);
  v.z = bitcast<uint32_t>(p2);
  v.w = bitcast<uint32_t>(p3);
  return bitcast<f16x8_t>(v);
}

// Same result with fewer instructions: the fp16 mantissa holds a nibble at
// bits 0-3 (value 1024 + u) or at bits 4-7 (value 1024 + 16u), so one shift
// and four v_and_or give all eight codes; (1024 + 16u)/16 - 72 = u - 8 is
// exact in one packed FMA.
__device__ __forceinline__ f16x8_t dword_to_f16x8_signed_fast(uint32_t w) {
  const f16x2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2_t off72 = {(_Float16)72.0f, (_Float16)72.0f};
  const uint32_t t = w >> 8;
  f16x2_t p0 = bitcast<f16x2_t>((w & 0x000F000Fu) | 0x64006400u) - off;
  f16x2_t p1 = bitcast<f16x2_t>((w & 0x00F000F0u) | 0x64006400u) * sixteenth - off72;
  f16x2_t p2 = bitcast<f16x2_t>((t & 0x000F000Fu) | 0x64006400u) - off;
  f16x2_t p3 = bitcast<f16x2_t>((t & 0x00F000F0u) | 0x64006400u) * sixteenth - off72;
  u32x4_t v;
  v.x = bitcast<uint32_t>(p0);
  v.y = bitcast<uint32_t>(p1);
  v.z = bitcast<uint32_t>(p2);
  v.w = bitcast<uint32_t>(p3);
  return bitcast<f16x8_t>(v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)bitcast<_Float16>(b);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, 64);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ u32x4_t load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

}  // namespace i4d
