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

// (a & m) | c in one instruction (the compiler splits it into two when both
// constants need the one constant-bus read a VOP3 instruction has here)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(c));
  return d;
}

// Codes of one dword as an exact f16 MFMA operand with no bias: the nibble
// is the mantissa of an f16 subnormal, so e in {0, 1, 4, 5} -> u * 2^-24 and
// e in {2, 3, 6, 7} -> 16 u * 2^-24 (nibble at mantissa bits 4-7).  The
// partner operand carries a factor 1/16 at e in {2, 3, 6, 7}, so every
// product is 2^-24 * (partner value) * u; the code offset 8 is removed after
// the MFMA as 8 * (sum of the partner values).
__device__ __forceinline__ f16x8_t dword_to_f16x8_sub(uint32_t w) {
  const uint32_t t = w >> 8;
  u32x4_t v;
  v.x = w & 0x000F000Fu;
  v.y = w & 0x00F000F0u;
  v.z = t & 0x000F000Fu;
  v.w = t & 0x00F000F0u;
  return bitcast<f16x8_t>(v);
}

// 8 codes of a dword as the bf16x8 MFMA operand (128 + u), k order e = 0..7:
// nibble pair (slot i, slot i + 4) under the magic exponent 0x4300 (128.0);
// value - 136 is the signed code
__device__ __forceinline__ bf16x8_t dword_to_bf16x8_biased(uint32_t w) {
  const uint32_t magic = 0x43004300u;
  u32x4_t v;
  v.x = and_or(w, 0x000F000Fu, magic);
  v.y = and_or(w >> 4, 0x000F000Fu, magic);
  v.z = and_or(w >> 8, 0x000F000Fu, magic);
  v.w = and_or(w >> 12, 0x000F000Fu, magic);
  return bitcast<bf16x8_t>(v);
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

// v of lane (lane ^ m) for m = 1, 2, 4, 8, 16, 32 (a compile-time constant
// after unrolling) without the LDS crossbar: DPP quad permutations for
// 1 and 2, a half-row mirror then a quad reversal for 4 (7 ^ 3), a row
// rotation by 8 for 8, and the gfx950 row-pair / half-wave swaps for 16
// and 32.  Same values as shfl_xor, so a butterfly built on it adds in the
// same order.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor(float v, int m, int lane) {
  if (m == 1) return dpp_f32<0xB1>(v);                  // quad_perm [1,0,3,2]
  if (m == 2) return dpp_f32<0x4E>(v);                  // quad_perm [2,3,0,1]
  if (m == 4) return dpp_f32<0x1B>(dpp_f32<0x141>(v));  // row_half_mirror, quad_perm [3,2,1,0]
  if (m == 8) return dpp_f32<0x128>(v);                 // row_ror:8
  const unsigned u = __float_as_uint(v);
  if (m == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  }
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((lane & 32) ? r[0] : r[1]);
}

// Workgroup barrier that waits for LDS traffic only: global loads stay in
// flight across it (__syncthreads would also drain every outstanding global
// load of the wave).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ u32x4_t load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

}  // namespace i4d
