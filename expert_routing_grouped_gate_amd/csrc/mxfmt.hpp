// MX (OCP microscaling) element and scale encoders shared by the quantising
// kernels: the dynamic MXFP8 quantiser, the router's fused quantisation of x
// and GEMM1's epilogue.  Block rule (32 consecutive elements): shared
// exponent e = floor(log2(amax)) - 8 clamped to [-127, 127] (amax 0 -> -127),
// element = E4M3FN round-to-nearest-even of v / 2^e saturated to +-448, a
// value rounding to zero keeping its sign bit.  Codes are a pure function of
// the fp32 input (no data-dependent rounding state), reproducible bit for bit.
#pragma once

#include "common.hpp"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// E4M3FN codes of four values already divided by their block scale: round
// to nearest even, saturating at +-448, NaN to +-448 with its sign, a value
// rounding to zero keeping its sign bit.  The hardware convert
// (v_cvt_pk_fp8_f32, OCP E4M3FN on gfx950) rounds to nearest even and keeps
// the sign of zero; clamping to +-448 first gives the saturation.  This equals
// an integer implementation of the rule on every fp32 input (an exhaustive
// check over all 2^32 bit patterns on gfx950).  Byte i = code of value i.
// The clamp works on the bits: the magnitude (an integer that orders like
// the float) is limited to 448's, which maps inf and NaN to 448 as well, and
// the sign is put back; no branch.
__device__ __forceinline__ float e4m3_clamp(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t mag = min(bits & 0x7fffffffu, 0x43e00000u);  // 0x43e00000 = 448.0f
  return __uint_as_float(mag | (bits & 0x80000000u));
}

__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), lo, true);
}

// Maximum of x over lanes l, l^16, l^32, l^48 (the four lanes that hold one
// row's 32-column block in the MFMA output layout), with the gfx950 row and
// half-wave swaps (VALU) instead of LDS-routed shuffles.  Every lane active.
__device__ __forceinline__ float max_lanes_16_32(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// SiLU(g) = g / (1 + e^-g) from the hardware exp2 and reciprocal (about one
// ulp each; the result is then quantised to E4M3, whose step is 2^-3
// relative).  Large negative g: e^-g overflows to inf and the result is -0.
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// floor(log2(amax)) - 8, clamped to [-127, 127]; amax zero or subnormal -> -127.
__device__ __forceinline__ int mx_exponent(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  if (ef == 0) return -127;
  const int e = ef - 127 - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as an fp32 (e in [-127, 127]; 2^127 is finite, 2^-127 is subnormal).
__device__ __forceinline__ float exp2_neg(int e) {
  const int p = -e;
  if (p >= -126) return __uint_as_float((uint32_t)(p + 127) << 23);
  return __uint_as_float(1u << (p + 149));  // subnormal powers of two
}

// -------------------------------------------------------- scaled MFMA -----
__device__ __forceinline__ f32x4 mfma_fp4_fp8(u32x4 a_fp4, i32x8 b_fp8, uint32_t sa, uint32_t sb,
                                              f32x4 c) {
  i32x8 a;
  a[0] = (int)a_fp4[0];
  a[1] = (int)a_fp4[1];
  a[2] = (int)a_fp4[2];
  a[3] = (int)a_fp4[3];
  a[4] = a[5] = a[6] = a[7] = 0;
  // A format 4 = E2M1, B format 0 = E4M3; scale byte 0 of each scale operand
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b_fp8, c, 4, 0, 0, (int)sa, 0, (int)sb);
}

// E4M3 operand of one lane: 16 bytes at p (k = 16g..) and 16 bytes at p + 64
// (k = 64 + 16g..), where p = row + k0 + 16g.
__device__ __forceinline__ i32x8 ld32_fp8(const uint8_t* p) {
  const u32x4 lo = ld16(p), hi = ld16(p + 64);
  i32x8 r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// Raw buffer descriptor over [p, p + bytes): loads address it as a uniform
// base (scalar registers) plus a 32-bit lane offset and a scalar offset.
// Word 3 = 0x00020000: the raw (untyped, stride 0) dword format on gfx9.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

}  // namespace moe
