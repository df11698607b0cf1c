// MX (OCP microscaling) element and scale encoders shared by the quantising
// kernels: the dynamic MXFP8 quantiser, the router's fused quantisation of x
// and GEMM1's epilogue.  Block rule (32 consecutive elements): shared
// exponent e = floor(log2(amax)) - 8 clamped to [-127, 127] (amax 0 -> -127),
// element = E4M3FN round-to-nearest-even of v / 2^e saturated to +-448, a
// value rounding to zero keeping its sign bit.  Integer-exact, no hardware
// convert, so codes are reproducible bit for bit.
#pragma once

#include "common.hpp"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// E4M3FN code of v (already divided by its block scale), RNE, saturating.
// Branch-free: both the subnormal code (grid 2^-9 below 2^-6) and the normal
// code are formed and one is selected.  Normal: E = floor(log2 a) in [-6, 8],
// m = rint(a * 2^(3-E)) in [8, 16]; code = ((E + 7) << 3) + (m - 8), where
// m = 16 carries into the exponent field by itself.  |v| >= 448 and NaN give
// +-448 (0x7e); a value rounding to zero keeps its sign bit.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fminf(__uint_as_float(bits & 0x7fffffffu), 448.f);  // (fminf(NaN, 448) = 448)
  const uint32_t sub = (uint32_t)rintf(a * 512.f);                     // 0..8 (8 = 2^-6 = code 0x08)
  const int E = max((int)(__float_as_uint(a) >> 23) - 127, -6);
  const float q = __uint_as_float((uint32_t)(127 + 3 - E) << 23) * a;  // a * 2^(3-E)
  const uint32_t code = min(((uint32_t)(E + 7) << 3) + ((uint32_t)rintf(q) - 8u), 0x7eu);
  return sign | (a < 0.015625f ? sub : code);
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
