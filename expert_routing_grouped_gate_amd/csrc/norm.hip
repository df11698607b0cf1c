// The step before the MoE layer: residual add + RMSNorm in one pass, with
// the outputs the layer takes.
//
// [Qwen3] "fused-operator optimisation": residual add, RMSNorm and dynamic
// MXFP8 quantisation are fused so that the intermediate results are not
// written and read back ("fused RMSNorm + MX quant"), and the norm before the
// MoE block returns its result in FP32 for the gate and in BF16 for the
// experts together with the updated residual ("fused RMSNorm + Cast").
// [Notes] section 2, "Add and RMSNorm": z = x + r, then
// y_i = z_i / sqrt(mean_j z_j^2 + eps) * w_i.
//
// One block of 256 threads per row; thread t holds the 16-byte chunks
// c = t + 256 j (8 elements each) in registers, so x and r are read once and
// every output is written once.  z = x + r in fp32 (exact for bf16 inputs);
// the sum of squares in fp32 in a fixed order (chunk order per thread, then a
// butterfly over the wave, then the four waves); 1/sqrt(mean + eps) in fp64
// once per row; y = z * rstd * w in fp32.  The MXFP8 output quantises that
// fp32 y per 32-element block (four consecutive threads) with the rule of
// moe_mx_quantize.
#include "common.hpp"
#include "launch.hpp"
#include "mxfmt.hpp"

namespace moe {

constexpr int kNormThreads = 256;

template <int NCH>
__global__ __launch_bounds__(kNormThreads) void add_rmsnorm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ res,
    const uint16_t* __restrict__ w, int H, float eps, float* __restrict__ yf,
    uint16_t* __restrict__ yb, uint16_t* __restrict__ rout, uint8_t* __restrict__ q,
    uint8_t* __restrict__ qs) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = H / 8;
  const size_t off = (size_t)blockIdx.x * H;
  float z[NCH][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + kNormThreads * j;
    if (c < nch) {
      const u32x4 xv = ld16(x + off + 8 * c);
      const u32x4 rv = res ? ld16(res + off + 8 * c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[j][2 * i] = bf16_to_f32(xv[i] & 0xffffu) + bf16_to_f32(rv[i] & 0xffffu);
        z[j][2 * i + 1] = bf16_to_f32(xv[i] >> 16) + bf16_to_f32(rv[i] >> 16);
      }
      if (rout) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(z[j][2 * i], z[j][2 * i + 1]);
        *reinterpret_cast<u32x4*>(rout + off + 8 * c) = o;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += z[j][i] * z[j][i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) z[j][i] = 0.f;
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) ss += __shfl_xor(ss, d, 64);
  __shared__ float part[kNormThreads / 64];
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  const float total = (part[0] + part[1]) + (part[2] + part[3]);
  const float rstd = (float)(1.0 / sqrt((double)total / (double)H + (double)eps));

#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + kNormThreads * j;
    const bool live = c < nch;  // H % 32 == 0: a 32-block's four threads agree
    float y[8];
    if (live) {
      const u32x4 wv = ld16(w + 8 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[2 * i] = z[j][2 * i] * rstd * bf16_to_f32(wv[i] & 0xffffu);
        y[2 * i + 1] = z[j][2 * i + 1] * rstd * bf16_to_f32(wv[i] >> 16);
      }
      if (yf) {
        float* p = yf + off + 8 * c;
        *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
        *reinterpret_cast<f32x4*>(p + 4) = f32x4{y[4], y[5], y[6], y[7]};
      }
      if (yb) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
        *reinterpret_cast<u32x4*>(yb + off + 8 * c) = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = 0.f;
    }
    if (q) {  // uniform: every thread of the block takes the shuffles
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int e = mx_exponent(amax);
      const float inv = exp2_neg(e);
      if (live) {
        u32x2 pk;
        pk.x = e4m3_pack4(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
        pk.y = e4m3_pack4(y[4] * inv, y[5] * inv, y[6] * inv, y[7] * inv);
        *reinterpret_cast<u32x2*>(q + off + 8 * c) = pk;
        if ((c & 3) == 0) qs[(size_t)blockIdx.x * (H / 32) + c / 4] = (uint8_t)(e + 127);
      }
    }
  }
}

template <int NCH>
static void launch_norm(const uint16_t* x, const uint16_t* res, const uint16_t* w, int T, int H,
                        float eps, float* yf, uint16_t* yb, uint16_t* rout, uint8_t* q,
                        uint8_t* qs, hipStream_t s) {
  hipLaunchKernelGGL(add_rmsnorm_kernel<NCH>, dim3(T), dim3(kNormThreads), 0, s, x, res, w, H,
                     eps, yf, yb, rout, q, qs);
}

// T >= 1, H % 32 == 0, H <= 16384 (checked by the caller).
int launch_add_rmsnorm(const uint16_t* x, const uint16_t* res, const uint16_t* w, int T, int H,
                       float eps, float* yf, uint16_t* yb, uint16_t* rout, uint8_t* q,
                       uint8_t* qs, hipStream_t s) {
  const int per = (H / 8 + kNormThreads - 1) / kNormThreads;  // chunks per thread
  if (per <= 1)
    launch_norm<1>(x, res, w, T, H, eps, yf, yb, rout, q, qs, s);
  else if (per <= 2)
    launch_norm<2>(x, res, w, T, H, eps, yf, yb, rout, q, qs, s);
  else if (per <= 4)
    launch_norm<4>(x, res, w, T, H, eps, yf, yb, rout, q, qs, s);
  else
    launch_norm<8>(x, res, w, T, H, eps, yf, yb, rout, q, qs, s);
  return launch_status();
}

}  // namespace moe
