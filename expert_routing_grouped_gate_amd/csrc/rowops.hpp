// Per-row building blocks shared by the combine (S7), the residual add +
// RMSNorm before the layer, and their fusion: the same arithmetic in the same
// order in every kernel that uses them, so a fused kernel reproduces the
// separate ones bit for bit.
#pragma once

#include "common.hpp"
#include "mxfmt.hpp"

namespace moe {

// finalize_routing for NCH chunks of 8 consecutive hidden elements of one
// token (chunk j at element c0 + 2048 j; chunks at or past H are skipped and
// return zero) ([Qwen3] "GMM enablement and routing optimisation": expert
// outputs back in token order, summed with the top-k weights; [Hy3] section
// 1.1: plus the shared expert's row): per element, fp32 accumulation in slot
// order, the shared row added last, rounded to bf16.  The shared row is
// loaded first and the rows of up to 8 slots are loaded for every chunk
// before any of them is accumulated, so a thread has all its loads in flight
// at once.  pos >= R (outside the rows of y) or < 0 counts as a dropped pair.
template <int NCH>
__device__ __forceinline__ void combine_chunks(const uint16_t* __restrict__ y,
                                               const int32_t* __restrict__ pp,
                                               const float* __restrict__ wt,
                                               const uint16_t* __restrict__ shared_row, int k,
                                               int R, int H, int c0, u32x4 (&res)[NCH]) {
  float acc[NCH][8];
  u32x4 sv[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
    const int c = c0 + 2048 * j;
    sv[j] = (shared_row != nullptr && c < H) ? ld16(shared_row + c) : u32x4{0u, 0u, 0u, 0u};
  }
  for (int j0 = 0; j0 < k; j0 += 8) {
    int pos[8];
    u32x4 v[NCH][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      pos[u] = j0 + u < k ? pp[j0 + u] : -1;
      if (pos[u] >= R) pos[u] = -1;
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = c0 + 2048 * j;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[j][u] = (pos[u] >= 0 && c < H) ? ld16(y + (size_t)pos[u] * H + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (pos[u] < 0) continue;
      const float wj = wt[j0 + u];
#pragma unroll
      for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[j][2 * q] = fmaf(wj, bf16_to_f32(v[j][u][q] & 0xffffu), acc[j][2 * q]);
          acc[j][2 * q + 1] = fmaf(wj, bf16_to_f32(v[j][u][q] >> 16), acc[j][2 * q + 1]);
        }
    }
  }
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = c0 + 2048 * j;
    if (shared_row != nullptr && c < H) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[j][2 * q] += bf16_to_f32(sv[j][q] & 0xffffu);
        acc[j][2 * q + 1] += bf16_to_f32(sv[j][q] >> 16);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) res[j][q] = pack_bf16x2(acc[j][2 * q], acc[j][2 * q + 1]);
  }
}

// Outputs of the residual add + RMSNorm of one row (each may be null; q and
// qs together).
struct NormOut {
  float* yf;       // [T, H] fp32 y
  uint16_t* yb;    // [T, H] bf16 y
  uint16_t* rout;  // [T, H] bf16 z (the updated residual)
  uint8_t* q;      // [T, H] E4M3 codes of y
  uint8_t* qs;     // [T, H/32] E8M0 scales
};

constexpr int kNormThreads = 256;

// Residual add + RMSNorm of row `row` by a block of kNormThreads threads
// ([Notes] section 2, "Add and RMSNorm": z = x + r, y_i = z_i /
// sqrt(mean_j z_j^2 + eps) * w_i).  Thread t holds the 16-byte chunks
// c = t + 256 j (8 elements each, element offset 8 c = 8 t + 2048 j) in
// registers: xv[j] the bf16 x of its chunk j, rv[j] and wv[j] its residual
// and weight (norm_row_loads); z = x + r in fp32 (exact for bf16 inputs);
// the sum of squares in fp32 in a fixed order (chunk order per thread, a
// butterfly over the wave, then the four waves); 1/sqrt(mean + eps) in fp64
// once per row; y = z * rstd * w in fp32; the MXFP8 output quantises that y
// per 32-element block (four consecutive threads) with the rule of
// moe_mx_quantize.  H % 32 == 0; NCH >= ceil(H / 8 / 256).  Contains one
// block barrier: every thread of the block must call it.

// Chunk j of thread t clamped to the row: chunks past the row load the
// row's last chunk, which is not used, so that the loads need no branches.
__device__ __forceinline__ int norm_chunk(int j, int nch) {
  return min((int)threadIdx.x + kNormThreads * j, nch - 1);
}

// The residual (zeros without one) and weight chunks of this thread for row
// `row`.  Issued by the kernels before their other loads' results are used:
// outputs never overlap inputs, and otherwise the compiler would keep these
// loads behind the stores of the x chunks.
template <int NCH>
__device__ __forceinline__ void norm_row_loads(const uint16_t* __restrict__ res,
                                               const uint16_t* __restrict__ w, int H, size_t row,
                                               u32x4 (&rv)[NCH], u32x4 (&wv)[NCH]) {
  const int nch = H / 8;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    wv[j] = ld16(w + 8 * norm_chunk(j, nch));
    rv[j] = u32x4{0u, 0u, 0u, 0u};
  }
  if (res != nullptr) {
    const uint16_t* r = res + row * (size_t)H;
#pragma unroll
    for (int j = 0; j < NCH; ++j) rv[j] = ld16(r + 8 * norm_chunk(j, nch));
  }
}

template <int NCH>
__device__ __forceinline__ void norm_row(const u32x4 (&xv)[NCH], const u32x4 (&rv)[NCH],
                                         const u32x4 (&wv)[NCH], int H, float eps, size_t row,
                                         const NormOut& o) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = H / 8;
  const size_t off = row * (size_t)H;
  float z[NCH][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + kNormThreads * j;
    if (c < nch) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[j][2 * i] = bf16_to_f32(xv[j][i] & 0xffffu) + bf16_to_f32(rv[j][i] & 0xffffu);
        z[j][2 * i + 1] = bf16_to_f32(xv[j][i] >> 16) + bf16_to_f32(rv[j][i] >> 16);
      }
      if (o.rout) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(z[j][2 * i], z[j][2 * i + 1]);
        *reinterpret_cast<u32x4*>(o.rout + off + 8 * c) = v;
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
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[2 * i] = z[j][2 * i] * rstd * bf16_to_f32(wv[j][i] & 0xffffu);
        y[2 * i + 1] = z[j][2 * i + 1] * rstd * bf16_to_f32(wv[j][i] >> 16);
      }
      if (o.yf) {
        float* p = o.yf + off + 8 * c;
        *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
        *reinterpret_cast<f32x4*>(p + 4) = f32x4{y[4], y[5], y[6], y[7]};
      }
      if (o.yb) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
        *reinterpret_cast<u32x4*>(o.yb + off + 8 * c) = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = 0.f;
    }
    if (o.q) {  // uniform: every thread of the block takes the shuffles
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
        *reinterpret_cast<u32x2*>(o.q + off + 8 * c) = pk;
        if ((c & 3) == 0) o.qs[row * (size_t)(H / 32) + c / 4] = (uint8_t)(e + 127);
      }
    }
  }
}

}  // namespace moe
