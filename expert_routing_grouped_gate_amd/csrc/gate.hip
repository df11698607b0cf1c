// S1 router logits and S2 gate top-k.
//
// [Qwen3] "fused RMSNorm + Cast": the gate consumes fp32 activations, so the
// router product is accumulated in fp32 from exactly upcast bf16 x.
// [Qwen3] "GMM enablement and routing optimisation": top-k + softmax fused in
// one operator.  [Hy3] section 1.3: sigmoid router with a learnable
// correction bias, renormalised top-k weights scaled by routed_scaling_factor,
// eps; section 5.1: the bias is added after the sigmoid and only steers
// selection.
#include "common.hpp"
#include "launch.hpp"
#include "mxfmt.hpp"

#include <type_traits>

namespace moe {

// ---------------------------------------------------------------- S1 ------
// Both router kernels compute x . w on bf16 MFMA exactly: each fp32 router
// weight is split into three bf16 terms, w = hi + mid + lo (hi and mid are
// truncations, lo is the exact remainder: 8 + 8 + 8 significand bits), so
// every product of the bf16 x with a term is exact in fp32 and the MFMA
// accumulates the three products in fp32.
__device__ __forceinline__ void split3_bf16(const float* w8, u32x4& hi, u32x4& mid, u32x4& lo) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t h2 = 0, m2 = 0, l2 = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float w = w8[2 * q + j];
      const uint32_t hb = __float_as_uint(w) & 0xffff0000u;   // truncation: top 8 bits
      const float r1 = w - __uint_as_float(hb);                  // exact
      const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
      const float r2 = r1 - __uint_as_float(mb);                 // exact, <= 8 bits
      const uint32_t lb = f32_to_bf16(r2);                        // exact
      h2 |= (hb >> 16) << (16 * j);
      m2 |= (mb >> 16) << (16 * j);
      l2 |= lb << (16 * j);
    }
    hi[q] = h2;
    mid[q] = m2;
    lo[q] = l2;
  }
}

// Few tokens (decode): split over H.  A wave computes the partial logits of
// 16 tokens x 16 experts over one 256-wide slice of H (8 K-steps, all loads
// issued at once: one memory round trip) and stores them to
// partial[slice][t][e]; the slices are summed in slice order afterwards
// (router_reduce, or the fused gate), so the result is deterministic.
// Grid (ceil(E/16), H/256, ceil(T/16)) of one-wave blocks (the 2 MB of Wr is
// spread over as many CUs as possible), block b: experts 16b ...  With
// xq != nullptr the waves also write the MXFP8
// quantisation of their x slice (each MX block of 32 is held by the 4 lanes
// of one token; the expert groups of a slice split its steps), so the W4A8
// path needs no separate quantiser launch.  With done != nullptr, block 0
// zeroes the counter the decode gate's blocks count themselves on (the gate
// runs after this kernel on the same stream, so it always starts at zero).
constexpr int RP_HS = 256;

// Many tokens: the MFMA router splits K over ks <= 8 blocks per output tile
// while that keeps the grid within 2048 blocks, ks a power of two dividing
// the H/32 K-steps; the ks partial tiles are summed in order by
// router_reduce, or inside the gate when the layer routes.
constexpr int RM_TT = 128, RM_TE = 64;

static int router_ksplit(int T, int H, int E) {
  const long long tiles = (long long)((T + RM_TT - 1) / RM_TT) * ((E + RM_TE - 1) / RM_TE);
  int ks = 1;
  while (ks < 8 && tiles * ks * 2 <= 2048 && (H / 32) % (ks * 2) == 0) ks *= 2;
  return ks;
}

size_t router_workspace_bytes(int T, int H, int E) {
  if (T <= 64) return (size_t)(H / RP_HS) * (size_t)T * (size_t)E * sizeof(float);
  const int ks = router_ksplit(T, H, E);
  return ks > 1 ? (size_t)ks * (size_t)T * (size_t)E * sizeof(float) : 0;
}

__global__ __launch_bounds__(64) void router_partial(const uint16_t* __restrict__ x,
                                                      const float* __restrict__ wr, int T, int H,
                                                      int E, float* __restrict__ partial,
                                                      uint8_t* __restrict__ xq,
                                                      uint8_t* __restrict__ xq_scales,
                                                      int32_t* __restrict__ done) {
  const int lane = threadIdx.x & 63;
  const int eg = blockIdx.x;
  const int e0 = eg * 16;
  if (done != nullptr && lane == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    *done = 0;
  if (e0 >= E) return;  // wave-uniform; the kernel has no barriers
  const int sl = blockIdx.y, h0 = sl * RP_HS, t0 = blockIdx.z * 16;
  const int fr = lane & 15, fc = lane >> 4;
  const int t = min(t0 + fr, T - 1);  // rows past T reuse a valid row
  const int e = min(e0 + fr, E - 1);
  const uint16_t* xp = x + (size_t)t * H + h0 + fc * 8;
  const float* wp = wr + (size_t)e * H + h0 + fc * 8;
  u32x4 xa[8];
  float4 wa[8][2];
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    xa[st] = ld16(xp + st * 32);
    wa[st][0] = *reinterpret_cast<const float4*>(wp + st * 32);
    wa[st][1] = *reinterpret_cast<const float4*>(wp + st * 32 + 4);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first use
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const float w8[8] = {wa[st][0].x, wa[st][0].y, wa[st][0].z, wa[st][0].w,
                         wa[st][1].x, wa[st][1].y, wa[st][1].z, wa[st][1].w};
    u32x4 h, m, l;
    split3_bf16(w8, h, m, l);
    acc = mfma16x16x32(xa[st], h, acc);
    acc = mfma16x16x32(xa[st], m, acc);
    acc = mfma16x16x32(xa[st], l, acc);
  }
  // D[m][n]: lane holds expert e0 + fr, tokens t0 + 4*fc + i
  if (e0 + fr < E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = t0 + 4 * fc + i;
      if (tt < T) partial[((size_t)sl * T + tt) * E + e0 + fr] = acc[i];
    }
  }
  if (xq != nullptr) {
    // lane (fr, fc) holds x[t][h0 + 32 st + 8 fc .. +8]: lanes fr, fr+16,
    // fr+32, fr+48 together hold one MX block of token t per step.  The
    // expert groups of a slice share its 8 steps (group g quantises the
    // steps st with st % groups == g % groups).
    const int ngroups = (E + 15) / 16;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st % ngroups != eg % ngroups) continue;  // wave-uniform
      float f[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = bf16_to_f32(xa[st][q] & 0xffffu);
        f[2 * q + 1] = bf16_to_f32(xa[st][q] >> 16);
      }
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = max_lanes_16_32(amax);
      const int ex = mx_exponent(amax);
      const float inv = exp2_neg(ex);
      const uint32_t lo = e4m3_pack4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
      const uint32_t hi = e4m3_pack4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
      if (t0 + fr < T) {
        const int col = h0 + 32 * st + 8 * fc;
        *reinterpret_cast<u32x2*>(xq + (size_t)(t0 + fr) * H + col) = u32x2{lo, hi};
        if (fc == 0) xq_scales[(size_t)(t0 + fr) * (H / 32) + col / 32] = (uint8_t)(ex + 127);
      }
    }
  }
}

// Sum of the S slice partials of one logit, in slice order; the loads of 8
// slices are issued together so that S slices cost S/8 memory round trips.
__device__ __forceinline__ float sum_slices(const float* __restrict__ p, int S, size_t stride) {
  float v = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) q[u] = s0 + u < S ? p[(size_t)(s0 + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) v = (s0 + u == 0) ? q[u] : v + q[u];
  }
  return v;
}

// logits[t][e] = sum over slices, in slice order.
__global__ __launch_bounds__(256) void router_reduce(const float* __restrict__ partial, int S,
                                                     int T, int E, float* __restrict__ logits) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * E) return;
  logits[i] = sum_slices(partial + i, S, (size_t)T * E);
}

// Many tokens (prefill): block tile 128 tokens x 64 experts, stages of KS
// K-steps of 32 in double-buffered LDS (the split is done once per block and
// stage, by the loading thread, and serves all 128 tokens); wave w owns
// tokens 32w..32w+31 of the tile (two 16-token fragments) and all 64 experts
// (four 16-expert groups x three parts: 24 MFMAs per K step).  Each
// accumulator takes its K-steps in order, the three parts of a step in the
// order hi, mid, lo, whatever KS is.  Block z of gridDim.z covers the z-th
// 1/gridDim.z of K and writes its partial tile to logits + z*T*E.  With
// xq != nullptr (W4A8 layers) blocks also write the MXFP8 codes of the x
// slice they load, so that no separate quantiser reads x again: the first
// expert tile's blocks the tile's first 64 rows, the second's the other 64
// (the first's all 128 when there is one expert tile), so that every
// element is quantised once over the K split.  A 32-column block of one row
// is the four loading threads of that row; the arithmetic is
// mx_quant_kernel's.

template <int KS>
__global__ __launch_bounds__(256) void router_logits_mfma(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr, int T,
                                                          int H, int E,
                                                          float* __restrict__ logits,
                                                          uint8_t* __restrict__ xq,
                                                          uint8_t* __restrict__ xq_scales) {
  __shared__ u32x4 xs[2][KS][RM_TT * 4];
  __shared__ u32x4 ws[2][KS][3][RM_TE * 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RM_TT, e0 = blockIdx.y * RM_TE;
  const int nk = H / (32 * KS) / (int)gridDim.z, kbeg = (int)blockIdx.z * nk * 32 * KS;
  logits += (size_t)blockIdx.z * T * E;
  // loaders: thread -> x rows tid/4 and 64 + tid/4, wr row (expert) tid/4;
  // 16-byte chunk tid%4 of each 32 columns of the stage (rows past T or E
  // reuse a valid row; their results are not stored)
  const int lrow = tid >> 2, lch = tid & 3;
  const uint16_t* xp0 = x + (size_t)min(t0 + lrow, T - 1) * H + kbeg + lch * 8;
  const uint16_t* xp1 = x + (size_t)min(t0 + 64 + lrow, T - 1) * H + kbeg + lch * 8;
  const float* wp = wr + (size_t)min(e0 + lrow, E - 1) * H + kbeg + lch * 8;
  struct Regs {
    u32x4 xa[KS], xb[KS];
    float w[KS][8];
  };
  // two register sets: stage k+2 is loaded while stage k computes and stage
  // k+1 waits to be split and stored into the other LDS buffer
  Regs r0, r1;
  auto gload = [&](Regs& r, int k0) {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int k = k0 + 32 * j;
      r.xa[j] = ld16(xp0 + k);
      r.xb[j] = ld16(xp1 + k);
      const float4 a = *reinterpret_cast<const float4*>(wp + k);
      const float4 b = *reinterpret_cast<const float4*>(wp + k + 4);
      r.w[j][0] = a.x; r.w[j][1] = a.y; r.w[j][2] = a.z; r.w[j][3] = a.w;
      r.w[j][4] = b.x; r.w[j][5] = b.y; r.w[j][6] = b.z; r.w[j][7] = b.w;
    }
  };
  // block-uniform: which of the tile's row halves this block quantises
  const bool quant_a = xq != nullptr && blockIdx.y == 0;
  const bool quant_b = xq != nullptr && blockIdx.y == (gridDim.y > 1 ? 1u : 0u);
  // 8 consecutive elements of x row `row` at column `col`: the four threads
  // of the row's 32-column block share one scale
  auto quant8 = [&](const u32x4 v, int row, int col) {
    float f[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = bf16_to_f32(v[q] & 0xffffu);
      f[2 * q + 1] = bf16_to_f32(v[q] >> 16);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    // the maximum over the quad (lanes xor 1, xor 2) by DPP: no LDS traffic
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0xB1, 0xF, 0xF, true)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(amax), 0x4E, 0xF, 0xF, true)));
    const int e = mx_exponent(amax);
    const float inv = exp2_neg(e);
    const uint32_t lo = e4m3_pack4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
    const uint32_t hi = e4m3_pack4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
    if (row < T) {
      *reinterpret_cast<u32x2*>(xq + (size_t)row * H + col) = u32x2{lo, hi};
      if (lch == 0) xq_scales[(size_t)row * (H / 32) + col / 32] = (uint8_t)(e + 127);
    }
  };
  auto lstore = [&](const Regs& r, int buf, int k0) {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int col = kbeg + k0 + 32 * j + lch * 8;
      if (quant_a) quant8(r.xa[j], t0 + lrow, col);
      if (quant_b) quant8(r.xb[j], t0 + 64 + lrow, col);
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      xs[buf][j][lrow * 4 + lch] = r.xa[j];
      xs[buf][j][(64 + lrow) * 4 + lch] = r.xb[j];
      u32x4 h, m, l;
      split3_bf16(r.w[j], h, m, l);
      ws[buf][j][0][lrow * 4 + lch] = h;
      ws[buf][j][1][lrow * 4 + lch] = m;
      ws[buf][j][2][lrow * 4 + lch] = l;
    }
  };
  f32x4 acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[mi][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fc = lane >> 4;
  auto compute = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const u32x4 a0 = xs[buf][j][(32 * wave + fr) * 4 + fc];
      const u32x4 a1 = xs[buf][j][(32 * wave + 16 + fr) * 4 + fc];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) {
          const u32x4 b = ws[buf][j][sp][(16 * g + fr) * 4 + fc];
          acc[0][g] = mfma16x16x32(a0, b, acc[0][g]);
          acc[1][g] = mfma16x16x32(a1, b, acc[1][g]);
        }
    }
  };
  constexpr int KW = 32 * KS;  // columns per stage
  gload(r0, 0);
  if (nk > 1) gload(r1, KW);
  lstore(r0, 0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    if (kt + 2 < nk) gload(r0, (kt + 2) * KW);
    compute(0);
    if (kt + 1 < nk) lstore(r1, 1, (kt + 1) * KW);
    __syncthreads();
    if (kt + 1 >= nk) break;
    if (kt + 3 < nk) gload(r1, (kt + 3) * KW);
    compute(1);
    if (kt + 2 < nk) lstore(r0, 0, (kt + 2) * KW);
    __syncthreads();
  }
  // D[m][n]: lane holds expert 16*g + (lane & 15), tokens 16*mi + 4*(lane>>4) + i
  // of the wave's 32
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int e = e0 + 16 * g + fr;
    if (e >= E) continue;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 32 * wave + 16 * mi + 4 * fc + i;
        if (t < T) logits[(size_t)t * E + e] = acc[mi][g][i];
      }
  }
}

// ------------------------------------------------ S1, fp32 hidden states ---
// The gate's input is fp32 ([Qwen3] "fused RMSNorm + Cast": the norm before
// the MoE block hands the gate an FP32 copy of the hidden states).  Block
// (token tile, expert tile, 256-column slice s of H): 64 tokens x 64 experts,
// partial[s][t][e] = sum over the slice of x[t][h] * Wr[e][h] with fp64
// accumulation (each product of two fp32 values is exact in fp64), rounded to
// fp32 once; router_reduce then sums the slices in order.  Operands are staged
// in LDS transposed (k-major), so a thread's 4 tokens and 4 experts at one k
// are two 16-byte reads; thread (ty, tx) owns tokens 4 ty.. and experts 4 tx...
constexpr int RF_T = 64, RF_E = 64, RF_K = 64;

__global__ __launch_bounds__(256) void router_partial_f32(const float* __restrict__ x,
                                                          const float* __restrict__ wr, int T,
                                                          int H, int E,
                                                          float* __restrict__ partial) {
  __shared__ float xs[RF_K][RF_T];
  __shared__ float ws[RF_K][RF_E];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RF_T, e0 = blockIdx.y * RF_E, h0 = blockIdx.z * RP_HS;
  const int ty = tid >> 4, tx = tid & 15;
  // loader: row (token or expert) tid / 4, 16 consecutive k at 16 * (tid % 4)
  const int lr = tid >> 2, lk = 16 * (tid & 3);
  const float* xrow = x + (size_t)min(t0 + lr, T - 1) * H + h0 + lk;  // rows past T reuse a valid row
  const float* wrow = wr + (size_t)min(e0 + lr, E - 1) * H + h0 + lk;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  for (int kc = 0; kc < RP_HS; kc += RF_K) {
    f32x4 xv[4], wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xv[q] = *reinterpret_cast<const f32x4*>(xrow + kc + 4 * q);
      wv[q] = *reinterpret_cast<const f32x4*>(wrow + kc + 4 * q);
    }
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xs[lk + 4 * q + i][lr] = xv[q][i];
        ws[lk + 4 * q + i][lr] = wv[q][i];
      }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < RF_K; ++k) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&xs[k][4 * ty]);
      const f32x4 b = *reinterpret_cast<const f32x4*>(&ws[k][4 * tx]);
      double bd[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bd[j] = (double)b[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double ad = (double)a[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fma(ad, bd[j], acc[i][j]);
      }
    }
  }
  float* out = partial + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * ty + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 4 * tx + j;
      if (e < E) out[(size_t)t * E + e] = (float)acc[i][j];
    }
  }
}

size_t router_f32_workspace_bytes(int T, int H, int E) {
  return (size_t)(H / RP_HS) * (size_t)T * (size_t)E * sizeof(float);
}

int launch_router_logits_f32(const float* x, const float* wr, int T, int H, int E, float* logits,
                             float* ws, hipStream_t s) {
  hipLaunchKernelGGL(router_partial_f32, dim3((T + RF_T - 1) / RF_T, (E + RF_E - 1) / RF_E, H / RP_HS),
                     dim3(256), 0, s, x, wr, T, H, E, ws);
  hipLaunchKernelGGL(router_reduce, dim3((T * E + 255) / 256), dim3(256), 0, s, ws, H / RP_HS, T,
                     E, logits);
  return launch_status();
}

int launch_router_partial(const uint16_t* x, const float* wr, int T, int H, int E,
                          float* partial, uint8_t* xq, uint8_t* xq_scales, int32_t* done,
                          hipStream_t s) {
  hipLaunchKernelGGL(router_partial, dim3((E + 15) / 16, H / RP_HS, (T + 15) / 16), dim3(64), 0,
                     s, x, wr, T, H, E, partial, xq, xq_scales, done);
  return launch_status();
}

// The partial-sum kernels of S1: returns the number S of slice partials
// written to ws ([S, T, E], summed in slice order afterwards), or 0 when the
// logits were written directly.  With xq != nullptr they also write the
// MXFP8 codes and scales of x.
static int launch_router_slices(const uint16_t* x, const float* wr, int T, int H, int E,
                                float* logits, float* ws, uint8_t* xq, uint8_t* xq_scales,
                                hipStream_t s) {
  if (T <= 64) {
    launch_router_partial(x, wr, T, H, E, ws, xq, xq_scales, nullptr, s);
    return H / RP_HS;
  }
  const int ks = router_ksplit(T, H, E);
  const dim3 grid((T + RM_TT - 1) / RM_TT, (E + RM_TE - 1) / RM_TE, ks);
  float* dst = ks > 1 ? ws : logits;
  // two 32-column steps per stage when every block's K range holds an even
  // number of them (the same sums either way)
  if ((H / 32 / ks) % 2 == 0)
    hipLaunchKernelGGL(router_logits_mfma<2>, grid, dim3(256), 0, s, x, wr, T, H, E, dst, xq,
                       xq_scales);
  else
    hipLaunchKernelGGL(router_logits_mfma<1>, grid, dim3(256), 0, s, x, wr, T, H, E, dst, xq,
                       xq_scales);
  return ks > 1 ? ks : 0;
}

int launch_router_logits(const uint16_t* x, const float* wr, int T, int H, int E, float* logits,
                         float* ws, hipStream_t s) {
  const int S = launch_router_slices(x, wr, T, H, E, logits, ws, nullptr, nullptr, s);
  if (S > 0)
    hipLaunchKernelGGL(router_reduce, dim3((T * E + 255) / 256), dim3(256), 0, s, ws, S, T, E,
                       logits);
  return launch_status();
}

// ---------------------------------------------------------------- S2 ------
// One wave per token.  Lane l holds experts l + 64 i, i < NSL = ceil(E/64).
// Each candidate has an order-preserving unsigned key (softmax: the fp32
// key; sigmoid: the fp64 key as hi:lo words), -0 folded into +0 and NaN
// treated as -inf; a candidate beats another on a larger key, then on a
// smaller id.  Each of the k rounds: the wave maximum of the (high) key word
// with v_max_u32 over DPP (quad xor 1 and 2, half-row and row mirror,
// row_bcast15 and row_bcast31; lane 63 ends with the maximum); in sigmoid
// mode the same for the low word among the candidates that reach the high
// maximum; then the smallest id holding the maximum from ballots, slot by
// slot (ids ascend with the slot, then the lane).  The owner retires it.
// 32-bit operations only, no per-round LDS traffic.  Weights are fp64.
__device__ __forceinline__ uint32_t ord_key32(float f) {
  f = (f != f) ? -__builtin_inff() : f + 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord_key32(uint32_t u) {
  return __uint_as_float((u >> 31) ? (u & 0x7fffffffu) : ~u);
}

__device__ __forceinline__ uint64_t ord_key64(double d) {
  d = (d != d) ? -__builtin_inf() : d + 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ uint32_t rdlane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
  return o > v ? o : v;
}

// Maximum of v over the wave (wave-uniform result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast15: rows 1, 3 take lane 15 of the row before
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast31: rows 2, 3 take lane 31
  return rdlane(v, 63);
}

// Sum of v over the wave: butterfly inside 16-lane rows (DPP), then the four
// row sums as (r0 + r1) + (r2 + r3).
__device__ __forceinline__ double wave_sum_f64(double v) {
  auto step = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)u, (int)(uint32_t)u, C, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(u >> 32),
                                                              (int)(uint32_t)(u >> 32), C, 0xF, 0xF, false);
    v += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  };
  step(std::integral_constant<int, 0xB1>{});
  step(std::integral_constant<int, 0x4E>{});
  step(std::integral_constant<int, 0x141>{});
  step(std::integral_constant<int, 0x140>{});
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  double r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = __longlong_as_double(
        (long long)(((uint64_t)rdlane((uint32_t)(u >> 32), 16 * q) << 32) | rdlane((uint32_t)u, 16 * q)));
  return (r[0] + r[1]) + (r[2] + r[3]);
}

// The bias of experts lane + 64 i (lanes past E read expert E - 1; 0
// without a bias).  Loaded before the logits, whose loads it does not depend
// on, so that the gate waits for one memory round trip, not two.  Buffer
// loads with no branches: without a bias the descriptor holds no records,
// and its loads return zeros without a memory access.
template <int NSL>
__device__ __forceinline__ void load_bias(const float* __restrict__ bias, int E, float (&bv)[4]) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t br = mx_rsrc(bias, bias != nullptr ? (uint32_t)E * 4u : 0u);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    bv[i] = i < NSL ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                          br, min(lane + 64 * i, E - 1) * 4, 0, 0))
                    : 0.f;
}

// Logits of token t (wave-uniform) as the slice-order sum of S partials
// ([S, T, E] fp32, the summation of router_reduce, so the same bits); lane
// holds experts lane + 64 i, i < NSL.  The partials were written by other
// CUs (other L2s), so every load of a batch of 16 slices is issued before
// the first add.  Buffer loads: slice and token go into the scalar offset,
// the lane's expert is a fixed byte offset (lanes past E read expert E - 1,
// ignored), and slices past S load slice S - 1 without being summed, so the
// loads need no address registers and no branches.  S * T * E * 4 < 2^31.
template <int NSL>
__device__ __forceinline__ void sum_token_slices(const float* __restrict__ partial, int S, int T,
                                                 int E, int t, float (&L)[4]) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t pr = mx_rsrc(partial, (uint32_t)S * (uint32_t)T * (uint32_t)E * 4u);
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    voff[i] = min(lane + 64 * i, E - 1) * 4;
    L[i] = 0.f;
  }
  for (int s0 = 0; s0 < S; s0 += 16) {
    float q[4][16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int soff = __builtin_amdgcn_readfirstlane((min(s0 + u, S - 1) * T + t) * E * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        q[i][u] = i < NSL ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(pr, voff[i], soff, 0))
                          : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (s0 + u < S) L[i] = (s0 + u == 0) ? q[i][u] : L[i] + q[i][u];
  }
}

// Top-k of one token.  L[i] = logit of expert lane + 64 i (ignored past E),
// bv[i] its bias (load_bias; used only when has_bias).  Writes ids[0..k) and
// weights[0..k) of the token; returns this lane's selected expert for
// lanes < k.
template <int MODE, int NSL>
__device__ __forceinline__ uint32_t gate_token(const float (&L)[4], const float (&bv)[4],
                                               bool has_bias, int E, int k, float routed_scale,
                                               float eps, int32_t* __restrict__ ids_row,
                                               float* __restrict__ w_row) {
  const int lane = threadIdx.x & 63;
  uint32_t khi[NSL], klo[NSL];  // 0 = retired or no expert (below every real key)
  double sval[NSL];
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    const int e = lane + 64 * i;
    khi[i] = 0;
    klo[i] = 0;
    sval[i] = 0.0;
    if (e < E) {
      if (MODE == 0) {
        khi[i] = ord_key32(has_bias ? (L[i] + bv[i]) : L[i]);  // fp32 add, as the oracle
      } else {
        const double sg = 1.0 / (1.0 + exp(-(double)L[i]));
        sval[i] = sg;
        const uint64_t o = ord_key64(has_bias ? sg + (double)bv[i] : sg);
        khi[i] = (uint32_t)(o >> 32);
        klo[i] = (uint32_t)o;
      }
    }
  }
  uint32_t my_key = 0, my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t m = khi[0];
#pragma unroll
    for (int i = 1; i < NSL; ++i) m = max(m, khi[i]);
    const uint32_t mh = wave_max_u32(m);
    uint32_t ml = 0;
    if (MODE == 1) {
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < NSL; ++i)
        if (khi[i] == mh) c = max(c, klo[i]);
      ml = wave_max_u32(c);
    }
    // smallest id holding the maximum: slot by slot, then the lowest lane
    uint32_t wid = 0;
#pragma unroll
    for (int i = NSL - 1; i >= 0; --i) {
      const unsigned long long bal =
          __ballot(khi[i] == mh && (MODE == 0 || klo[i] == ml) && (khi[i] | klo[i]) != 0);
      if (bal) wid = 64u * i + (uint32_t)(__ffsll((long long)bal) - 1);
    }
    // the owner retires it
#pragma unroll
    for (int i = 0; i < NSL; ++i)
      if ((uint32_t)(lane + 64 * i) == wid) {
        khi[i] = 0;
        klo[i] = 0;
      }
    if (lane == j) {
      my_key = mh;
      my_id = wid;
    }
  }
  double v;
  if (MODE == 0) {
    const double k0 = (double)unord_key32(__shfl(my_key, 0, 64));
    v = (lane < k) ? exp((double)unord_key32(my_key) - k0) : 0.0;
  } else {
    // the unbiased sigmoid of this lane's winner, from its owner lane
    const int src = (int)(my_id & 63u), slot = (int)(my_id >> 6);
    double sv = 0.0;
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      const double o = __shfl(sval[i], src, 64);
      if (slot == i) sv = o;
    }
    v = (lane < k) ? sv : 0.0;
  }
  const double sum = wave_sum_f64(v);
  if (lane < k) {
    double w;
    if (MODE == 0)
      w = v / sum;
    else
      w = v / (sum + (double)eps) * (double)routed_scale;
    ids_row[lane] = (int32_t)my_id;
    w_row[lane] = (float)w;
  }
  return my_id;
}

template <int MODE, int NSL>
__global__ __launch_bounds__(256) void gate_topk_kernel(const float* __restrict__ logits,
                                                        const float* __restrict__ bias, int T,
                                                        int E, int k, float routed_scale,
                                                        float eps, int32_t* __restrict__ ids,
                                                        float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; no barriers
  float bv[4];
  load_bias<NSL>(bias, E, bv);
  float L[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    L[i] = e < E ? logits[(size_t)t * E + e] : 0.f;
  }
  gate_token<MODE, NSL>(L, bv, bias != nullptr, E, k, routed_scale, eps, ids + (size_t)t * k,
                        wout + (size_t)t * k);
}

// S1's last step fused into S2: wave t sums token t's slice partials (the
// summation of router_reduce, so the logits are the same bits), stores them
// and runs the gate; saves a launch and a round trip of the logits.
template <int MODE, int NSL>
__global__ __launch_bounds__(256) void gate_topk_slices_kernel(
    const float* __restrict__ partial, int S, const float* __restrict__ bias, int T, int E, int k,
    float routed_scale, float eps, float* __restrict__ logits, int32_t* __restrict__ ids,
    float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; no barriers
  float bv[4];
  load_bias<NSL>(bias, E, bv);
  float L[4];
  sum_token_slices<NSL>(partial, S, T, E, t, L);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    if (i < NSL && e < E) logits[(size_t)t * E + e] = L[i];
  }
  gate_token<MODE, NSL>(L, bv, bias != nullptr, E, k, routed_scale, eps, ids + (size_t)t * k,
                        wout + (size_t)t * k);
}

// --------------------------------------------------- S1+S2+S3/S4, decode ---
// Few tokens (T <= 16, T*k <= 1024), after router_partial: one one-wave
// block per token, each on its own CU.  Block t sums token t's slice
// partials (slice order, as router_reduce) into its logits, stores them and
// runs the top-k of gate_token.  Then it counts itself done on a device
// counter that router_partial zeroed: a release fence, one atomic add; no
// block waits for another.  The block that counts last (it sees T - 1) takes
// an acquire fence, so every block's ids are visible to it, and does
// init_routing and the expert-token counts ([Qwen3] "GMM enablement and
// routing optimisation") for the T*k pairs: per-expert counts in LDS, their
// exclusive scan, then the pairs in chunks of 64 in pair order, those with
// the same expert matched with ballots over the 8 id bits and ranked by lane.
// The order (expert, then pair index) is the stable counting sort of the
// standalone route kernels.
template <int MODE, int NSL>
__global__ __launch_bounds__(64) void gate_route_decode(
    const float* __restrict__ partial, int S, const float* __restrict__ bias, int T, int E, int k,
    float routed_scale, float eps, float* __restrict__ logits, int32_t* __restrict__ ids,
    float* __restrict__ wout, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ dev_status, int32_t* __restrict__ done) {
  __shared__ int cnt[256];  // per-expert counts, then the next free position
  __shared__ int last;
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  {
    float bv[4];
    load_bias<NSL>(bias, E, bv);
    float L[4];
    sum_token_slices<NSL>(partial, S, T, E, t, L);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (i < NSL && e < E) logits[(size_t)t * E + e] = L[i];
    }
    gate_token<MODE, NSL>(L, bv, bias != nullptr, E, k, routed_scale, eps, ids + (size_t)t * k,
                          wout + (size_t)t * k);
  }
  // this block's stores before its count; the count of the block that sees
  // T - 1 comes after every other block's
  __threadfence();
  __syncthreads();
  if (lane == 0) last = atomicAdd(done, 1) == T - 1;
  __syncthreads();
  if (!last) return;  // block-uniform; no barriers after this for the others
  __threadfence();
  const int R = T * k;
  for (int e = lane; e < 256; e += 64) cnt[e] = 0;
  __syncthreads();
  bool bad = false;
  for (int p = lane; p < R; p += 64) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    else bad = true;
  }
  __syncthreads();
  // exclusive scan of the counts: lane l holds experts 4l .. 4l+3 (E <= 256)
  int v[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;
    v[j] = e < E ? cnt[e] : 0;
    sum += v[j];
  }
  const int incl = wave_incl_scan(sum);
  int run = incl - sum;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;
    if (e < E) {
      counts[e] = v[j];
      offsets[e] = run;
      cnt[e] = run;
    }
    run += v[j];
  }
  if (lane == 63) offsets[E] = run;
  __syncthreads();
  for (int p0 = 0; p0 < R; p0 += 64) {  // chunks in pair order
    const int p = p0 + lane;
    const int e = p < R ? ids[p] : -1;
    const bool ok = e >= 0 && e < E;
    unsigned long long match = __ballot(ok);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = ok && ((e >> bit) & 1);
      const unsigned long long bb = __ballot(on);
      match &= ((e >> bit) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(match & ((1ull << lane) - 1ull));
    const int pos = ok ? cnt[e] + rank : -1;
    __syncthreads();  // every lane has read its expert's position
    if (ok) {
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
      if (rank == 0) cnt[e] += __popcll(match);
    } else if (p < R) {
      pair_pos[p] = -1;
    }
    __syncthreads();
  }
  const bool any_bad = __ballot(bad) != 0ull;
  if (lane == 0 && dev_status != nullptr) *dev_status = any_bad ? 1 : 0;
}

// Slots per lane for E experts (lane l holds experts l + 64 i).
template <template <int, int> class F, typename... A>
static void by_mode_slots(int mode, int E, A... args) {
  const int nsl = (E + 63) / 64;
  if (mode == 0) {
    if (nsl <= 1) F<0, 1>::run(args...);
    else if (nsl == 2) F<0, 2>::run(args...);
    else if (nsl == 3) F<0, 3>::run(args...);
    else F<0, 4>::run(args...);
  } else {
    if (nsl <= 1) F<1, 1>::run(args...);
    else if (nsl == 2) F<1, 2>::run(args...);
    else if (nsl == 3) F<1, 3>::run(args...);
    else F<1, 4>::run(args...);
  }
}

template <int MODE, int NSL>
struct GateRouteDecode {
  static void run(hipStream_t s, const float* partial, int S, const float* bias, int T, int E, int k,
                  float routed_scale, float eps, float* logits, int32_t* ids, float* w,
                  int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                  int32_t* dev_status, int32_t* done) {
    hipLaunchKernelGGL((gate_route_decode<MODE, NSL>), dim3(T), dim3(64), 0, s, partial, S, bias,
                       T, E, k, routed_scale, eps, logits, ids, w, counts, offsets, sorted_pair,
                       pair_pos, dev_status, done);
  }
};

template <int MODE, int NSL>
struct GateTopk {
  static void run(hipStream_t s, const float* logits, const float* bias, int T, int E, int k,
                  float routed_scale, float eps, int32_t* ids, float* w) {
    hipLaunchKernelGGL((gate_topk_kernel<MODE, NSL>), dim3((T + 3) / 4), dim3(256), 0, s, logits,
                       bias, T, E, k, routed_scale, eps, ids, w);
  }
};

template <int MODE, int NSL>
struct GateTopkSlices {
  static void run(hipStream_t s, const float* partial, int S, const float* bias, int T, int E,
                  int k, float routed_scale, float eps, float* logits, int32_t* ids, float* w) {
    hipLaunchKernelGGL((gate_topk_slices_kernel<MODE, NSL>), dim3((T + 3) / 4), dim3(256), 0, s,
                       partial, S, bias, T, E, k, routed_scale, eps, logits, ids, w);
  }
};

int launch_router_gate(const uint16_t* x, const float* wr, int T, int H, int E, int k, int mode,
                       float routed_scale, float eps, const float* bias, float* logits,
                       int32_t* ids, float* w, float* ws, uint8_t* xq, uint8_t* xq_scales,
                       hipStream_t s) {
  const int S = launch_router_slices(x, wr, T, H, E, logits, ws, xq, xq_scales, s);
  if (S > 0)
    by_mode_slots<GateTopkSlices>(mode, E, s, static_cast<const float*>(ws), S, bias, T, E, k,
                                  routed_scale, eps, logits, ids, w);
  else
    by_mode_slots<GateTopk>(mode, E, s, static_cast<const float*>(logits), bias, T, E, k,
                            routed_scale, eps, ids, w);
  return launch_status();
}

int launch_gate_route_decode(const float* partial, int H, const float* bias, int T, int E, int k,
                             int mode, float routed_scale, float eps, float* logits, int32_t* ids,
                             float* w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                             int32_t* pair_pos, int32_t* dev_status, int32_t* done,
                             hipStream_t s) {
  by_mode_slots<GateRouteDecode>(mode, E, s, partial, H / RP_HS, bias, T, E, k, routed_scale, eps,
                                 logits, ids, w, counts, offsets, sorted_pair, pair_pos,
                                 dev_status, done);
  return launch_status();
}

int launch_gate_topk(const float* logits, const float* bias, int T, int E, int k, int mode,
                     float routed_scale, float eps, int32_t* ids, float* w, hipStream_t s) {
  by_mode_slots<GateTopk>(mode, E, s, logits, bias, T, E, k, routed_scale, eps, ids, w);
  return launch_status();
}

}  // namespace moe
