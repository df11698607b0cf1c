// W4A8 path: MXFP8 (E4M3FN) activations x MXFP4 (E2M1) expert weights with
// E8M0 block scales, on gfx950's block-scaled MFMA.
//
// [Qwen3] "MoE EP optimisation -> compute decomposition (AllGather scheme,
// W4A8)": hidden_states are quantised dynamically to MXFP8 data plus a scale
// tensor before the grouped matmul; "fused-operator optimisation": the MX
// quantisation uses round_mode rint and dst_type float8_e4m3fn.  [Hy3]
// section 5.2: on the quantised path the SwiGLU output is group-quantised
// before the down projection.
//
// Block rule (blocks of 32 along the reduction dimension): shared exponent
// e = floor(log2(amax)) - 8 clamped to [-127, 127] (amax 0 -> -127), scale
// code e + 127, element = E4M3 round-to-nearest-even of v / 2^e saturated to
// +-448; a value rounding to zero keeps its sign bit.  The encoder is
// integer-exact (no hardware convert), so codes are reproducible bit for bit.
//
// S0 (mx_quant): four lanes per 32-block, 8 elements per lane.
// S5/S6 (ffn_mx_up / ffn_mx_down): the skinny weight-streaming tiles of the
// bf16 path with v_mfma_scale_f32_16x16x128_f8f6f4 (E2M1 weights as the A
// operand, E4M3 activations as B).  Operand layout of one 128-wide K step,
// lane l = 16*g + i (row or column i, g = 0..3), measured on gfx950:
//   E2M1: 16 bytes holding k = 32g .. 32g+31, low nibble = even k;
//   E4M3: bytes 0-15 hold k = 16g .. 16g+15, bytes 16-31 hold
//         k = 64+16g .. 64+16g+15;
//   scale operand (byte 0): the E8M0 scale of row/column i, 32-block g.
// GEMM1's epilogue forms SiLU(g) * u and quantises it to MXFP8 along I
// (32-column blocks) before storing.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// E4M3FN code of v (already divided by its block scale), RNE, saturating.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7fffffffu);
  if (!(a < 448.f)) return sign | 0x7eu;  // saturate (also catches NaN)
  if (a < 0.015625f) {                    // below 2^-6: subnormal grid 2^-9
    const uint32_t m = (uint32_t)rintf(a * 512.f);  // 0..8; 8 is 2^-6 = code 0x08
    return sign | m;
  }
  int E = (int)((bits >> 23) & 0xffu) - 127;  // floor(log2 a), -6..8
  const float q = __uint_as_float((uint32_t)(127 + 3 - E) << 23) * a;  // a * 2^(3-E) in [8,16)
  uint32_t m = (uint32_t)rintf(q);
  if (m == 16u) {
    m = 8u;
    ++E;
  }
  uint32_t code = ((uint32_t)(E + 7) << 3) | (m - 8u);
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
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

// ------------------------------------------------------------ S0 quant ---
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t* __restrict__ x, int rows,
                                                       int cols, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const long long chunk = (long long)blockIdx.x * 256 + threadIdx.x;  // 8 elements each
  const long long nchunks = (long long)rows * cols / 8;
  const bool ok = chunk < nchunks;
  const long long c = ok ? chunk : nchunks - 1;
  const u32x4 v = ld16(x + c * 8);
  float f[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = bf16_to_f32(v[q] & 0xffffu);
    f[2 * q + 1] = bf16_to_f32(v[q] >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int e = mx_exponent(amax);
  const float inv = exp2_neg(e);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= e4m3_encode(f[i] * inv) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= e4m3_encode(f[4 + i] * inv) << (8 * i);
  if (ok) {
    *reinterpret_cast<u32x2*>(codes + c * 8) = u32x2{lo, hi};
    if ((threadIdx.x & 3) == 0) scales[c / 4] = (uint8_t)(e + 127);
  }
}

int launch_mx_quantize(const uint16_t* x, int rows, int cols, uint8_t* codes, uint8_t* scales,
                       hipStream_t s) {
  const long long nchunks = (long long)rows * cols / 8;
  const long long blocks = (nchunks + 255) / 256;
  hipLaunchKernelGGL(mx_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, cols,
                     codes, scales);
  return launch_status();
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

// ---------------------------------------------------- GEMM1 (+SwiGLU) -----
// Tile: 16 rows x 32 output columns (gate rows n0..n0+31 and up rows
// I+n0..I+n0+31).  WK waves split K; each wave issues the loads of all S of
// its 128-wide K steps before the first MFMA (the whole slice is one memory
// round trip), then the waves reduce through LDS.  S == 0 selects a loop
// over the steps for shapes without a fixed split.
template <int WK, int S>
__device__ __forceinline__ void mx_up_tile(const GroupedGemm& g, int lane, int wk, int n_tile,
                                           int grp, int row0, int nrows) {
  const int li = lane & 15, kb = lane >> 4;  // row in a 16-group, 32-block in a 128-step
  const int n0 = n_tile * 32;
  const int K = g.K;
  const int r = row0 + min(li, nrows - 1);
  const int arow = g.gather ? g.sorted_pair[r] / g.topk : r;
  const int Kw = K / WK, kbeg = wk * Kw;
  const uint8_t* xa = static_cast<const uint8_t*>(g.A) + (size_t)arow * K + kbeg + 16 * kb;
  const uint8_t* xs = g.A_scales + (size_t)arow * (K / 32) + kbeg / 32 + kb;
  const uint8_t* W = static_cast<const uint8_t*>(g.W) + (size_t)grp * g.w_gstride;
  const uint8_t* Sc = g.W_scales + (size_t)grp * g.ws_gstride;
  const int rows4[4] = {n0 + li, n0 + 16 + li, g.up_off + n0 + li, g.up_off + n0 + 16 + li};
  const uint8_t* wp[4];
  const uint8_t* sp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    wp[j] = W + (size_t)rows4[j] * (K / 2) + (kbeg + 32 * kb) / 2;
    sp[j] = Sc + (size_t)rows4[j] * (K / 32) + kbeg / 32 + kb;
  }
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (S > 0) {
    u32x4 wa[S > 0 ? S : 1][4];
    uint32_t ws[S > 0 ? S : 1][4], xsc[S > 0 ? S : 1];
    i32x8 xb[S > 0 ? S : 1];
#pragma unroll
    for (int st = 0; st < S; ++st) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wa[st][j] = ld16_stream(wp[j] + st * 64);
        ws[st][j] = sp[j][st * 4];
      }
      xb[st] = ld32_fp8(xa + st * 128);
      xsc[st] = xs[st * 4];
    }
#pragma unroll
    for (int st = 0; st < S; ++st)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma_fp4_fp8(wa[st][j], xb[st], ws[st][j], xsc[st], acc[j]);
  } else {
    const int nsteps = Kw / 128;
    for (int st = 0; st < nsteps; ++st) {
      u32x4 wa[4];
      uint32_t ws[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wa[j] = ld16_stream(wp[j] + st * 64);
        ws[j] = sp[j][st * 4];
      }
      const i32x8 xb = ld32_fp8(xa + st * 128);
      const uint32_t xsc = xs[st * 4];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma_fp4_fp8(wa[j], xb, ws[j], xsc, acc[j]);
    }
  }
  if (WK > 1) {
    __shared__ f32x4 red[WK > 1 ? WK - 1 : 1][4][64];
    if (wk > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wk - 1][j][lane] = acc[j];
    }
    __syncthreads();
    if (wk != 0) {
      __syncthreads();
      return;
    }
#pragma unroll
    for (int w = 0; w < WK - 1; ++w)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += red[w][j][lane];
    __syncthreads();
  }
  // D[n][m]: lane holds token li, columns n0 + 4*kb + i (lo) and n0 + 16 + 4*kb + i (hi)
  float a[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = (acc[0][i] / (1.f + expf(-acc[0][i]))) * acc[2][i];
    a[4 + i] = (acc[1][i] / (1.f + expf(-acc[1][i]))) * acc[3][i];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(a[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  const int e = mx_exponent(amax);
  const float inv = exp2_neg(e);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= e4m3_encode(a[i] * inv) << (8 * i);
    hi |= e4m3_encode(a[4 + i] * inv) << (8 * i);
  }
  if (li < nrows) {
    uint8_t* orow = static_cast<uint8_t*>(g.out) + (size_t)(row0 + li) * g.N;
    *reinterpret_cast<uint32_t*>(orow + n0 + 4 * kb) = lo;
    *reinterpret_cast<uint32_t*>(orow + n0 + 16 + 4 * kb) = hi;
    if (kb == 0) g.out_scales[(size_t)(row0 + li) * (g.N / 32) + n0 / 32] = (uint8_t)(e + 127);
  }
}

template <int WK, int S>
__global__ __launch_bounds__(64 * WK) void ffn_mx_up(GroupedGemm g, int n_tiles) {
  const int lane = threadIdx.x & 63, wk = threadIdx.x >> 6;
  TileMap tm;
  tm.init(g.offsets, g.G, g.ident_rows, 16);
  const int total = tm.total * n_tiles;
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int id = xcd_remap(t, total);
    const int n_tile = id / tm.total;
    int grp, row0, nrows;
    tm.find(id - n_tile * tm.total, grp, row0, nrows);
    mx_up_tile<WK, S>(g, lane, wk, n_tile, grp, row0, nrows);
  }
}

// ------------------------------------------------------------- GEMM2 -----
// Tile: 16 rows x 16*WN output columns; wave (wn, wk) streams 16 rows of w2
// over K slice wk (all S steps loaded at once when S > 0), then the WK
// partial sums of each column group are reduced through LDS.
template <int WN, int WK, int S>
__global__ __launch_bounds__(64 * WN * WK) void ffn_mx_down(GroupedGemm g, int n_tiles) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % WN, wk = wave / WN;
  const int li = lane & 15, kb = lane >> 4;
  TileMap tm;
  tm.init(g.offsets, g.G, g.ident_rows, 16);
  const int total = tm.total * n_tiles;
  const int K = g.K;
  const int Kw = K / WK, kbeg = wk * Kw;
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int id = xcd_remap(t, total);
    const int n_tile = id / tm.total;
    int grp, row0, nrows;
    tm.find(id - n_tile * tm.total, grp, row0, nrows);
    const int n0 = n_tile * 16 * WN + wn * 16;
    const int r = row0 + min(li, nrows - 1);
    const uint8_t* xa = static_cast<const uint8_t*>(g.A) + (size_t)r * K + kbeg + 16 * kb;
    const uint8_t* xs = g.A_scales + (size_t)r * (K / 32) + kbeg / 32 + kb;
    const uint8_t* wp = static_cast<const uint8_t*>(g.W) + (size_t)grp * g.w_gstride +
                        (size_t)(n0 + li) * (K / 2) + (kbeg + 32 * kb) / 2;
    const uint8_t* sp = g.W_scales + (size_t)grp * g.ws_gstride + (size_t)(n0 + li) * (K / 32) +
                        kbeg / 32 + kb;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (S > 0) {
      u32x4 wa[S > 0 ? S : 1];
      uint32_t ws[S > 0 ? S : 1], xsc[S > 0 ? S : 1];
      i32x8 xb[S > 0 ? S : 1];
#pragma unroll
      for (int u = 0; u < S; ++u) {
        wa[u] = ld16_stream(wp + u * 64);
        ws[u] = sp[u * 4];
        xb[u] = ld32_fp8(xa + u * 128);
        xsc[u] = xs[u * 4];
      }
#pragma unroll
      for (int u = 0; u < S; ++u) acc = mfma_fp4_fp8(wa[u], xb[u], ws[u], xsc[u], acc);
    } else {
      const int nsteps = Kw / 128;
      for (int u = 0; u < nsteps; ++u)
        acc = mfma_fp4_fp8(ld16_stream(wp + u * 64), ld32_fp8(xa + u * 128), sp[u * 4], xs[u * 4], acc);
    }
    if (WK > 1) {
      __shared__ f32x4 red[WK > 1 ? WK - 1 : 1][WN][64];
      if (wk > 0) red[wk - 1][wn][lane] = acc;
      __syncthreads();
      if (wk == 0) {
#pragma unroll
        for (int w = 0; w < WK - 1; ++w) acc += red[w][wn][lane];
      }
      __syncthreads();
      if (wk != 0) continue;
    }
    if (li < nrows) {
      const int nc = n0 + 4 * kb;
      u32x2 pk;
      pk.x = pack_bf16x2(acc[0], acc[1]);
      pk.y = pack_bf16x2(acc[2], acc[3]);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.out) + (size_t)(row0 + li) * g.N + nc) = pk;
    }
  }
}

// ----------------------------------------------------------- launchers ----

static inline long long mx_tiles_bound(const GroupedGemm& g, int n_tiles) {
  const int groups = g.offsets ? g.G : 1;
  return ((long long)(g.total_rows + 15) / 16 + groups) * n_tiles;
}

template <int WK, int S>
static void launch_mx_up(const GroupedGemm& g, hipStream_t s) {
  const int nt = g.N / 32;
  auto k = ffn_mx_up<WK, S>;
  const int grid = resident_grid(reinterpret_cast<const void*>(k), 64 * WK, mx_tiles_bound(g, nt));
  hipLaunchKernelGGL(k, dim3(grid), dim3(64 * WK), 0, s, g, nt);
}

// K = H: 128-wide steps split over WK waves, S steps each (all in flight).
int launch_ffn_up_w4a8(const GroupedGemm& g, hipStream_t s) {
  const int steps = g.K / 128;
  if (steps == 32)
    launch_mx_up<8, 4>(g, s);
  else if (steps == 16)
    launch_mx_up<4, 4>(g, s);
  else if (steps == 8)
    launch_mx_up<2, 4>(g, s);
  else if (steps == 4)
    launch_mx_up<1, 4>(g, s);
  else if (steps == 2)
    launch_mx_up<1, 2>(g, s);
  else if (steps % 4 == 0)
    launch_mx_up<4, 0>(g, s);
  else
    launch_mx_up<1, 0>(g, s);
  return launch_status();
}

template <int WN, int WK, int S>
static void launch_mx_down(const GroupedGemm& g, hipStream_t s) {
  const int nt = g.N / (16 * WN);
  auto k = ffn_mx_down<WN, WK, S>;
  const int grid = resident_grid(reinterpret_cast<const void*>(k), 64 * WN * WK, mx_tiles_bound(g, nt));
  hipLaunchKernelGGL(k, dim3(grid), dim3(64 * WN * WK), 0, s, g, nt);
}

// K = I: same idea; N = H is a multiple of 64.
int launch_ffn_down_w4a8(const GroupedGemm& g, hipStream_t s) {
  const int steps = g.K / 128;
  if (steps == 12)
    launch_mx_down<4, 1, 12>(g, s);
  else if (steps == 8)
    launch_mx_down<2, 2, 4>(g, s);
  else if (steps == 4)
    launch_mx_down<4, 1, 4>(g, s);
  else if (steps == 2)
    launch_mx_down<4, 1, 2>(g, s);
  else if (steps == 1)
    launch_mx_down<4, 1, 1>(g, s);
  else
    launch_mx_down<4, 1, 0>(g, s);
  return launch_status();
}

}  // namespace moe
