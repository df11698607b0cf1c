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
// the hardware E4M3 convert after a +-448 clamp, equal to the rule on every
// fp32 input, so codes are reproducible bit for bit.
//
// S0 (mx_quant): four lanes per 32-block, 8 elements per lane.
// S5/S6 (ffn_mx_stream): weight-streaming grouped GEMMs on
// v_mfma_scale_f32_16x16x128_f8f6f4 (E2M1 weights as the A operand, E4M3
// activations as B), one wave per 16-row tile.  Operand layout of one 128-wide K step,
// lane l = 16*g + i (row or column i, g = 0..3), measured on gfx950:
//   E2M1: 16 bytes holding k = 32g .. 32g+31, low nibble = even k;
//   E4M3: bytes 0-15 hold k = 16g .. 16g+15, bytes 16-31 hold
//         k = 64+16g .. 64+16g+15;
//   scale operand (byte 0): the E8M0 scale of row/column i, 32-block g.
// GEMM1's epilogue forms SiLU(g) * u and quantises it to MXFP8 along I
// (32-column blocks) before storing.
#include "common.hpp"
#include "launch.hpp"
#include "mxfmt.hpp"

namespace moe {



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
  const uint32_t lo = e4m3_pack4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
  const uint32_t hi = e4m3_pack4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
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

// ------------------------------------------------------- weight pack -----
// Packed W4A8 weight layout, per matrix of R rows (R % 16 == 0) and K
// reduction columns (K % 128 == 0), ns = K/128 steps, nq = ceil(ns/4):
//   codes : block (q, s) at byte (q*ns + s)*1024 (q = group of 16 rows,
//           s = K-step); its lane l = 16*kb + i holds the 16 bytes
//           [64s + 16kb, +16) of row 16q + i, i.e. E2M1 k = 128s + 32kb ..
//           +31: exactly the A operand of lane l for step s.
//   scales: block (q, c) at byte (q*nq + c)*256; lane l = 16*kb + i holds a
//           dword whose byte u is the E8M0 scale of row 16q + i, 32-block
//           4(4c + u) + kb (steps 4c .. 4c+3; zero past the last step).
// Codes keep their size; scales grow only when ns % 4 != 0.
size_t mx_packed_scales_bytes(int rows, int K) {
  const int ns = K / 128, nq = (ns + 3) / 4;
  return (size_t)(rows / 16) * (size_t)nq * 256u;
}

__global__ __launch_bounds__(256) void mx_pack_codes(const uint8_t* __restrict__ codes, long long n,
                                                     int R, int K, uint8_t* __restrict__ pc) {
  const int ns = K / 128;
  for (long long c = (long long)blockIdx.x * 256 + threadIdx.x; c < n;
       c += (long long)gridDim.x * 256) {
    // c = ((g*(R/16) + q)*ns + s)*64 + l: the 16-byte chunk c of the packed matrix
    const int l = (int)(c & 63);
    const long long blk = c >> 6;
    const int s = (int)(blk % ns);
    const long long gq = blk / ns;  // g*(R/16) + q
    const long long row = gq * 16 + (l & 15);  // global row g*R + 16q + i
    const u32x4 v = ld16(codes + row * (K / 2) + s * 64 + 16 * (l >> 4));
    *reinterpret_cast<u32x4*>(pc + c * 16) = v;
  }
}

__global__ __launch_bounds__(256) void mx_pack_scales(const uint8_t* __restrict__ scales, long long n,
                                                      int R, int K, uint8_t* __restrict__ ps) {
  const int ns = K / 128, nq = (ns + 3) / 4;
  for (long long d = (long long)blockIdx.x * 256 + threadIdx.x; d < n;
       d += (long long)gridDim.x * 256) {
    // d = ((g*(R/16) + q)*nq + c)*64 + l: the dword d of the packed scales
    const int l = (int)(d & 63);
    const long long blk = d >> 6;
    const int c = (int)(blk % nq);
    const long long row = (blk / nq) * 16 + (l & 15);
    uint32_t w = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int st = 4 * c + u;
      if (st < ns) w |= (uint32_t)scales[row * (K / 32) + 4 * st + (l >> 4)] << (8 * u);
    }
    *reinterpret_cast<uint32_t*>(ps + d * 4) = w;
  }
}

int launch_mx_pack(const uint8_t* codes, const uint8_t* scales, int G, int R, int K,
                   uint8_t* pc, uint8_t* ps, hipStream_t s) {
  const long long nc = (long long)G * R * (K / 32);                        // 16-byte chunks
  const long long nd = (long long)G * (long long)(mx_packed_scales_bytes(R, K) / 4);  // dwords
  const int grid = 2048;
  hipLaunchKernelGGL(mx_pack_codes, dim3(grid), dim3(256), 0, s, codes, nc, R, K, pc);
  hipLaunchKernelGGL(mx_pack_scales, dim3(grid), dim3(256), 0, s, scales, nd, R, K, ps);
  return launch_status();
}

// ------------------------------------------------ streaming W4A8 GEMMs ---
// One wave owns a whole tile (16 activation rows x 4 groups of 16 weight
// rows, the full K) and walks its tiles as one sequence of U-step batches,
// double-buffered in registers: the loads of the next batch, which may be the
// first batch of the wave's next tile, are issued before the MFMAs of the
// current one.  The weight stream of a wave therefore does not pause at tile
// boundaries, and no LDS, barrier or cross-wave reduction is involved.
// GEMM1 (SWIGLU): groups = gate rows n0.., n0+16.., up rows I+n0.., I+n0+16..
// (32 output columns, one MX block of the quantised output).  GEMM2: groups =
// rows n0 + 16j (64 output columns).
struct MxTile {
  int grp, n0, row0, nrows;  // wave-uniform (scalar registers)
  int live;                  // 0: no tile (its weight loads read nothing)
  const uint8_t* xa;         // this lane's activation row, + 16*kb
  const uint8_t* xs;         // this lane's activation scale row
};

template <bool SWIGLU>
__device__ __forceinline__ MxTile mx_tile_at(const GroupedGemm& g, const TileMap& tm, int id,
                                             int li, int kb) {
  MxTile t;
  const int n_tile = id / tm.total;
  int grp, row0, nrows;
  tm.find(id - n_tile * tm.total, grp, row0, nrows);
  t.grp = __builtin_amdgcn_readfirstlane(grp);
  t.row0 = __builtin_amdgcn_readfirstlane(row0);
  t.nrows = __builtin_amdgcn_readfirstlane(nrows);
  t.n0 = __builtin_amdgcn_readfirstlane(n_tile * (SWIGLU ? 32 : 64));
  const int r = t.row0 + min(li, t.nrows - 1);  // rows past the tile end reuse a valid row
  const int arow = gather_row(g.sorted_pair, g.gather, g.topk, g.total_rows, r);
  t.xa = static_cast<const uint8_t*>(g.A) + (size_t)arow * g.K + 16 * kb;
  t.xs = g.A_scales + (size_t)arow * (g.K / 32);
  t.live = 1;
  return t;
}

template <int U>
struct MxBatch {
  u32x4 w[U][4];   // E2M1 weights, 32 k per lane
  i32x8 x[U];      // E4M3 activations, 32 k per lane
  uint32_t ws[4];  // packed weight scales: byte (step & 3) of the step's quad
  uint32_t xs[U];  // activation scale words; this lane's byte is kb
  int sh;          // 8 * (first step & 3): bit offset of the first step's byte
};

// First row of weight group j (uniform); the lane adds li.
template <bool SWIGLU>
__device__ __forceinline__ int mx_wrow0(const GroupedGemm& g, int n0, int j) {
  if (SWIGLU) return (j >= 2 ? g.up_off : 0) + n0 + 16 * (j & 1);
  return n0 + 16 * j;
}

// Batch of U K-steps (128 each) starting at step st0 of tile t.  The weights
// are in the packed layout (moe_mx_pack_weight): the 16 rows of group j for
// one step are one contiguous 1 KB block in lane order, their scales for 4
// steps one 256-byte block (a dword per lane).  Both are read through buffer
// descriptors over the expert's matrix: the lane offset is fixed, the block
// index goes into the scalar offset, so each load instruction reads whole
// cache lines and the stream needs no per-tile vector address registers.
template <bool SWIGLU, int U>
__device__ __forceinline__ void mx_load(MxBatch<U>& b, const GroupedGemm& g, const MxTile& t,
                                        int st0, int lane) {
  const int ns = g.K / 128, nq = (ns + 3) / 4;  // K-steps, scale quads per row group
  // a dead tile gets empty descriptors: its loads return zeros without a
  // memory access
  const uint32_t wrows = SWIGLU ? 2u * (uint32_t)g.up_off : (uint32_t)g.N;  // rows of one matrix
  const __amdgpu_buffer_rsrc_t wr =
      mx_rsrc(static_cast<const uint8_t*>(g.W) + (size_t)t.grp * g.w_gstride,
              t.live ? wrows * (uint32_t)(g.K / 2) : 0u);
  const __amdgpu_buffer_rsrc_t sr = mx_rsrc(g.W_scales + (size_t)t.grp * g.ws_gstride,
                                            t.live ? wrows / 16u * (uint32_t)nq * 256u : 0u);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = mx_wrow0<SWIGLU>(g, t.n0, j) / 16;
#pragma unroll
    for (int u = 0; u < U; ++u)
      b.w[u][j] = __builtin_amdgcn_raw_buffer_load_b128(wr, lane * 16, (q * ns + st0 + u) * 1024, 0);
    // U <= 2 and st0 % U == 0: the batch's steps share one quad
    b.ws[j] = __builtin_amdgcn_raw_buffer_load_b32(sr, lane * 4, (q * nq + st0 / 4) * 256, 0);
  }
  b.sh = 8 * (st0 & 3);
#pragma unroll
  for (int u = 0; u < U; ++u) b.x[u] = ld32_fp8(t.xa + st0 * 128 + u * 128);
  if (U == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(t.xs + st0 * 4);
    b.xs[0] = v.x;
    b.xs[U - 1] = v.y;
  } else {
    b.xs[0] = *reinterpret_cast<const uint32_t*>(t.xs + st0 * 4);
  }
}

template <int U>
__device__ __forceinline__ void mx_compute(const MxBatch<U>& b, f32x4* acc, int kb) {
  const int sh = 8 * kb;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t xsc = (b.xs[u] >> sh) & 0xffu;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = mfma_fp4_fp8(b.w[u][j], b.x[u], (b.ws[j] >> (b.sh + 8 * u)) & 0xffu, xsc, acc[j]);
  }
}

// D[n][m]: lane (li, kb) holds activation row li and, for weight group j,
// output columns (group base) + 4*kb + i.
template <bool SWIGLU>
__device__ __forceinline__ void mx_store(const GroupedGemm& g, const MxTile& t, const f32x4* acc,
                                         int li, int kb) {
  if (SWIGLU) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = silu_fast(acc[0][i]) * acc[2][i];
      a[4 + i] = silu_fast(acc[1][i]) * acc[3][i];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(a[i]));
    amax = max_lanes_16_32(amax);
    const int e = mx_exponent(amax);
    const float inv = exp2_neg(e);
    const uint32_t lo = e4m3_pack4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
    const uint32_t hi = e4m3_pack4(a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv);
    if (li < t.nrows) {
      uint8_t* orow = static_cast<uint8_t*>(g.out) + (size_t)(t.row0 + li) * g.N;
      *reinterpret_cast<uint32_t*>(orow + t.n0 + 4 * kb) = lo;
      *reinterpret_cast<uint32_t*>(orow + t.n0 + 16 + 4 * kb) = hi;
      if (kb == 0) g.out_scales[(size_t)(t.row0 + li) * (g.N / 32) + t.n0 / 32] = (uint8_t)(e + 127);
    }
  } else if (li < t.nrows) {
    uint16_t* orow = static_cast<uint16_t*>(g.out) + (size_t)(t.row0 + li) * g.N + t.n0 + 4 * kb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 pk;
      pk.x = pack_bf16x2(acc[j][0], acc[j][1]);
      pk.y = pack_bf16x2(acc[j][2], acc[j][3]);
      *reinterpret_cast<u32x2*>(orow + 16 * j) = pk;
    }
  }
}

// At most 168 registers: three waves per SIMD, so that a decode layer's
// tiles (touched experts x column tiles, ~2,000-2,700) need about one wave each.
template <bool SWIGLU, int U, int D>
__global__ __launch_bounds__(256, 3) void ffn_mx_stream(GroupedGemm g, int n_tiles) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, kb = lane >> 4;
  // wave-major numbering: the first gridDim.x tiles go to wave 0 of every
  // block, so however few tiles there are, they spread over all CUs
  const int nw = gridDim.x * 4;
  // (readfirstlane: these are wave-uniform, and the buffer loads need their
  // scalar offsets in scalar registers)
  const int gw = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) * gridDim.x + blockIdx.x);
  TileMap tm;
  tm.init(g.offsets, g.G, g.ident_rows, 16, g.total_rows);
  const int total = __builtin_amdgcn_readfirstlane(tm.total * n_tiles);
  if (gw >= total) return;  // the kernel has no barriers
  const int nb = g.K / 128 / U;
  MxTile cur = mx_tile_at<SWIGLU>(g, tm, gw, li, kb);
  if constexpr (D == 3) {
    // three register batches in rotation (nb % 3 == 0): batches j+1 and j+2
    // are in flight while batch j computes; the last two loads of a tile
    // fetch the next tile's batches 0 and 1, so every tile starts with both
    // loaded
    MxBatch<U> b0, b1, b2;
    mx_load<SWIGLU, U>(b0, g, cur, 0, lane);
    mx_load<SWIGLU, U>(b1, g, cur, U, lane);
    for (int id = gw; id < total; id += nw) {
      MxTile nxt = cur;
      if (id + nw < total)
        nxt = mx_tile_at<SWIGLU>(g, tm, id + nw, li, kb);
      else
        nxt.live = 0;  // the batches loaded past the last tile read nothing
      f32x4 acc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int b = 0; b < nb; b += 3) {
        mx_load<SWIGLU, U>(b2, g, b + 2 < nb ? cur : nxt, b + 2 < nb ? (b + 2) * U : (b + 2 - nb) * U, lane);
        __builtin_amdgcn_sched_barrier(0);
        mx_compute<U>(b0, acc, kb);
        __builtin_amdgcn_sched_barrier(0);
        mx_load<SWIGLU, U>(b0, g, b + 3 < nb ? cur : nxt, b + 3 < nb ? (b + 3) * U : (b + 3 - nb) * U, lane);
        __builtin_amdgcn_sched_barrier(0);
        mx_compute<U>(b1, acc, kb);
        __builtin_amdgcn_sched_barrier(0);
        mx_load<SWIGLU, U>(b1, g, b + 4 < nb ? cur : nxt, b + 4 < nb ? (b + 4) * U : (b + 4 - nb) * U, lane);
        __builtin_amdgcn_sched_barrier(0);
        mx_compute<U>(b2, acc, kb);
        __builtin_amdgcn_sched_barrier(0);
      }
      mx_store<SWIGLU>(g, cur, acc, li, kb);
      cur = nxt;
    }
    return;
  }
  MxBatch<U> b0, b1;
  mx_load<SWIGLU, U>(b0, g, cur, 0, lane);
  for (int id = gw; id < total; id += nw) {
    MxTile nxt = cur;
    if (id + nw < total)
      nxt = mx_tile_at<SWIGLU>(g, tm, id + nw, li, kb);
    else
      nxt.live = 0;  // the batch loaded past the last tile reads nothing
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < nb; b += 2) {
      // batch b+1 -> b1 (the next tile's batch 0 after this tile's last)
      mx_load<SWIGLU, U>(b1, g, b + 1 < nb ? cur : nxt, b + 1 < nb ? (b + 1) * U : 0, lane);
      __builtin_amdgcn_sched_barrier(0);
      mx_compute<U>(b0, acc, kb);
      __builtin_amdgcn_sched_barrier(0);
      if (b + 1 < nb) {
        mx_load<SWIGLU, U>(b0, g, b + 2 < nb ? cur : nxt, b + 2 < nb ? (b + 2) * U : 0, lane);
        __builtin_amdgcn_sched_barrier(0);
        mx_compute<U>(b1, acc, kb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mx_store<SWIGLU>(g, cur, acc, li, kb);
    if (nb & 1) b0 = b1;  // an odd batch count left the next tile's first batch in b1
    cur = nxt;
  }
}

// ----------------------------------------------------------- launchers ----

static inline long long mx_tiles_bound(const GroupedGemm& g, int n_tiles) {
  const int groups = g.offsets ? g.G : 1;
  return ((long long)(g.total_rows + 15) / 16 + groups) * n_tiles;
}

// The buffer descriptors address one expert matrix with 32-bit offsets.
static inline bool mx_matrix_fits(const GroupedGemm& g, bool swiglu) {
  const long long rows = swiglu ? 2ll * g.up_off : (long long)g.N;
  return rows * (g.K / 2) < (1ll << 31);
}

template <bool SWIGLU, int U, int D = 2>
static void launch_mx_stream(const GroupedGemm& g, hipStream_t s) {
  const int nt = g.N / (SWIGLU ? 32 : 64);
  auto k = ffn_mx_stream<SWIGLU, U, D>;
  const int grid = resident_grid(reinterpret_cast<const void*>(k), 256, (mx_tiles_bound(g, nt) + 3) / 4);
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, g, nt);
}

// K = H (a multiple of 256): batches of 2 K-steps.  Many rows per expert
// (not streamed) and whole tiles: the LDS-tiled kernel (mx_tiled.hip).
int launch_ffn_up_w4a8(const GroupedGemm& g, bool streamed, hipStream_t s) {
  if (!mx_matrix_fits(g, true)) return -3;  // MOE_ERR_UNSUPPORTED
  if (!streamed && mx_tiled_fits(g, true))
    launch_mx_tiled(g, true, s);
  else if ((g.K / 128) % 2 == 0)
    launch_mx_stream<true, 2>(g, s);
  else
    launch_mx_stream<true, 1>(g, s);
  return launch_status();
}

// K = I (a multiple of 128); N = H (a multiple of 64).  Single-step batches
// (a tile is only 12 steps at K = 1536).  When the step count is a multiple
// of 3 (I = 1536), three batches rotate (two in flight while one computes;
// 148 registers, three waves per SIMD); otherwise two batches (120
// registers, four waves per SIMD).  Many rows per expert and K a multiple of
// 512: the LDS-tiled kernel.
int launch_ffn_down_w4a8(const GroupedGemm& g, bool streamed, hipStream_t s) {
  if (!mx_matrix_fits(g, false)) return -3;  // MOE_ERR_UNSUPPORTED
  if (!streamed && mx_tiled_fits(g, false))
    launch_mx_tiled(g, false, s);
  else if ((g.K / 128) % 3 == 0)
    launch_mx_stream<false, 1, 3>(g, s);
  else
    launch_mx_stream<false, 1>(g, s);
  return launch_status();
}

}  // namespace moe
