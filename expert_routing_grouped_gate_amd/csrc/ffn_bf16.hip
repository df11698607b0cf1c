// S5/S6: grouped expert GEMMs in bf16 with fp32 accumulation on MFMA
// ([Qwen3] "GMM enablement and routing optimisation": one grouped matmul
// over all experts instead of a per-expert loop; "MoE TP optimisation ->
// compute decomposition": w13 = gate rows then up rows, SwiGLU =
// SiLU(first half) * second half, fused here into the GEMM1 epilogue).
//
// Tiles are scheduled on the device from the routing offsets (TileMap): a
// persistent grid of resident blocks walks the real tile list, whose length
// every block computes from the offsets.  Nothing is read back to the host,
// so the launch is graph-capturable.
//
// Two tile shapes of one scheduling scheme:
//  * skinny (few rows per expert: decode).  A block covers 16 rows; each
//    wave streams 16 weight rows (SwiGLU: 16 gate + 16 up rows) straight
//    from HBM into MFMA operand registers (each weight byte is used once),
//    double-buffered in batches of U K-steps; waves may split K and reduce
//    in LDS.
//  * tiled (many rows per expert: prefill).  128 x 128 block tile, K step 64,
//    both operands staged through double-buffered, XOR-swizzled LDS; 2 x 2
//    waves each own a 64 x 64 sub-tile of 16x16x32 MFMAs; the epilogue goes
//    through LDS so global stores are 16-byte and row-contiguous.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

__device__ __forceinline__ float silu_f32(float g) { return g / (1.f + expf(-g)); }

// ------------------------------------------------------------- skinny -----
template <bool SWIGLU, int WN, int WK, int U>
__device__ __forceinline__ void skinny_tile(const GroupedGemm& g, int lane, int wn, int wk,
                                            int n_tile, int grp, int row0, int nrows) {
  const int li = lane & 15;        // weight row (A operand) / activation row (B operand)
  const int kq = (lane >> 4) * 8;  // this lane's 8 k values inside a 32-step
  const int n0 = n_tile * 16 * WN + wn * 16;
  const int r = row0 + min(li, nrows - 1);  // rows past the tile end reuse a valid row
  const int arow = g.gather ? g.sorted_pair[r] / g.topk : r;
  const int K = g.K;
  const int Kw = K / WK;
  const int kbeg = wk * Kw;
  const uint16_t* Ap = static_cast<const uint16_t*>(g.A) + (size_t)arow * K + kbeg + kq;
  const uint16_t* Wp = static_cast<const uint16_t*>(g.W) + (size_t)grp * g.w_gstride +
                       (size_t)(n0 + li) * K + kbeg + kq;
  const size_t upoff = (size_t)g.up_off * K;

  f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = Kw / 32;
  // Two register batches of U K-steps: the loads of batch b+1 are issued
  // before the MFMAs of batch b (the scheduling barrier keeps the compiler
  // from interleaving them), so up to 2U steps of loads are in flight.
  u32x4 wa0[U], wb0[U], xa0[U], wa1[U], wb1[U], xa1[U];
  auto issue = [&](u32x4* wa, u32x4* wb, u32x4* xa, int st) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wa[u] = ld16_stream(Wp + (st + u) * 32);
      if (SWIGLU) wb[u] = ld16_stream(Wp + upoff + (st + u) * 32);
      xa[u] = ld16(Ap + (st + u) * 32);
    }
  };
  auto compute = [&](const u32x4* wa, const u32x4* wb, const u32x4* xa) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      accg = mfma16x16x32(wa[u], xa[u], accg);
      if (SWIGLU) accu = mfma16x16x32(wb[u], xa[u], accu);
    }
  };
  const int nb = nsteps / U;
  if (nb > 0) issue(wa0, wb0, xa0, 0);
  for (int b = 0; b < nb; b += 2) {
    if (b + 1 < nb) issue(wa1, wb1, xa1, (b + 1) * U);
    __builtin_amdgcn_sched_barrier(0);
    compute(wa0, wb0, xa0);
    if (b + 1 < nb) {
      if (b + 2 < nb) issue(wa0, wb0, xa0, (b + 2) * U);
      __builtin_amdgcn_sched_barrier(0);
      compute(wa1, wb1, xa1);
    }
  }
  for (int st = nb * U; st < nsteps; ++st) {
    const u32x4 wa = ld16_stream(Wp + st * 32);
    const u32x4 xa = ld16(Ap + st * 32);
    accg = mfma16x16x32(wa, xa, accg);
    if (SWIGLU) accu = mfma16x16x32(ld16_stream(Wp + upoff + st * 32), xa, accu);
  }

  if (WK > 1) {
    __shared__ f32x4 red[WK > 1 ? WK - 1 : 1][WN][2][64];
    if (wk > 0) {
      red[wk - 1][wn][0][lane] = accg;
      red[wk - 1][wn][1][lane] = accu;
    }
    __syncthreads();
    if (wk != 0) {
      __syncthreads();  // red[] is reused by the next tile
      return;
    }
#pragma unroll
    for (int w = 0; w < WK - 1; ++w) {
      accg += red[w][wn][0][lane];
      accu += red[w][wn][1][lane];
    }
    __syncthreads();
  }

  // D[n][m]: this lane holds activation row li, output columns n0 + 4*(lane>>4) + i
  if (li < nrows) {
    const int nc = n0 + 4 * (lane >> 4);
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = SWIGLU ? silu_f32(accg[i]) * accu[i] : accg[i];
    u32x2 pk;
    pk.x = pack_bf16x2(v[0], v[1]);
    pk.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.out) + (size_t)(row0 + li) * g.N + nc) = pk;
  }
}

template <bool SWIGLU, int WN, int WK, int U>
__global__ __launch_bounds__(64 * WN * WK) void ffn_skinny(GroupedGemm g, int n_tiles) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave % WN;
  const int wk = wave / WN;
  TileMap tm;
  tm.init(g.offsets, g.G, g.ident_rows, 16);
  const int total = tm.total * n_tiles;
  // persistent: block b takes tiles b, b + gridDim.x, ... (gridDim.x % 8 == 0
  // keeps every tile of a block on the block's XCD)
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int id = xcd_remap(t, total);
    const int n_tile = id / tm.total;
    int grp, row0, nrows;
    tm.find(id - n_tile * tm.total, grp, row0, nrows);
    skinny_tile<SWIGLU, WN, WK, U>(g, lane, wn, wk, n_tile, grp, row0, nrows);
  }
}

// -------------------------------------------------------------- tiled -----
constexpr int TBM = 128, TBN = 128, TBK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

template <bool SWIGLU>
__device__ __forceinline__ void tiled_tile(const GroupedGemm& g, u32x4 (*smem)[(TBM + TBN) * 8],
                                           int n_tile, int grp, int row0, int nrows) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  constexpr int BNOUT = SWIGLU ? TBN / 2 : TBN;
  const int n0 = n_tile * BNOUT;
  const int K = g.K;
  const uint16_t* Wg = static_cast<const uint16_t*>(g.W) + (size_t)grp * g.w_gstride;

  // global -> LDS assignment: 4 A chunks and 4 B chunks of 16 B per thread
  const uint16_t* aptr[4];
  const uint16_t* bptr[4];
  const int lchunk = tid & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 3) + 32 * i;
    const int r = row0 + min(row, nrows - 1);
    const int arow = g.gather ? g.sorted_pair[r] / g.topk : r;
    aptr[i] = static_cast<const uint16_t*>(g.A) + (size_t)arow * K + lchunk * 8;
    int wrow;
    if (SWIGLU)
      wrow = row < 64 ? n0 + row : g.up_off + n0 + (row - 64);
    else
      wrow = n0 + row;
    bptr[i] = Wg + (size_t)wrow * K + lchunk * 8;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ld16(aptr[i] + k0);
      rb[i] = ld16_stream(bptr[i] + k0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 32 * i;
      smem[buf][swz(row, lchunk)] = ra[i];
      smem[buf][swz(TBM + row, lchunk)] = rb[i];
    }
  };

  // fragment rows inside the LDS tile
  int arow_l[4], brow_l[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) arow_l[mi] = wm * 64 + mi * 16 + (lane & 15);
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    int rr;
    if (SWIGLU)
      rr = (ni < 2) ? wn * 32 + ni * 16 : 64 + wn * 32 + (ni - 2) * 16;
    else
      rr = wn * 64 + ni * 16;
    brow_l[ni] = TBM + rr + (lane & 15);
  }
  const int kc = lane >> 4;

  const int nk = K / TBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * TBK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 af[4], bfr[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) af[mi] = smem[buf][swz(arow_l[mi], ks * 4 + kc)];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) bfr[ni] = smem[buf][swz(brow_l[ni], ks * 4 + kc)];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma16x16x32(af[mi], bfr[ni], acc[mi][ni]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue through LDS: C tile [128][BNOUT] bf16, rows padded by 16 B
  constexpr int CST = BNOUT + 8;  // elements per LDS row
  uint16_t* ct = reinterpret_cast<uint16_t*>(&smem[0][0]);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 64 + mi * 16 + 4 * (lane >> 4) + i;
      if (SWIGLU) {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          const int n = wn * 32 + gi * 16 + (lane & 15);
          const float a = silu_f32(acc[mi][gi][i]) * acc[mi][gi + 2][i];
          ct[m * CST + n] = (uint16_t)f32_to_bf16(a);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int n = wn * 64 + ni * 16 + (lane & 15);
          ct[m * CST + n] = (uint16_t)f32_to_bf16(acc[mi][ni][i]);
        }
      }
    }
  }
  __syncthreads();
  constexpr int CPR = BNOUT / 8;  // 16-byte chunks per row
  uint16_t* out = static_cast<uint16_t*>(g.out);
  for (int idx = tid; idx < TBM * CPR; idx += 256) {
    const int row = idx / CPR, c = idx - row * CPR;
    if (row < nrows)
      *reinterpret_cast<u32x4*>(out + (size_t)(row0 + row) * g.N + n0 + c * 8) =
          *reinterpret_cast<const u32x4*>(ct + row * CST + c * 8);
  }
  __syncthreads();  // the next tile overwrites the LDS
}

template <bool SWIGLU>
__global__ __launch_bounds__(256, 2) void ffn_tiled(GroupedGemm g, int n_tiles) {
  // [buffer][A rows 0..127 | B rows 128..255][8 chunks of 16 B]
  __shared__ u32x4 smem[2][(TBM + TBN) * 8];
  TileMap tm;
  tm.init(g.offsets, g.G, g.ident_rows, TBM);
  const int total = tm.total * n_tiles;
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int id = xcd_remap(t, total);
    const int n_tile = id / tm.total;
    int grp, row0, nrows;
    tm.find(id - n_tile * tm.total, grp, row0, nrows);
    tiled_tile<SWIGLU>(g, smem, n_tile, grp, row0, nrows);
  }
}

// ----------------------------------------------------------- launchers ----
// Persistent grids: (resident blocks per CU) x (CUs), a multiple of 8, capped
// by an upper bound of the tile count.
template <typename Kern>
static int persistent_grid(Kern kernel, int block, long long max_tiles) {
  static int cache[64];  // per device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, block, 0) != hipSuccess || occ <= 0)
      occ = 1;
    cache[dev] = ((cus * occ + 7) / 8) * 8;
  }
  long long cap = ((max_tiles + 7) / 8) * 8;
  return (int)(cap < cache[dev] ? cap : cache[dev]);
}

static inline long long tiles_bound(const GroupedGemm& g, int BM, int n_tiles) {
  const int groups = g.offsets ? g.G : 1;
  return ((long long)(g.total_rows + BM - 1) / BM + groups) * n_tiles;
}

template <bool SWIGLU, int WN, int WK, int U>
static void launch_skinny(const GroupedGemm& g, hipStream_t s) {
  const int nt = g.N / (16 * WN);
  auto k = ffn_skinny<SWIGLU, WN, WK, U>;
  const int grid = persistent_grid(k, 64 * WN * WK, tiles_bound(g, 16, nt));
  hipLaunchKernelGGL(k, dim3(grid), dim3(64 * WN * WK), 0, s, g, nt);
}

template <bool SWIGLU>
static void launch_tiled(const GroupedGemm& g, hipStream_t s) {
  const int nt = g.N / (SWIGLU ? TBN / 2 : TBN);
  auto k = ffn_tiled<SWIGLU>;
  const int grid = persistent_grid(k, 256, tiles_bound(g, TBM, nt));
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, g, nt);
}

int launch_ffn_up_bf16(const GroupedGemm& g, bool small_m, hipStream_t s) {
  if (small_m)
    launch_skinny<true, 1, 4, 4>(g, s);
  else
    launch_tiled<true>(g, s);
  return launch_status();
}

int launch_ffn_down_bf16(const GroupedGemm& g, bool small_m, hipStream_t s) {
  if (small_m)
    launch_skinny<false, 4, 1, 4>(g, s);
  else
    launch_tiled<false>(g, s);
  return launch_status();
}

}  // namespace moe
