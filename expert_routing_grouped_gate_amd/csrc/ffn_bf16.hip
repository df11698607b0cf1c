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
//  * tiled (many rows per expert: prefill).  128 x 256 block tile (256
//    weight rows), K step 64, both operands staged through double-buffered,
//    XOR-swizzled LDS; 2 x 2 waves each own a 64 x 128 sub-tile of 16x16x32
//    MFMAs (the larger wave tile halves LDS reads per MFMA against 64 x 64);
//    the epilogue goes through LDS so global stores are 16-byte and
//    row-contiguous.
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
  const int arow = gather_row(g.sorted_pair, g.gather, g.topk, g.total_rows, r);
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
  tm.init(g.offsets, g.G, g.ident_rows, 16, g.total_rows);
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
// Block tile BM x BN (BN weight rows; with SwiGLU the first BN/2 are gate
// rows n0.., the last BN/2 the matching up rows), K step 64, WM x WN waves,
// each owning a (BM/WM) x (BN/WN) sub-tile of 16x16x32 MFMAs.  Operands are
// staged through two XOR-swizzled LDS buffers: the global loads of step k+1
// are in flight while step k computes.
constexpr int TBK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

template <bool SWIGLU, int BM, int BN, int WM, int WN, int NS>
struct Tiled {
  static constexpr int NW = WM * WN;
  static constexpr int NTHR = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int MT = TM / 16, NT = TN / 16;
  static constexpr int BNOUT = SWIGLU ? BN / 2 : BN;
  static constexpr int STAGE = (BM + BN) * 8;  // u32x4 entries per LDS stage
  static constexpr int NSTAGE = NS;  // LDS stages; NS - 1 K-steps in flight
  static constexpr int LPW = (BM + BN) / 8 / NW;  // 1 KB loads per wave per stage
  static_assert((BM + BN) % (8 * NW) == 0, "row groups split evenly over waves");
  static_assert(!SWIGLU || NT % 2 == 0, "gate/up pairs");
  static_assert(BM * (BNOUT + 8) * 2 <= NSTAGE * STAGE * 16, "epilogue tile fits");
};

// One output tile.  LDS holds NSTAGE stages of [A rows 0..BM-1 | B rows
// BM..BM+BN-1] x 8 chunks of 16 B (one K step of 64), chunk c of row r stored
// at c ^ (r & 7).  Stages are filled by global_load_lds_dwordx4: each wave
// instruction writes 1 KB = 8 rows, lane l taking row l/8, physical chunk
// l%8, so it loads logical chunk (l%8) ^ (l/8).  Step k+2 is in flight while
// step k computes; waits are explicit (vmcnt counts this wave's DMA loads)
// and the block barrier carries no memory fence, so the loads of the next
// step stay in flight across it.
template <bool SWIGLU, int BM, int BN, int WM, int WN, int NS>
__device__ __forceinline__ void tiled_tile(const GroupedGemm& g, u32x4* smem, int n_tile, int grp,
                                           int row0, int nrows) {
  using C = Tiled<SWIGLU, BM, BN, WM, WN, NS>;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int n0 = n_tile * C::BNOUT;
  const int K = g.K;
  const uint16_t* Wg = static_cast<const uint16_t*>(g.W) + (size_t)grp * g.w_gstride;

  const uint16_t* src[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int rg = wave + C::NW * i;
    const int row = rg * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (lane >> 3);
    if (row < BM) {
      const int r = row0 + min(row, nrows - 1);
      const int arow = gather_row(g.sorted_pair, g.gather, g.topk, g.total_rows, r);
      src[i] = static_cast<const uint16_t*>(g.A) + (size_t)arow * K + c * 8;
    } else {
      const int br = row - BM;
      int wrow;
      if (SWIGLU)
        wrow = br < BN / 2 ? n0 + br : g.up_off + n0 + (br - BN / 2);
      else
        wrow = n0 + br;
      src[i] = Wg + (size_t)wrow * K + c * 8;
    }
  }
  auto issue = [&](int buf, int k0) {
    u32x4* st = smem + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int rg = wave + C::NW * i;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src[i] + k0),
          (__attribute__((address_space(3))) void*)(st + rg * 64), 16, 0, 0);
    }
  };

  f32x4 acc[C::MT][C::NT];
#pragma unroll
  for (int a = 0; a < C::MT; ++a)
#pragma unroll
    for (int b = 0; b < C::NT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  int arow_l[C::MT], brow_l[C::NT];
#pragma unroll
  for (int mi = 0; mi < C::MT; ++mi) arow_l[mi] = wm * C::TM + mi * 16 + (lane & 15);
#pragma unroll
  for (int ni = 0; ni < C::NT; ++ni) {
    int rr;
    if (SWIGLU)
      rr = (ni < C::NT / 2) ? wn * (C::TN / 2) + ni * 16
                            : BN / 2 + wn * (C::TN / 2) + (ni - C::NT / 2) * 16;
    else
      rr = wn * C::TN + ni * 16;
    brow_l[ni] = BM + rr + (lane & 15);
  }
  const int kc = lane >> 4;

  // Software pipeline over half-steps (K = 32): the fragments of the next
  // half-step are read from LDS while the MFMAs of the current one run.
  // Iteration k: read stage k's second half -> F1; MFMAs on F0 (first half);
  // wait for this wave's DMA of stage k+1; barrier (stage k+1 is complete for
  // every wave and stage k's buffer is free); DMA of stage k+NS into stage
  // k's buffer; read stage k+1's first half -> F0; MFMAs on F1.
  static_assert(NS >= 2, "at least two stages");
  const int nk = K / TBK;
#pragma unroll
  for (int p = 0; p < NS; ++p)
    if (p < nk) issue(p, p * TBK);
  u32x4 af0[C::MT], bf0[C::NT], af1[C::MT], bf1[C::NT];
  auto read_frags = [&](u32x4* af, u32x4* bfr, int b, int ks) {
    const u32x4* st = smem + b * C::STAGE;
#pragma unroll
    for (int mi = 0; mi < C::MT; ++mi) af[mi] = st[swz(arow_l[mi], ks * 4 + kc)];
#pragma unroll
    for (int ni = 0; ni < C::NT; ++ni) bfr[ni] = st[swz(brow_l[ni], ks * 4 + kc)];
  };
  auto mfmas = [&](const u32x4* af, const u32x4* bfr) {
#pragma unroll
    for (int mi = 0; mi < C::MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < C::NT; ++ni) acc[mi][ni] = mfma16x16x32(af[mi], bfr[ni], acc[mi][ni]);
  };
  // stage 0 ready -> first half into F0
  if (nk > NS - 1)
    wait_vm_lgkm0<(NS - 1) * C::LPW>();
  else
    wait_vm_lgkm0<0>();
  block_barrier();
  read_frags(af0, bf0, 0, 0);
  // retire every scalar load here: with none pending, the LDS reads in the
  // loop can be waited for by count (scalar loads return out of order)
  wait_lgkm<0>();
  int buf = 0;
  for (int kt = 0; kt < nk; ++kt) {
    read_frags(af1, bf1, buf, 1);
    // F0 was requested before F1 and LDS reads complete in order: waiting
    // until at most F1's reads are pending leaves those in flight during the
    // MFMAs below
    wait_lgkm<(C::MT + C::NT < 15 ? C::MT + C::NT : 15)>();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(af0, bf0);
    __builtin_amdgcn_sched_barrier(0);
    // F1's LDS reads must have landed before the barrier (after it, other
    // waves refill stage kt's buffer); this wave's DMA of stage kt+1 must be
    // done; stages kt+2 .. kt+NS-1 may stay in flight
    use_regs<C::MT>(af1);
    use_regs<C::NT>(bf1);
    const int later = min(NS - 2, nk - 2 - kt);
    if (NS >= 3 && later >= 1) {
      if (NS >= 4 && later >= 2)
        wait_vm<2 * C::LPW>();
      else
        wait_vm<C::LPW>();
    } else {
      wait_vm<0>();
    }
    block_barrier();
    if (kt + NS < nk) issue(buf, (kt + NS) * TBK);
    const int nbuf = buf == NS - 1 ? 0 : buf + 1;
    read_frags(af0, bf0, nbuf, 0);  // (stale and unused after the last step)
    __builtin_amdgcn_sched_barrier(0);
    mfmas(af1, bf1);
    __builtin_amdgcn_sched_barrier(0);
    buf = nbuf;
  }
  wait_vm_lgkm0<0>();
  block_barrier();  // every wave is done with the stages before the C tile reuses them

  // epilogue through LDS: C tile [BM][BNOUT] bf16, rows padded by 16 B
  constexpr int CST = C::BNOUT + 8;
  uint16_t* ct = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int mi = 0; mi < C::MT; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * C::TM + mi * 16 + 4 * (lane >> 4) + i;
      if (SWIGLU) {
#pragma unroll
        for (int ni = 0; ni < C::NT / 2; ++ni) {
          const int n = wn * (C::TN / 2) + ni * 16 + (lane & 15);
          const float a = silu_f32(acc[mi][ni][i]) * acc[mi][ni + C::NT / 2][i];
          ct[m * CST + n] = (uint16_t)f32_to_bf16(a);
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < C::NT; ++ni) {
          const int n = wn * C::TN + ni * 16 + (lane & 15);
          ct[m * CST + n] = (uint16_t)f32_to_bf16(acc[mi][ni][i]);
        }
      }
    }
  }
  __syncthreads();
  constexpr int CPR = C::BNOUT / 8;  // 16-byte chunks per row
  uint16_t* out = static_cast<uint16_t*>(g.out);
  for (int idx = tid; idx < BM * CPR; idx += C::NTHR) {
    const int row = idx / CPR, c = idx - row * CPR;
    if (row < nrows)
      *reinterpret_cast<u32x4*>(out + (size_t)(row0 + row) * g.N + n0 + c * 8) =
          *reinterpret_cast<const u32x4*>(ct + row * CST + c * 8);
  }
  __syncthreads();  // the next tile overwrites the LDS
}

template <bool SWIGLU, int BM, int BN, int WM, int WN, int NS, int OCC>
__global__ __launch_bounds__(64 * WM * WN, OCC) void ffn_tiled(GroupedGemm g, int n_tiles) {
  using C = Tiled<SWIGLU, BM, BN, WM, WN, NS>;
  __shared__ u32x4 smem[C::NSTAGE * C::STAGE];
  TileMap tm;
  tm.init(g.offsets, g.G, g.ident_rows, BM, g.total_rows);
  const int total = tm.total * n_tiles;
  // Tile order: expert_major_tile (the ~n_tiles x m-tiles tiles of an expert
  // fit in the concurrent blocks of one XCD, so its gathered activation rows
  // stay in that L2 for all n-tiles).
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const TileRef r = expert_major_tile(tm, xcd_remap(t, total), n_tiles);
    tiled_tile<SWIGLU, BM, BN, WM, WN, NS>(g, smem, r.n_tile, r.grp, r.row0, r.nrows);
  }
}

// ----------------------------------------------------------- launchers ----
// Persistent grids: (resident blocks per CU) x (CUs), a multiple of 8, capped
// by an upper bound of the tile count.

static inline long long tiles_bound(const GroupedGemm& g, int BM, int n_tiles) {
  const int groups = g.offsets ? g.G : 1;
  return ((long long)(g.total_rows + BM - 1) / BM + groups) * n_tiles;
}

template <bool SWIGLU, int WN, int WK, int U>
static void launch_skinny(const GroupedGemm& g, hipStream_t s) {
  const int nt = g.N / (16 * WN);
  auto k = ffn_skinny<SWIGLU, WN, WK, U>;
  const int grid = resident_grid(reinterpret_cast<const void*>(k), 64 * WN * WK, tiles_bound(g, 16, nt));
  hipLaunchKernelGGL(k, dim3(grid), dim3(64 * WN * WK), 0, s, g, nt);
}

template <bool SWIGLU, int BM, int BN, int WM, int WN, int NS, int OCC>
static void launch_tiled(const GroupedGemm& g, hipStream_t s) {
  const int nt = g.N / (SWIGLU ? BN / 2 : BN);
  auto k = ffn_tiled<SWIGLU, BM, BN, WM, WN, NS, OCC>;
  const int grid = resident_grid(reinterpret_cast<const void*>(k), 64 * WM * WN, tiles_bound(g, BM, nt));
  hipLaunchKernelGGL(k, dim3(grid), dim3(64 * WM * WN), 0, s, g, nt);
}

int launch_ffn_up_bf16(const GroupedGemm& g, bool streamed, hipStream_t s) {
  if (streamed)
    launch_skinny<true, 1, 4, 4>(g, s);
  else if (tiled4_fits(g, true))
    launch_tiled4(g, true, s);
  else
    launch_tiled<true, 128, 256, 2, 4, 3, 1>(g, s);
  return launch_status();
}

int launch_ffn_down_bf16(const GroupedGemm& g, bool streamed, hipStream_t s) {
  if (streamed)
    launch_skinny<false, 4, 1, 4>(g, s);
  else if (tiled4_fits(g, false))
    launch_tiled4(g, false, s);
  else
    launch_tiled<false, 128, 256, 2, 4, 3, 1>(g, s);
  return launch_status();
}

}  // namespace moe
