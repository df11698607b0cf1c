// Shared device helpers for the gfx950 MoE kernels: bf16 conversion, wave
// reductions, the XCD-aware block order and the device-side ragged tile
// scheduler used by every grouped GEMM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even, on the gfx950 convert instruction
// (v_cvt_pk_bf16_f32: one instruction per pair; a NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// 16-byte load of the weight stream.  Plain cached loads: the MFMA operand
// layout reads each 128-byte line in two halves, and non-temporal loads
// (which let the first half's line be evicted early) measured ~11% slower.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16].
// Lane l supplies A row (l % 16), B column (l % 16), and the 8 consecutive
// k values 8*(l/16) .. 8*(l/16)+7 of each.  D: lane l holds column (l % 16),
// rows 4*(l/16) + {0,1,2,3}.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Hardware dispatches block b to XCD (b mod 8).  Give every XCD a contiguous
// range of logical tile ids so that neighbouring tiles (which share weight
// tiles) run on the same XCD and meet in its L2.  Bijective for any count.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int xcd = bid & 7, local = bid >> 3;
  const int base = nblocks >> 3, rem = nblocks & 7;
  return xcd * base + (xcd < rem ? xcd : rem) + local;
}

// Explicit waits and barriers of the LDS-staged GEMMs (DMA ring + MFMA).
// s_waitcnt lgkmcnt(n) only (vmcnt and expcnt left open; gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (N << 8));
}

// s_waitcnt with vmcnt(n), lgkmcnt(0), expcnt left open (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// s_waitcnt vmcnt(n) only (lgkmcnt and expcnt left open).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Make the compiler treat these registers as read here, so that it waits
// for their pending LDS loads at this point (its own, tracked wait).
template <int N>
__device__ __forceinline__ void use_regs(const u32x4* r) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(r[i]));
}

__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Activation row of sorted row r: the token of pair sorted_pair[r] when
// gathering (clamped into [0, rows/topk)), else r itself.
__device__ __forceinline__ int gather_row(const int32_t* __restrict__ sorted_pair, int gather,
                                          int topk, int total_rows, int r) {
  if (!gather) return r;
  const int t = max(sorted_pair[r], 0) / topk;
  return min(t, total_rows / topk - 1);
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Ragged tile scheduler.  Group g owns rows [offsets[g], offsets[g+1]) and
// ceil(rows / BM) consecutive m-tiles.  init() loads the offsets (each lane
// up to 5 consecutive groups, all loads independent), counts the tiles and
// scans them across the wave; find() maps an m-tile index to (group, first
// row, valid rows) from registers only.  When offsets == nullptr there is a
// single group of `ident_rows` rows starting at row 0.  With extra_rows > 0
// one more group G follows the G groups of `offsets`: rows [offsets[G],
// offsets[G] + extra_rows) (the shared expert run in the same launch).
// Every lane of the wave holds the same results; no LDS and no barrier are
// used.
struct TileMap {
  int per, gbeg, excl, total, BM;
  int o[6];      // offsets[gbeg .. gbeg + per] (clamped)
  int tiles[5];
  const int* offsets;
  int ident_rows;

  // Offsets are clamped to [0, max_rows] (max_rows: rows the output can
  // hold), so even malformed offsets yield tiles inside the buffers.
  __device__ __forceinline__ void init(const int* __restrict__ offs, int G, int ident, int bm,
                                       int max_rows, int extra_rows = 0) {
    offsets = offs;
    ident_rows = ident;
    BM = bm;
    if (offs == nullptr) {
      total = (ident + bm - 1) / bm;
      return;
    }
    const int lane = threadIdx.x & 63;
    const int Gt = G + (extra_rows > 0 ? 1 : 0);
    per = (Gt + 63) >> 6;
    gbeg = lane * per;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int j = gbeg + i;
      o[i] = min(max(offs[min(j, G)], 0), max_rows) + (j > G ? extra_rows : 0);
    }
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int t = (i < per && gbeg + i < Gt) ? max(o[i + 1] - o[i] + bm - 1, 0) / bm : 0;
      tiles[i] = t;
      sum += t;
    }
    const int incl = wave_incl_scan(sum);
    excl = incl - sum;
    total = __shfl(incl, 63, 64);
  }

  // m-tile index mt < total -> group, first row, rows in the tile
  __device__ __forceinline__ void find(int mt, int& g_out, int& row0, int& nrows) const {
    if (offsets == nullptr) {
      g_out = 0;
      row0 = mt * BM;
      nrows = min(BM, ident_rows - row0);
      return;
    }
    const int lane = threadIdx.x & 63;
    const bool mine = mt >= excl && mt < excl + (tiles[0] + tiles[1] + tiles[2] + tiles[3] + tiles[4]);
    const unsigned long long bal = __ballot(mine);
    const int src = __ffsll((long long)bal) - 1;
    int g = 0, r0 = 0, nr = 0;
    if (lane == src) {
      int s = excl;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        if (mt >= s && mt < s + tiles[i]) {
          g = gbeg + i;
          r0 = o[i] + (mt - s) * BM;
          nr = min(BM, o[i + 1] - r0);
        }
        s += tiles[i];
      }
    }
    g_out = __shfl(g, src, 64);
    row0 = __shfl(r0, src, 64);
    nrows = __shfl(nr, src, 64);
  }

  // The group owning m-tile q: its index, first m-tile, m-tile count, first
  // row and end row.
  __device__ __forceinline__ void find_group(int q, int& g_out, int& first_mt, int& n_mt,
                                             int& grow0, int& grow1) const {
    if (offsets == nullptr) {
      g_out = 0;
      first_mt = 0;
      n_mt = total;
      grow0 = 0;
      grow1 = ident_rows;
      return;
    }
    const int lane = threadIdx.x & 63;
    const bool mine = q >= excl && q < excl + (tiles[0] + tiles[1] + tiles[2] + tiles[3] + tiles[4]);
    const unsigned long long bal = __ballot(mine);
    const int src = __ffsll((long long)bal) - 1;
    int g = 0, f = 0, n = 0, a = 0, b = 0;
    if (lane == src) {
      int s = excl;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        if (q >= s && q < s + tiles[i]) {
          g = gbeg + i;
          f = s;
          n = tiles[i];
          a = o[i];
          b = o[i + 1];
        }
        s += tiles[i];
      }
    }
    g_out = __shfl(g, src, 64);
    first_mt = __shfl(f, src, 64);
    n_mt = __shfl(n, src, 64);
    grow0 = __shfl(a, src, 64);
    grow1 = __shfl(b, src, 64);
  }
};

// TileMap's per-lane state, parked in LDS between the tiles of a persistent
// block so that it costs no registers during a K loop: kTileMapWords words per
// lane, `slot` = this wave's [kTileMapWords][64] ints.  Parked only when the
// map has groups (offsets != nullptr); the identity map needs nothing.
constexpr int kTileMapWords = 13;

__device__ __forceinline__ void park_tilemap(const TileMap& tm, int* slot) {
  int* mine = slot + (threadIdx.x & 63);
  mine[0] = tm.excl;
  mine[64] = tm.gbeg;
#pragma unroll
  for (int i = 0; i < 5; ++i) mine[64 * (2 + i)] = tm.tiles[i];
#pragma unroll
  for (int i = 0; i < 6; ++i) mine[64 * (7 + i)] = tm.o[i];
}

__device__ __forceinline__ TileMap unpark_tilemap(const int* slot, const int* offsets,
                                                  int ident_rows, int total, int BM) {
  TileMap tl;
  tl.offsets = offsets;
  tl.ident_rows = ident_rows;
  tl.total = total;
  tl.BM = BM;
  if (offsets != nullptr) {
    const int* mine = slot + (threadIdx.x & 63);
    tl.excl = mine[0];
    tl.gbeg = mine[64];
#pragma unroll
    for (int i = 0; i < 5; ++i) tl.tiles[i] = mine[64 * (2 + i)];
#pragma unroll
    for (int i = 0; i < 6; ++i) tl.o[i] = mine[64 * (7 + i)];
  }
  return tl;
}

// One output tile of a grouped GEMM (wave-uniform); grow0 = its group's
// first row.
struct TileRef {
  int grp, n_tile, row0, nrows, grow0;
};

// Tile `id` (after xcd_remap) of the expert-major order: group, then n-tile,
// then the group's m-tiles.  The m-tiles that share a weight tile are
// neighbours (they start together and the weight tile streams through L2
// once), and a group's tiles stay on one XCD.
__device__ __forceinline__ TileRef expert_major_tile(const TileMap& tl, int id, int n_tiles) {
  int grp, first_mt, n_mt, grow0, grow1;
  tl.find_group(id / n_tiles, grp, first_mt, n_mt, grow0, grow1);
  const int local = id - first_mt * n_tiles;
  const int n_tile = local / n_mt;
  const int row0 = grow0 + (local - n_tile * n_mt) * tl.BM;
  TileRef r;
  r.grp = __builtin_amdgcn_readfirstlane(grp);
  r.n_tile = __builtin_amdgcn_readfirstlane(n_tile);
  r.row0 = __builtin_amdgcn_readfirstlane(row0);
  r.nrows = __builtin_amdgcn_readfirstlane(min(tl.BM, grow1 - row0));
  r.grow0 = __builtin_amdgcn_readfirstlane(grow0);
  return r;
}

}  // namespace moe
