// Tiled W4A8 grouped GEMMs for experts with many rows (prefill): MXFP8
// activations x packed MXFP4 weights on v_mfma_scale_f32_16x16x128_f8f6f4,
// operands staged through an LDS ring filled by DMA (global_load_lds).
//
// [Qwen3] "MoE EP optimisation -> compute decomposition (AllGather scheme,
// W4A8)": the grouped matmuls take MXFP8 activations and MXFP4 weights with
// their block scales; [Hy3] section 5.2: SwiGLU output group-quantised before
// the down projection.  The arithmetic is that of the weight-streaming
// kernels in mx.hip (same operands, same epilogue); only the data movement
// differs: a block computes a 128 x 256 tile (activation rows x weight rows)
// and reads each operand once per tile instead of once per 16 rows.
//
// Block tile: BM = 128 activation rows x BN = 256 weight rows (GEMM1: the
// 128 gate rows n0.. and the matching 128 up rows, 128 output columns;
// GEMM2: 256 output columns), K step 128 (one scaled-MFMA depth).  One LDS
// stage (32 KB) holds
//   [0, 16 KB):  activation rows, 128 B each (one step of E4M3 codes); the
//                16-byte chunk c of row r sits at chunk c ^ (r & 7);
//   [16, 32 KB): the 16 weight blocks of the step, copied unchanged from the
//                packed layout (block = 16 rows x 128 k, lane order), so the
//                A operand of lane l is the 16 bytes at 16 l.
// The E8M0 scales stay in registers: a packed dword per weight group (four
// steps) and 16 bytes per activation row (four steps x four 32-blocks), both
// loaded one quad of steps ahead.
#include "common.hpp"
#include "launch.hpp"
#include "mxfmt.hpp"

#include <type_traits>

namespace moe {

template <bool SWIGLU, int WM, int WN, int NS>
struct MxTiled {
  static constexpr int BM = 128, BN = 256;
  static constexpr int NW = WM * WN, NTHR = 64 * NW;
  static constexpr int MT = BM / 16 / WM;  // activation groups per wave
  static constexpr int NT = BN / 16 / WN;  // weight groups per wave
  static constexpr int BNOUT = SWIGLU ? BN / 2 : BN;
  static constexpr int ABYTES = BM * 128;
  static constexpr int STAGE = ABYTES + (BN / 16) * 1024;  // bytes
  static constexpr int LPA = BM / 8 / NW;   // 1 KB activation loads per wave per stage
  static constexpr int LPB = BN / 16 / NW;  // 1 KB weight loads per wave per stage
  static constexpr int LPW = LPA + LPB;
  static_assert(LPA * NW * 8 == BM && LPB * NW * 16 == BN, "loads split evenly over waves");
  static_assert(!SWIGLU || NT % 4 == 0, "a wave's gate/up groups cover whole 32-column blocks");
  static_assert(NS == 4, "four stages: the stage buffer of step kt is kt % 4");
};

// Make the compiler treat these registers as read here, so that it waits for
// their pending LDS loads at this point (its own, tracked wait).
template <int N>
__device__ __forceinline__ void use_frags(const i32x8* r) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    asm volatile("" ::"v"(r[i].lo));
    asm volatile("" ::"v"(r[i].hi));
  }
}

// Row of the weight matrix holding tile block jb (16 rows each).
template <bool SWIGLU, int BN>
__device__ __forceinline__ int mx_block_row(const GroupedGemm& g, int n0, int jb) {
  if (SWIGLU) return jb < BN / 32 ? n0 + 16 * jb : g.up_off + n0 + 16 * (jb - BN / 32);
  return n0 + 16 * jb;
}

// Tile block used by this wave's weight group ni: GEMM1 waves take NT/2
// consecutive gate blocks and the matching up blocks, GEMM2 waves NT
// consecutive blocks.
template <bool SWIGLU, int NT, int BN>
__device__ __forceinline__ int mx_wave_block(int wn, int ni) {
  if (SWIGLU) return ni < NT / 2 ? wn * (NT / 2) + ni : BN / 32 + wn * (NT / 2) + (ni - NT / 2);
  return wn * NT + ni;
}

// Per-tile state.  The ring streams across tiles: during the last quad of
// K-steps of a tile, once stage u of the ring has been read by every wave, the
// DMA of the next tile's step u goes into it, and the next tile's first scale
// quad is loaded with its step 0; the row gathers of the next tile are issued
// when the current tile starts.  A block's tile sequence is t, t + gridDim.x,
// ... in the expert-major order (the m-tiles that share a weight tile are
// neighbours; an expert's tiles stay on one XCD).
struct MxTileInfo {
  int grp, n0, row0, nrows;  // wave-uniform
};

template <bool SWIGLU, int WM, int WN, int NS>
__global__ __launch_bounds__(64 * WM * WN, 1) void ffn_mx_tiled(GroupedGemm g, int n_tiles) {
  using C = MxTiled<SWIGLU, WM, WN, NS>;
  constexpr int MT = C::MT, NT = C::NT;
  // One LDS array: the ring, then the scheduler's per-lane table (one copy
  // per wave, park_tilemap).  (A second __shared__ variable makes the
  // compiler wait for every outstanding DMA to LDS before each LDS read.)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * C::STAGE + C::NW * kTileMapWords * 64 * 4];
  TileMap tm;
  tm.init(g.offsets, g.G, g.ident_rows, C::BM, g.total_rows);
  const int total = __builtin_amdgcn_readfirstlane(tm.total * n_tiles);
  int t = blockIdx.x;
  if (t >= total) return;  // uniform per block: no barrier is left waiting

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int* const tm_slot = reinterpret_cast<int*>(smem + NS * C::STAGE) + wave * kTileMapWords * 64;
  if (g.offsets != nullptr) park_tilemap(tm, tm_slot);
  const int wm = wave % WM, wn = wave / WM;
  const int li = lane & 15, kb = lane >> 4;
  const int K = g.K, ns = K / 128, nq = ns / 4;  // nq >= 2 (launcher)
  const uint8_t* A = static_cast<const uint8_t*>(g.A);
  const int arows_total = g.gather ? g.total_rows / g.topk : g.total_rows;
  const __amdgpu_buffer_rsrc_t asr = mx_rsrc(g.A_scales, (uint32_t)arows_total * (uint32_t)(K / 32));
  const uint32_t wrows = SWIGLU ? 2u * (uint32_t)g.up_off : (uint32_t)g.N;
  const uint32_t wscale_bytes = wrows / 16u * (uint32_t)nq * 256u;

  auto locate = [&](int tt) {
    const TileMap tl = unpark_tilemap(tm_slot, g.offsets, g.ident_rows, tm.total, C::BM);
    const TileRef r = expert_major_tile(tl, xcd_remap(tt, total), n_tiles);
    MxTileInfo ti;
    ti.grp = r.grp;
    ti.n0 = __builtin_amdgcn_readfirstlane(r.n_tile * C::BNOUT);
    ti.row0 = r.row0;
    ti.nrows = r.nrows;
    return ti;
  };
  // Per-lane rows of a tile, in two halves so that no load result is used
  // right after its load.  gather_issue: the sorted row of each of this lane's
  // LPA DMA rows (activation group ra = wave + NW i, 8 rows; lane l fills row
  // 8 ra + l/8) and MT fragment rows, and with a gather the pair ids stored
  // there, all loads issued together.  gather_finish: adma[i] = byte offset
  // in A of the 16 bytes DMA i reads at step 0 (physical chunk l % 8 holds
  // logical chunk (l % 8) ^ (l / 8)); aoff[mi] = byte offset of the scale row
  // of fragment row mi.  Rows past the tile end reuse a valid row; pair ids
  // are clamped into the token range.
  constexpr int NRAW = C::LPA + MT;
  auto gather_issue = [&](const MxTileInfo& ti, int* raw) {
    int r[NRAW];
#pragma unroll
    for (int i = 0; i < C::LPA; ++i) r[i] = ti.row0 + min(8 * (wave + C::NW * i) + (lane >> 3), ti.nrows - 1);
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) r[C::LPA + mi] = ti.row0 + min(16 * (mi * WM + wm) + li, ti.nrows - 1);
    if (g.gather) {
#pragma unroll
      for (int j = 0; j < NRAW; ++j) raw[j] = g.sorted_pair[r[j]];
    } else {
#pragma unroll
      for (int j = 0; j < NRAW; ++j) raw[j] = r[j];
    }
  };
  // (DMA rows past the tile end get an offset past the end of A: the buffer
  // load returns zeros without touching memory; those rows are never stored.)
  auto gather_finish = [&](const MxTileInfo& ti, const int* raw, uint32_t* adma, uint32_t* aoff) {
    uint32_t arow[NRAW];
#pragma unroll
    for (int j = 0; j < NRAW; ++j)
      arow[j] = g.gather ? (uint32_t)min(max(raw[j], 0) / g.topk, g.total_rows / g.topk - 1)
                         : (uint32_t)raw[j];
#pragma unroll
    for (int i = 0; i < C::LPA; ++i) {
      const bool pad = 8 * (wave + C::NW * i) + (lane >> 3) >= ti.nrows;
      adma[i] = pad ? (uint32_t)arows_total * (uint32_t)K
                    : arow[i] * (uint32_t)K + 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) aoff[mi] = arow[C::LPA + mi] * (uint32_t)(K / 32);
  };
  // DMA of step st of tile ti into stage buffer buf: LPA activation groups
  // and LPB weight blocks of 1 KB per wave, as buffer loads to LDS: the
  // per-lane part of each address is a VGPR that lives for the whole tile
  // (adma[i], or lane*16 for the weights) and the per-step part a scalar
  // offset, so no address register is rebuilt (and reused) every step.
  const __amdgpu_buffer_rsrc_t ar = mx_rsrc(A, (uint32_t)arows_total * (uint32_t)K);
  const uint32_t wbytes = wrows * (uint32_t)(K / 2);
  const uint32_t wlane = (uint32_t)lane * 16u;
  auto issue = [&](const MxTileInfo& ti, const uint32_t* adma, int buf, int st) {
    uint8_t* stg = smem + buf * C::STAGE;
    const __amdgpu_buffer_rsrc_t wr =
        mx_rsrc(static_cast<const uint8_t*>(g.W) + (size_t)ti.grp * g.w_gstride, wbytes);
#pragma unroll
    for (int i = 0; i < C::LPA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ar, (__attribute__((address_space(3))) void*)(stg + (wave + C::NW * i) * 1024), 16,
          adma[i], st * 128, 0, 0);
#pragma unroll
    for (int i = 0; i < C::LPB; ++i) {
      const int q = mx_block_row<SWIGLU, C::BN>(g, ti.n0, wave + C::NW * i) / 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (__attribute__((address_space(3))) void*)(stg + C::ABYTES + (wave + C::NW * i) * 1024),
          16, wlane, (q * ns + st) * 1024, 0, 0);
    }
  };

  // ---- scales (registers) ------------------------------------------------
  // Weight scales: the packed dword of group ni for a quad (byte u = step
  // 4c + u).  Activation scales: 16 bytes per row per quad (word u = the four
  // 32-blocks of step 4c + u), compacted to the byte of this lane's block kb.
  u32x4 as_nxt[MT];     // activation scales of the next quad, as loaded
  uint32_t as_cur[MT];  // byte u: this lane's 32-block (kb) at step 4c + u
  uint32_t ws_cur[NT], ws_nxt[NT];
  auto load_scales = [&](const MxTileInfo& ti, const uint32_t* aoff, int c) {  // quad c
    const __amdgpu_buffer_rsrc_t wsr = mx_rsrc(g.W_scales + (size_t)ti.grp * g.ws_gstride, wscale_bytes);
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) {
      const int q = mx_block_row<SWIGLU, C::BN>(g, ti.n0, mx_wave_block<SWIGLU, NT, C::BN>(wn, ni)) / 16;
      ws_nxt[ni] = __builtin_amdgcn_raw_buffer_load_b32(wsr, lane * 4, (q * nq + c) * 256, 0);
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
      as_nxt[mi] = __builtin_amdgcn_raw_buffer_load_b128(asr, aoff[mi] + 16 * c, 0, 0);
  };
  auto next_quad_scales = [&]() {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      uint32_t v = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) v |= ((as_nxt[mi][u] >> (8 * kb)) & 0xffu) << (8 * u);
      as_cur[mi] = v;
    }
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) ws_cur[ni] = ws_nxt[ni];
  };

  // ---- fragments (LDS -> registers) --------------------------------------
  int aread[MT];  // byte offset of this lane's first activation chunk in a stage
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    const int r = 16 * (mi * WM + wm) + li;
    aread[mi] = r * 128 + 16 * (kb ^ (r & 7));
  }
  int wread[NT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni)
    wread[ni] = C::ABYTES + mx_wave_block<SWIGLU, NT, C::BN>(wn, ni) * 1024 + lane * 16;
  i32x8 af[2][MT];
  u32x4 wf[2][NT];
  auto read_frags = [&](int f, int buf) {
    const uint8_t* stg = smem + buf * C::STAGE;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(stg + aread[mi]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(stg + (aread[mi] ^ 64));
      af[f][mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) wf[f][ni] = *reinterpret_cast<const u32x4*>(stg + wread[ni]);
  };

  MxTileInfo cur = locate(t), nxt = cur;
  uint32_t cur_adma[C::LPA], cur_aoff[MT], nxt_adma[C::LPA], nxt_aoff[MT];
  int nxt_raw[NRAW];
  int c_cur = 0, kt_base = 0;  // current quad and its first step

  // ---- pipeline ------------------------------------------------------------
  // Step kt (stage buffer kt % 4): the fragments of step kt are in registers
  // (read one step earlier); wait until this wave's DMA of stage kt+1 is
  // done; barrier (stage kt+1 complete for every wave, stage kt's buffer read
  // by every wave); DMA into stage kt's buffer (this tile's step kt+4, or in
  // the last quad the next tile's step kt % 4); read step kt+1's fragments;
  // MFMAs of step kt.  Every wait counts only DMA loads (8 per wave and step,
  // issued after the target on every path: two later steps' worth); other
  // loads and stores in between only make it stricter.  The block's last tile
  // streams its own first steps in again as "next" (in-bounds reads that are
  // never used; drained before the block exits), so that the last quad has one
  // form.  Each step is straight-line code: a branch inside would let the
  // MFMAs be moved past the barriers.
  enum { MID = 0, LAST = 1 };
  auto step = [&](f32x4 (&acc)[MT][NT], auto U, auto MODE) {
    constexpr int u = decltype(U)::value;
    constexpr int mode = decltype(MODE)::value;
    constexpr int f = u & 1;
    // this wave's fragment reads of stage kt must land before the barrier
    use_frags<MT>(af[f]);
    use_regs<NT>(wf[f]);
    // stages kt+2, kt+3 (or the next tile's first) may stay in flight; the
    // last step of a tile has no stage to wait for
    if (mode == MID || u < 3) wait_vm<2 * C::LPW>();
    if (mode == MID && u == 3) {
      // This wait has also retired the scale loads of step 0 (issued before
      // the DMA of step 1 of this quad) and the next tile's row loads (issued
      // when this tile started): mark them as read here, so that the
      // compiler's own waits for them (where paths merge) do not drain the ring.
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) asm volatile("" : "+v"(ws_nxt[ni]));
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) asm volatile("" : "+v"(as_nxt[mi]));
#pragma unroll
      for (int j = 0; j < NRAW; ++j) asm volatile("" : "+v"(nxt_raw[j]));
    }
    block_barrier();
    if (mode == MID) {
      issue(cur, cur_adma, u, kt_base + u + 4);
      if (u == 0) load_scales(cur, cur_aoff, c_cur + 1);
    } else {
      issue(nxt, nxt_adma, u, u);
      if (u == 0) load_scales(nxt, nxt_aoff, 0);
    }
    if (mode == MID || u < 3) read_frags(f ^ 1, (u + 1) & 3);
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const uint32_t xsc = (as_cur[mi] >> (8 * u)) & 0xffu;
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
        acc[mi][ni] = mfma_fp4_fp8(wf[f][ni], af[f][mi], (ws_cur[ni] >> (8 * u)) & 0xffu, xsc,
                                   acc[mi][ni]);
    }
    // Issue order: one MFMA, then one of the step's global loads (DMA, and
    // the scale loads at the start of a quad), then one MFMA and two LDS
    // reads, and so on: with one wave per SIMD the memory instructions issue
    // while the matrix core works instead of before it.
    {
#pragma unroll
      for (int i = 0; i < C::LPW + (u == 0 ? MT + NT : 0); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
      }
    }
    if (mode == MID || u < 3) {
#pragma unroll
      for (int i = 0; i < (2 * MT + NT) / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using Mid = std::integral_constant<int, MID>;
  using Last = std::integral_constant<int, LAST>;

  // first tile: its rows, then stage 0, its first scale quad and stages 1..3
  // (the order in which the last quad of a tile starts the next one)
  gather_issue(cur, nxt_raw);
  gather_finish(cur, nxt_raw, cur_adma, cur_aoff);
  issue(cur, cur_adma, 0, 0);
  load_scales(cur, cur_aoff, 0);
#pragma unroll
  for (int p = 1; p < 4; ++p) issue(cur, cur_adma, p, p);

  for (;;) {
    const int tn = t + (int)gridDim.x;
    const bool has_next = tn < total;
    if (has_next) nxt = locate(tn);
    gather_issue(nxt, nxt_raw);  // (the current tile again when there is no next)
    f32x4 acc[MT][NT];  // (scoped to the tile: no accumulator value crosses tiles)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
    // stage 0 of this tile: stages 1..3 were issued after it, and after this
    // tile's first scale quad, which this wait therefore retires as well
    wait_vm<3 * C::LPW>();
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) asm volatile("" : "+v"(ws_nxt[ni]));
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) asm volatile("" : "+v"(as_nxt[mi]));
    next_quad_scales();
    block_barrier();
    read_frags(0, 0);
    for (c_cur = 0; c_cur < nq - 1; ++c_cur) {  // quads 0 .. nq-2
      kt_base = 4 * c_cur;
      step(acc, I0{}, Mid{});
      step(acc, I1{}, Mid{});
      step(acc, I2{}, Mid{});
      step(acc, I3{}, Mid{});
      next_quad_scales();
    }
    kt_base = 4 * c_cur;
    gather_finish(nxt, nxt_raw, nxt_adma, nxt_aoff);
    step(acc, I0{}, Last{});
    step(acc, I1{}, Last{});
    step(acc, I2{}, Last{});
    step(acc, I3{}, Last{});
    // (The accumulators are pinned here so that the last MFMAs are not sunk
    // into the row-guarded stores below.)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) asm volatile("" : "+a"(acc[mi][ni]));

    // ---- epilogue (registers -> global) -----------------------------------
    // D[n][m]: lane (li, kb) holds activation row li of group mi and, for
    // weight group ni, weight rows (= output columns) 4 kb .. 4 kb + 3.
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const int r = 16 * (mi * WM + wm) + li;
      if (SWIGLU) {
#pragma unroll
        for (int b = 0; b < NT / 4; ++b) {
          const f32x4 g0 = acc[mi][2 * b], g1 = acc[mi][2 * b + 1];
          const f32x4 u0 = acc[mi][NT / 2 + 2 * b], u1 = acc[mi][NT / 2 + 2 * b + 1];
          float a[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i] = silu_fast(g0[i]) * u0[i];
            a[4 + i] = silu_fast(g1[i]) * u1[i];
          }
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(a[i]));
          amax = max_lanes_16_32(amax);
          const int e = mx_exponent(amax);
          const float inv = exp2_neg(e);
          const uint32_t lo = e4m3_pack4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
          const uint32_t hi = e4m3_pack4(a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv);
          if (r < cur.nrows) {
            const int col0 = cur.n0 + 16 * (wn * (NT / 2) + 2 * b);
            uint8_t* orow = static_cast<uint8_t*>(g.out) + (size_t)(cur.row0 + r) * g.N;
            *reinterpret_cast<uint32_t*>(orow + col0 + 4 * kb) = lo;
            *reinterpret_cast<uint32_t*>(orow + col0 + 16 + 4 * kb) = hi;
            if (kb == 0)
              g.out_scales[(size_t)(cur.row0 + r) * (g.N / 32) + col0 / 32] = (uint8_t)(e + 127);
          }
        }
      } else {
        // groups (ni, ni + 1): lanes of 16-lane rows kb and kb ^ 1 swap halves
        // (v_permlane16_swap) so that each lane stores 8 consecutive columns
        // (even kb: group ni, odd kb: group ni + 1) with one 16-byte store
        const int odd = kb & 1;
        uint16_t* orow = static_cast<uint16_t*>(g.out) +
                         (size_t)(cur.row0 + min(r, cur.nrows - 1)) * g.N + cur.n0 + 16 * wn * NT +
                         8 * (kb >> 1);
#pragma unroll
        for (int ni = 0; ni < NT; ni += 2) {
          const uint32_t a0 = pack_bf16x2(acc[mi][ni][0], acc[mi][ni][1]);
          const uint32_t a1 = pack_bf16x2(acc[mi][ni][2], acc[mi][ni][3]);
          const uint32_t b0 = pack_bf16x2(acc[mi][ni + 1][0], acc[mi][ni + 1][1]);
          const uint32_t b1 = pack_bf16x2(acc[mi][ni + 1][2], acc[mi][ni + 1][3]);
          const auto s0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
          const auto s1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
          const u32x4 o = odd ? u32x4{s0[0], s1[0], b0, b1} : u32x4{a0, a1, s0[1], s1[1]};
          if (r < cur.nrows) *reinterpret_cast<u32x4*>(orow + 16 * (ni + odd)) = o;
        }
      }
    }
    if (!has_next) {
      wait_vm<0>();  // the repeated first steps: no DMA may outlive the block's LDS
      break;
    }
    t = tn;
    cur = nxt;
#pragma unroll
    for (int i = 0; i < C::LPA; ++i) cur_adma[i] = nxt_adma[i];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) cur_aoff[mi] = nxt_aoff[mi];
  }
}

// Shapes the tiled kernels take: whole 128-column (GEMM1) / 256-column
// (GEMM2) output tiles, K a multiple of 512 (whole quads of steps) with at
// least two quads (the last quad of a tile is peeled off the loop), and
// activation offsets that fit 32 bits.
bool mx_tiled_fits(const GroupedGemm& g, bool swiglu) {
  const long long arows = g.gather ? g.total_rows / g.topk : g.total_rows;
  return g.N % (swiglu ? 128 : 256) == 0 && g.K % 512 == 0 && g.K >= 1024 &&
         arows * g.K < (1ll << 32);
}

template <bool SWIGLU, int WM, int WN, int NS>
static void launch_tiled_impl(const GroupedGemm& g, hipStream_t s) {
  using C = MxTiled<SWIGLU, WM, WN, NS>;
  const int nt = g.N / C::BNOUT;
  const int groups = g.offsets ? g.G : 1;
  const long long bound = ((long long)(g.total_rows + C::BM - 1) / C::BM + groups) * nt;
  auto k = ffn_mx_tiled<SWIGLU, WM, WN, NS>;
  const int grid = resident_grid(reinterpret_cast<const void*>(k), C::NTHR, bound);
  hipLaunchKernelGGL(k, dim3(grid), dim3(C::NTHR), 0, s, g, nt);
}

void launch_mx_tiled(const GroupedGemm& g, bool swiglu, hipStream_t s) {
  if (swiglu)
    launch_tiled_impl<true, 2, 2, 4>(g, s);
  else
    launch_tiled_impl<false, 2, 2, 4>(g, s);
}

}  // namespace moe
