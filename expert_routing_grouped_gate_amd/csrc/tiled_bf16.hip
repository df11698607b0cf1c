// S5/S6 for experts with many rows (prefill): bf16 grouped GEMMs on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation, two waves per SIMD.
//
// [Qwen3] "GMM enablement and routing optimisation": one grouped matmul over
// all experts; "MoE TP optimisation -> compute decomposition": w13 = gate
// rows then up rows, SwiGLU = SiLU(first half) * second half, fused into the
// GEMM1 epilogue.  Same accumulation order as the 8-wave tiled kernels of
// ffn_bf16.hip; SiLU from the hardware exp2 and reciprocal (about an ulp of
// fp32 each, far below the bf16 rounding of the output).
//
// Block tile: BM = 128 activation rows x BN = 256 weight rows (GEMM1: the 128
// gate rows n0.. and the matching 128 up rows, 128 output columns; GEMM2: 256
// output columns), K step 64.  Eight waves (2 x 4, two per SIMD), each a
// 64 x 64 sub-tile of 4 x 4 MFMAs (64 fp32 accumulators per lane).  Copies
// into LDS are issued per wave, and eight issuing waves move more of them
// per CU than four (measured on L2-resident data: ~91 against ~56 B/ns per
// CU); rows stay 128 B per stage, since a 64 B row slice doubles the cache
// lines each 1 KB copy touches and fills the texture address queue.  One LDS
// stage (48 KB) holds the step's 128 activation rows then 256 weight rows,
// 128 B each, the 16-byte chunk c of row r at chunk c ^ (r & 7).  Stages are
// filled by buffer loads to LDS (DMA): each wave instruction writes 1 KB = 8
// rows; lane l takes row l / 8, physical chunk l % 8, so it loads logical
// chunk (l % 8) ^ (l / 8).  The per-lane part of every DMA address is a
// register fixed for the tile (gathered activation rows) or for the whole
// kernel (weight rows); the step and the n-tile go in the scalar offset.
//
// The three LDS stages form one ring over the block's whole sequence of
// K-steps: global step s sits in stage s % 3, and the last three steps of a
// tile DMA the next tile's first three, so the stream never drains between
// tiles.  Fragments are read from LDS a half-step (K = 32) ahead of the
// MFMAs that use them.
//
// Both operands depend on L2 reuse: an expert's m-tiles share each weight
// slab and its n-tiles each activation tile, and the blocks of one XCD run
// neighbouring tiles at once.  Marking either operand's copies non-temporal
// made the kernel 26-35% slower; with half of the weight lines hitting L2 (a
// timing probe) it ran 15% faster, so the weight lines fetched from beyond
// L2 are what the stream waits for.
//
// Epilogue: SwiGLU (GEMM1) and bf16 stores from registers.  GEMM1 stores each
// lane's 8 columns directly (a wave holds 32 output columns: 64-byte row
// slices); GEMM2 passes each wave's 16 x 64 results through 2 KB of LDS past
// the ring so that one store writes 8 whole 128-byte row slices.
#include "common.hpp"
#include "launch.hpp"
#include "mxfmt.hpp"

namespace moe {

template <bool SWIGLU>
struct Tiled4 {
  static constexpr int BM = 128, BN = 256, WM = 2, WN = 4, NW = 8, NTHR = 512;
  static constexpr int MT = BM / 16 / WM;  // activation groups per wave (4)
  static constexpr int NT = BN / 16 / WN;  // weight groups per wave (4)
  static constexpr int BNOUT = SWIGLU ? BN / 2 : BN;
  static constexpr int ABYTES = BM * 128;
  static constexpr int STAGE = (BM + BN) * 128;  // bytes
  static constexpr int NS = 3;
  static constexpr int LPA = BM / 8 / NW;  // 1 KB activation DMAs per wave per stage (2)
  static constexpr int LPB = BN / 8 / NW;  // 1 KB weight DMAs per wave per stage (4)
  static constexpr int LPW = LPA + LPB;
  static_assert(NS * STAGE <= 160 * 1024, "LDS");
};

struct T4Tile {
  int grp, n0, row0, nrows;  // wave-uniform
  int ext, rel0;             // the extra (shared-expert) group; its first row relative to the group
};

// Half-step fragments: MT activation and NT weight operands of 16 B.
template <int MT, int NT>
struct Frags {
  u32x4 a[MT];
  u32x4 b[NT];
};

// GATHER (uniform for a launch, a template parameter so that the two row
// paths never merge: a register loaded on one path and moved on the other
// made the compiler drain every load before the move): activation row of
// sorted row r is the token of pair sorted_pair[r], else r itself.
template <bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(512, 1) void ffn_tiled4(GroupedGemm g, int n_tiles) {
  using C = Tiled4<SWIGLU>;
  constexpr int MT = C::MT, NT = C::NT, NW = C::NW;
  // One LDS array, the ring (a second __shared__ variable makes the compiler
  // wait for every outstanding DMA before each LDS read); the scheduler's
  // table stays in registers.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::NS * C::STAGE + (SWIGLU ? 0 : C::NW * 2048)];
  TileMap tm;
  tm.init(g.offsets, g.G, g.ident_rows, C::BM, g.total_rows, g.xg_rows);
  const int total = __builtin_amdgcn_readfirstlane(tm.total * n_tiles);
  int t = blockIdx.x;
  if (t >= total) return;  // uniform per block: no barrier is left waiting

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves w and w + 4 share a SIMD: they take the two row halves of the
  // same 64 columns, so a half of padding rows idles one wave per SIMD
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int li = lane & 15, kc = lane >> 4;
  const int K = g.K, nk = K / 64;  // nk >= 5 (launcher)
  const uint32_t rowb = 2u * (uint32_t)K;  // bytes per row
  const int arows_total = GATHER ? g.total_rows / g.topk : g.total_rows;
  const __amdgpu_buffer_rsrc_t ar = mx_rsrc(g.A, (uint32_t)arows_total * rowb);
  // the extra group's activations (identity rows, no gather)
  const __amdgpu_buffer_rsrc_t arx = mx_rsrc(g.xg_rows > 0 ? g.xg_A : g.A, (uint32_t)g.xg_rows * rowb);
  const uint32_t wrows = SWIGLU ? 2u * (uint32_t)g.up_off : (uint32_t)g.N;
  const uint32_t wbytes = wrows * rowb;
  const uint32_t dchunk = 16u * (uint32_t)((lane & 7) ^ (lane >> 3));

  auto locate = [&](int tt) {
    const TileRef r = expert_major_tile(tm, xcd_remap(tt, total), n_tiles);
    T4Tile ti;
    ti.grp = r.grp;
    ti.n0 = __builtin_amdgcn_readfirstlane(r.n_tile * C::BNOUT);
    ti.row0 = r.row0;
    ti.nrows = r.nrows;
    ti.ext = __builtin_amdgcn_readfirstlane(g.xg_rows > 0 && r.grp == g.G ? 1 : 0);
    ti.rel0 = __builtin_amdgcn_readfirstlane(r.row0 - r.grow0);
    return ti;
  };
  // Activation rows of this lane's LPA DMAs (group ra = wave + NW i, 8 rows;
  // lane l fills row 8 ra + l / 8), in two halves so that no loaded value is
  // used right after its load: gather_issue loads the pair ids (rows past the
  // tile end reuse a valid row), gather_finish turns them into byte offsets
  // of the rows' step-0 chunk (pair ids clamped into the token range).  The
  // extra group's rows are its own row indices (the pair ids loaded for them,
  // from a clamped index, go unused: selects, not branches, keep the two
  // kinds of tile on one path).
  auto tile_rows = [&](const T4Tile& ti, int* r) {
#pragma unroll
    for (int i = 0; i < C::LPA; ++i) r[i] = ti.row0 + min(8 * (wave + NW * i) + (lane >> 3), ti.nrows - 1);
  };
  auto gather_issue = [&](const T4Tile& ti, int* raw) {
    if (GATHER) {
      int r[C::LPA];
      tile_rows(ti, r);
#pragma unroll
      for (int i = 0; i < C::LPA; ++i) raw[i] = g.sorted_pair[min(r[i], g.total_rows - 1)];
    }
  };
  // Rows past the tile end get an offset past the end of A: the buffer load
  // returns zeros without touching memory (those rows are never stored).
  const uint32_t a_oob = (uint32_t)arows_total * rowb;
  const uint32_t ax_oob = (uint32_t)g.xg_rows * rowb;
  auto gather_finish = [&](const T4Tile& ti, const int* raw, uint32_t* adma) {
    int r[C::LPA];
    tile_rows(ti, r);
#pragma unroll
    for (int i = 0; i < C::LPA; ++i) {
      const uint32_t arow = GATHER ? (uint32_t)min(max(raw[i], 0) / g.topk, arows_total - 1)
                                   : (uint32_t)r[i];
      const uint32_t xrow = (uint32_t)(r[i] - ti.row0 + ti.rel0);
      const bool pad = 8 * (wave + NW * i) + (lane >> 3) >= ti.nrows;
      adma[i] = pad ? (ti.ext ? ax_oob : a_oob) : (ti.ext ? xrow : arow) * rowb + dchunk;
    }
  };
  // Weight rows of this lane's LPB DMAs relative to the tile's n0 (group rb =
  // wave + NW i of the 256 tile rows; GEMM1: rows 0..127 gate, 128..255 up).
  uint32_t wdma[C::LPB];
#pragma unroll
  for (int i = 0; i < C::LPB; ++i) {
    const int br = 8 * (wave + NW * i) + (lane >> 3);
    const uint32_t row = SWIGLU ? (br < C::BN / 2 ? (uint32_t)br : (uint32_t)(g.up_off + br - C::BN / 2))
                                : (uint32_t)br;
    wdma[i] = row * rowb + dchunk;
  }
  const uint16_t* Wbase = static_cast<const uint16_t*>(g.W);
  // DMA of step st of tile ti into stage buf.  (The builtin's offsets are
  // int: an unsigned argument made the host pass drop the kernel's stub.)
  auto issue = [&](const T4Tile& ti, const uint32_t* adma, int buf, int st) {
    uint8_t* stg = smem + buf * C::STAGE;
    const __amdgpu_buffer_rsrc_t wr =
        mx_rsrc(ti.ext ? g.xg_W : static_cast<const void*>(Wbase + (size_t)ti.grp * g.w_gstride), wbytes);
    const __amdgpu_buffer_rsrc_t a_r = ti.ext ? arx : ar;
    const uint32_t aso = (uint32_t)st * 128u;
    const uint32_t wso = (uint32_t)ti.n0 * rowb + aso;
#pragma unroll
    for (int i = 0; i < C::LPA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_r, (__attribute__((address_space(3))) void*)(stg + (wave + NW * i) * 1024), 16, (int)adma[i],
          (int)aso, 0, 0);
#pragma unroll
    for (int i = 0; i < C::LPB; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (__attribute__((address_space(3))) void*)(stg + C::ABYTES + (wave + NW * i) * 1024), 16,
          (int)wdma[i], (int)wso, 0, 0);
  };

  // Fragment offsets in a stage for half-step h: activation row
  // 64 wm + 16 mi + li, weight tile row (GEMM1) 64 wn + 16 ni + li for the
  // gate groups ni < 4 and 128 + 64 wn + 16 (ni - 4) + li for the up groups,
  // (GEMM2) 128 wn + 16 ni + li; 16-byte chunk 4 h + kc of the row.  Rows are
  // multiples of 8 apart, so every row of a lane has the same swizzle.
  int aoff[2], boff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ch = 16 * ((4 * h + kc) ^ (li & 7));
    aoff[h] = (64 * wm + li) * 128 + ch;
    boff[h] = C::ABYTES + ((SWIGLU ? C::BN / 2 : C::BN) / C::WN * wn + li) * 128 + ch;
  }
  auto bgroup = [](int ni) {
    if (SWIGLU) return ni < NT / 2 ? ni * 2048 : (C::BN / 2) * 128 + (ni - NT / 2) * 2048;
    return ni * 2048;
  };
  auto read_half = [&](Frags<MT, NT>& f, int buf, int h) {
    const uint8_t* stg = smem + buf * C::STAGE;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) f.a[mi] = *reinterpret_cast<const u32x4*>(stg + aoff[h] + mi * 2048);
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) f.b[ni] = *reinterpret_cast<const u32x4*>(stg + boff[h] + bgroup(ni));
  };

  T4Tile cur = locate(t), nxt = cur;
  uint32_t cur_adma[C::LPA], nxt_adma[C::LPA];
  int nxt_raw[C::LPA] = {};
  Frags<MT, NT> f0, f1;
  int buf = 0;  // stage of the current step (global step % 3)

  // One K-step.  On entry f0 holds the first half-step of the step's stage
  // `buf`.  Read the second half into f1 while f0's MFMAs run; wait for this
  // wave's DMA of the next stage (the one after it may stay in flight) and
  // for f1; barrier (the next stage is complete for every wave, this stage
  // has been read by every wave); DMA (ti, st) into this stage; read the next
  // stage's first half into f0 while f1's MFMAs run.  Every wait counts only
  // DMA loads (LPW per wave and step, one step's worth issued after the
  // target on every path); other loads and stores in between only make it
  // stricter.
  //
  // A wave whose 64 rows of the current tile are all padding (an expert's
  // last, partial m-tile) skips the MFMAs and the second-half reads: it keeps
  // its share of the DMA, the waits and the barrier, and reads the next first
  // half like every wave, so both kinds of step leave the same state behind.
  bool act = true;  // this wave's 64 rows hold valid rows of the current tile
  auto step = [&](f32x4 (&acc)[MT][NT], const T4Tile& ti, const uint32_t* adma, int st) {
    if (!act) {
      wait_vm<C::LPW>();
      block_barrier();
      issue(ti, adma, buf, st);
      buf = buf == C::NS - 1 ? 0 : buf + 1;
      read_half(f0, buf, 0);
      return;
    }
    read_half(f1, buf, 1);
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = mfma16x16x32(f0.b[ni], f0.a[mi], acc[mi][ni]);
#pragma unroll
    for (int i = 0; i < MT + NT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
    use_regs<MT>(f1.a);
    use_regs<NT>(f1.b);
    wait_vm<C::LPW>();
    block_barrier();
    issue(ti, adma, buf, st);
    buf = buf == C::NS - 1 ? 0 : buf + 1;
    read_half(f0, buf, 0);
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = mfma16x16x32(f1.b[ni], f1.a[mi], acc[mi][ni]);
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM (DMA)
    }
#pragma unroll
    for (int i = 0; i < MT + NT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // first tile: its rows, then stages 0..2, then stage 0's first half
  gather_issue(cur, nxt_raw);
  gather_finish(cur, nxt_raw, cur_adma);
#pragma unroll
  for (int p = 0; p < C::NS; ++p) issue(cur, cur_adma, p, p);
  wait_vm<(C::NS - 1) * C::LPW>();
  block_barrier();
  read_half(f0, 0, 0);

  for (;;) {
    const int tn = t + (int)gridDim.x;
    const bool has_next = tn < total;
    if (has_next) nxt = locate(tn);
    gather_issue(nxt, nxt_raw);  // (the current tile again when there is no next)
    act = __builtin_amdgcn_readfirstlane(64 * wm < cur.nrows ? 1 : 0) != 0;
    f32x4 acc[MT][NT];  // (scoped to the tile: no accumulator value crosses tiles)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
    step(acc, cur, cur_adma, 3);
    step(acc, cur, cur_adma, 4);
    // The wait in step 1 retired every load issued before step 0's DMA,
    // including the pair ids above: mark them read here, so that the
    // compiler's own wait for them (where paths merge) does not drain the ring.
#pragma unroll
    for (int i = 0; i < C::LPA; ++i) asm volatile("" : "+v"(nxt_raw[i]));
    gather_finish(nxt, nxt_raw, nxt_adma);
    for (int kt = 2; kt < nk - 3; ++kt) step(acc, cur, cur_adma, kt + 3);
    // the last three steps stream in the next tile's first three
    step(acc, nxt, nxt_adma, 0);
    step(acc, nxt, nxt_adma, 1);
    step(acc, nxt, nxt_adma, 2);
    // (pinned so that the last MFMAs are not sunk into the row-guarded stores)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) asm volatile("" : "+a"(acc[mi][ni]));

    // ---- epilogue (registers -> global) -----------------------------------
    // D[n][m]: lane (li, kc) holds activation row li of group mi and, for
    // weight group ni, weight rows (= output columns) 4 kc .. 4 kc + 3.  For a
    // pair of groups (ni, ni + 1) the lanes of 16-lane rows kc and kc ^ 1 swap
    // halves (v_permlane16_swap), so that an even-kc lane holds 8 consecutive
    // columns of group ni and its odd partner 8 of group ni + 1: one 16-byte
    // store per lane and pair instead of two 8-byte ones.
    // the extra group's rows go to its own output, row rel0 + r
    uint16_t* out = static_cast<uint16_t*>(cur.ext ? g.xg_out : g.out);
    const int orow0 = cur.ext ? cur.rel0 : cur.row0;
    constexpr int NG = SWIGLU ? NT / 2 : NT;  // output groups per wave
    const int odd = kc & 1;
    const int col = (SWIGLU ? C::BN / 2 : C::BN) / C::WN * wn + 8 * (kc >> 1);
    // GEMM2: this wave's 2 KB of LDS past the ring, for the row-slice stores
    uint8_t* const oscr = smem + C::NS * C::STAGE + wave * 2048;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const int r = 64 * wm + 16 * mi + li;
      uint16_t* orow = out + (size_t)(orow0 + min(r, cur.nrows - 1)) * g.N + cur.n0 + col;
#pragma unroll
      for (int np = 0; np < NG; np += 2) {
        u32x2 pk[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ni = np + h;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[i] = SWIGLU ? silu_fast(acc[mi][ni][i]) * acc[mi][ni + NT / 2][i] : acc[mi][ni][i];
          pk[h].x = pack_bf16x2(v[0], v[1]);
          pk[h].y = pack_bf16x2(v[2], v[3]);
        }
        // vdst = group np, vsrc = group np + 1: odd rows receive the even
        // partner's np + 1 words, even rows the odd partner's np words
        const auto s0 = __builtin_amdgcn_permlane16_swap(pk[0].x, pk[1].x, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(pk[0].y, pk[1].y, false, false);
        u32x4 o;
        if (odd) {
          o = u32x4{s0[0], s1[0], pk[1].x, pk[1].y};  // group np + 1, columns 8 (kc>>1) ..
        } else {
          o = u32x4{pk[0].x, pk[0].y, s0[1], s1[1]};  // group np, columns 8 (kc>>1) ..
        }
        if (SWIGLU) {
          if (r < cur.nrows) *reinterpret_cast<u32x4*>(orow + 16 * (np + odd)) = o;
        } else {
          // 16-byte chunk 2 (np + odd) + (kc >> 1) of row li of the wave's
          // 128-byte row slices, XOR-swizzled by the row
          *reinterpret_cast<u32x4*>(oscr + li * 128 + 16 * ((2 * (np + odd) + (kc >> 1)) ^ (li & 7))) = o;
        }
      }
      if (!SWIGLU) {
        // the wave's 16 rows x 64 columns back from LDS as whole 128-byte
        // row slices: lane l takes chunk l % 8 of row l / 8 (+ 8), so one
        // store covers 8 full rows instead of 16 half rows
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int rr = 8 * j + (lane >> 3), c = lane & 7;
          const u32x4 o = *reinterpret_cast<const u32x4*>(oscr + rr * 128 + 16 * (c ^ (rr & 7)));
          const int rg = 64 * wm + 16 * mi + rr;
          if (rg < cur.nrows)
            *reinterpret_cast<u32x4*>(out + (size_t)(orow0 + rg) * g.N + cur.n0 + C::BN / C::WN * wn + 8 * c) = o;
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
  }
}

// Shapes the kernel takes: whole output tiles, K a multiple of 64 with at
// least 5 steps (two leading steps and the last three are peeled off the
// loop), and operands addressable with 32-bit offsets.
bool tiled4_fits(const GroupedGemm& g, bool swiglu) {
  const long long arows = g.gather ? g.total_rows / g.topk : g.total_rows;
  const long long wrows = swiglu ? 2ll * g.up_off : g.N;
  return g.N % (swiglu ? 128 : 256) == 0 && g.K % 64 == 0 && g.K >= 320 &&
         arows * g.K * 2 < (1ll << 32) && wrows * g.K * 2 < (1ll << 32) &&
         (long long)g.xg_rows * g.K * 2 < (1ll << 32);
}

template <bool SWIGLU, bool GATHER>
static void launch_tiled4_impl(const GroupedGemm& g, hipStream_t s) {
  using C = Tiled4<SWIGLU>;
  const int nt = g.N / C::BNOUT;
  const int groups = g.offsets ? g.G : 1;
  const long long bound =
      ((long long)(g.total_rows + g.xg_rows + C::BM - 1) / C::BM + groups + (g.xg_rows > 0)) * nt;
  auto k = ffn_tiled4<SWIGLU, GATHER>;
  const int grid = resident_grid(reinterpret_cast<const void*>(k), C::NTHR, bound);
  hipLaunchKernelGGL(k, dim3(grid), dim3(C::NTHR), 0, s, g, nt);
}

void launch_tiled4(const GroupedGemm& g, bool swiglu, hipStream_t s) {
  if (swiglu)
    g.gather ? launch_tiled4_impl<true, true>(g, s) : launch_tiled4_impl<true, false>(g, s);
  else
    g.gather ? launch_tiled4_impl<false, true>(g, s) : launch_tiled4_impl<false, false>(g, s);
}

}  // namespace moe
