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

template <bool SWIGLU, int WM, int WN, int NS>
__device__ __forceinline__ void mx_tiled_tile(const GroupedGemm& g, uint8_t* smem, int n_tile,
                                              int grp, int row0, int nrows) {
  using C = MxTiled<SWIGLU, WM, WN, NS>;
  constexpr int MT = C::MT, NT = C::NT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int li = lane & 15, kb = lane >> 4;
  const int K = g.K, ns = K / 128, nq = ns / 4;
  const int n0 = n_tile * C::BNOUT;
  const uint8_t* A = static_cast<const uint8_t*>(g.A);
  const uint8_t* Wg = static_cast<const uint8_t*>(g.W) + (size_t)grp * g.w_gstride;

  // ---- DMA sources (per lane) -------------------------------------------
  // activation group ra (8 rows): lane l fills row 8 ra + l/8, physical
  // chunk l % 8, i.e. it loads logical chunk (l % 8) ^ (l / 8)
  const uint8_t* asrc[C::LPA];
#pragma unroll
  for (int i = 0; i < C::LPA; ++i) {
    const int row = 8 * (wave + C::NW * i) + (lane >> 3);
    const int r = row0 + min(row, nrows - 1);  // rows past the tile end reuse a valid row
    const int arow = gather_row(g.sorted_pair, g.gather, g.topk, g.total_rows, r);
    asrc[i] = A + (size_t)arow * K + 16 * ((lane & 7) ^ (lane >> 3));
  }
  const uint8_t* wsrc[C::LPB];
#pragma unroll
  for (int i = 0; i < C::LPB; ++i) {
    const int q = mx_block_row<SWIGLU, C::BN>(g, n0, wave + C::NW * i) / 16;
    wsrc[i] = Wg + (size_t)q * ns * 1024 + lane * 16;
  }
  auto issue = [&](int buf, int st) {
    uint8_t* stg = smem + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::LPA; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(asrc[i] + st * 128),
          (__attribute__((address_space(3))) void*)(stg + (wave + C::NW * i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < C::LPB; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(wsrc[i] + (size_t)st * 1024),
          (__attribute__((address_space(3))) void*)(stg + C::ABYTES + (wave + C::NW * i) * 1024),
          16, 0, 0);
  };

  // ---- scales (registers) ------------------------------------------------
  const int arows_total = g.gather ? g.total_rows / g.topk : g.total_rows;
  const __amdgpu_buffer_rsrc_t asr = mx_rsrc(g.A_scales, (uint32_t)arows_total * (uint32_t)(K / 32));
  const uint32_t wrows = SWIGLU ? 2u * (uint32_t)g.up_off : (uint32_t)g.N;
  const __amdgpu_buffer_rsrc_t wsr =
      mx_rsrc(g.W_scales + (size_t)grp * g.ws_gstride, wrows / 16u * (uint32_t)nq * 256u);
  uint32_t aoff[MT];  // byte offset of this lane's activation scale row
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    const int r = row0 + min(16 * (mi * WM + wm) + li, nrows - 1);
    aoff[mi] = (uint32_t)gather_row(g.sorted_pair, g.gather, g.topk, g.total_rows, r) * (uint32_t)(K / 32);
  }
  int wq[NT];  // weight group (16-row block index) of group ni, wave-uniform
#pragma unroll
  for (int ni = 0; ni < NT; ++ni)
    wq[ni] = mx_block_row<SWIGLU, C::BN>(g, n0, mx_wave_block<SWIGLU, NT, C::BN>(wn, ni)) / 16;
  u32x4 as_nxt[MT];     // activation scales of the next quad, as loaded
  uint32_t as_cur[MT];  // byte u: this lane's 32-block (kb) at step 4c + u
  uint32_t ws_cur[NT], ws_nxt[NT];
  // word u of the 16 bytes holds the four 32-blocks of step 4c + u
  auto compact = [&]() {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      uint32_t v = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) v |= ((as_nxt[mi][u] >> (8 * kb)) & 0xffu) << (8 * u);
      as_cur[mi] = v;
    }
  };
  auto load_scales = [&](u32x4* as, uint32_t* ws, int c) {  // quad c
#pragma unroll
    for (int ni = 0; ni < NT; ++ni)
      ws[ni] = __builtin_amdgcn_raw_buffer_load_b32(wsr, lane * 4, (wq[ni] * nq + c) * 256, 0);
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
      as[mi] = __builtin_amdgcn_raw_buffer_load_b128(asr, aoff[mi] + 16 * c, 0, 0);
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

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  int c_cur = 0, kt_base = 0;  // current quad and its first step

  // ---- pipeline ------------------------------------------------------------
  // Quad 0's scales first, then stages 0 .. 3 (ns >= 4).  Step kt (stage
  // buffer kt % 4): the fragments of step kt are in registers (read one step
  // earlier); wait until this wave's DMA of stage kt+1 is done; barrier (stage
  // kt+1 complete for every wave, stage kt's buffer read by every wave); DMA
  // of step kt+4 into stage kt's buffer; read step kt+1's fragments; MFMAs of
  // step kt.  The explicit vmcnt waits count only the DMA loads (the scale
  // loads in between only make them stricter).  The last quad is peeled off,
  // so every wait count is a constant and the loop body has no branch (a
  // branch would let the MFMAs be moved past the barriers).
  auto step = [&](auto U, auto LAST) {
    constexpr int u = decltype(U)::value;
    constexpr bool last = decltype(LAST)::value;
    constexpr int f = u & 1;
    // this wave's fragment reads of stage kt must land before the barrier
    use_frags<MT>(af[f]);
    use_regs<NT>(wf[f]);
    if (!last || u == 0)
      wait_vm<2 * C::LPW>();  // stages kt+2, kt+3 may stay in flight
    else if (u == 1)
      wait_vm<C::LPW>();
    else
      wait_vm<0>();
    block_barrier();
    if (!last) {
      issue(u, kt_base + u + 4);
      if (u == 0) load_scales(as_nxt, ws_nxt, c_cur + 1);
    }
    if (!last || u < 3) read_frags(f ^ 1, (u + 1) & 3);
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
    if (!last) {
#pragma unroll
      for (int i = 0; i < C::LPW + (u == 0 ? MT + NT : 0); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
      }
    }
    if (!last || u < 3) {
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
  using Mid = std::integral_constant<bool, false>;
  using Last = std::integral_constant<bool, true>;

  load_scales(as_nxt, ws_cur, 0);
  compact();
#pragma unroll
  for (int p = 0; p < 4; ++p) issue(p, p);
  wait_vm<3 * C::LPW>();
  block_barrier();
  read_frags(0, 0);
  for (c_cur = 0; c_cur < nq - 1; ++c_cur) {
    kt_base = 4 * c_cur;
    step(I0{}, Mid{});
    step(I1{}, Mid{});
    step(I2{}, Mid{});
    step(I3{}, Mid{});
    compact();
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) ws_cur[ni] = ws_nxt[ni];
  }
  kt_base = 4 * c_cur;
  step(I0{}, Last{});
  step(I1{}, Last{});
  step(I2{}, Last{});
  step(I3{}, Last{});
  // Every DMA and LDS read of this tile has completed before the last
  // barrier: the next tile may refill the ring.  (The accumulators are
  // pinned here so that the last MFMAs are not sunk into the row-guarded
  // stores below.)
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) asm volatile("" : "+a"(acc[mi][ni]));

  // ---- epilogue (registers -> global) -------------------------------------
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
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int e = mx_exponent(amax);
        const float inv = exp2_neg(e);
        const uint32_t lo = e4m3_pack4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
        const uint32_t hi = e4m3_pack4(a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv);
        if (r < nrows) {
          const int col0 = n0 + 16 * (wn * (NT / 2) + 2 * b);
          uint8_t* orow = static_cast<uint8_t*>(g.out) + (size_t)(row0 + r) * g.N;
          *reinterpret_cast<uint32_t*>(orow + col0 + 4 * kb) = lo;
          *reinterpret_cast<uint32_t*>(orow + col0 + 16 + 4 * kb) = hi;
          if (kb == 0) g.out_scales[(size_t)(row0 + r) * (g.N / 32) + col0 / 32] = (uint8_t)(e + 127);
        }
      }
    } else if (r < nrows) {
      uint16_t* orow = static_cast<uint16_t*>(g.out) + (size_t)(row0 + r) * g.N + n0 +
                       16 * wn * NT + 4 * kb;
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) {
        u32x2 pk;
        pk.x = pack_bf16x2(acc[mi][ni][0], acc[mi][ni][1]);
        pk.y = pack_bf16x2(acc[mi][ni][2], acc[mi][ni][3]);
        *reinterpret_cast<u32x2*>(orow + 16 * ni) = pk;
      }
    }
  }
}

template <bool SWIGLU, int WM, int WN, int NS>
__global__ __launch_bounds__(64 * WM * WN, 1) void ffn_mx_tiled(GroupedGemm g, int n_tiles) {
  using C = MxTiled<SWIGLU, WM, WN, NS>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * C::STAGE];
  TileMap tm;
  tm.init(g.offsets, g.G, g.ident_rows, C::BM, g.total_rows);
  const int total = tm.total * n_tiles;
  // Expert-major tile order (as in the bf16 tiled kernel): the m-tiles that
  // share a weight tile are neighbours, and an expert's tiles stay on one XCD.
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int id = xcd_remap(t, total);
    int grp, first_mt, n_mt, grow0, grow1;
    tm.find_group(id / n_tiles, grp, first_mt, n_mt, grow0, grow1);
    const int local = id - first_mt * n_tiles;
    const int n_tile = local / n_mt;
    const int row0 = grow0 + (local - n_tile * n_mt) * C::BM;
    mx_tiled_tile<SWIGLU, WM, WN, NS>(g, smem, __builtin_amdgcn_readfirstlane(n_tile),
                                      __builtin_amdgcn_readfirstlane(grp),
                                      __builtin_amdgcn_readfirstlane(row0),
                                      __builtin_amdgcn_readfirstlane(min(C::BM, grow1 - row0)));
  }
}

// Shapes the tiled kernels take: whole 128-column (GEMM1) / 256-column
// (GEMM2) output tiles and K a multiple of 512 (whole quads of steps).
bool mx_tiled_fits(const GroupedGemm& g, bool swiglu) {
  return g.N % (swiglu ? 128 : 256) == 0 && g.K % 512 == 0;
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
