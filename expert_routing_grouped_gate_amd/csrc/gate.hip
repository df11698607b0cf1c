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

namespace moe {

// ---------------------------------------------------------------- S1 ------
// Few tokens (decode): one block of 256 threads per (expert, 16-token tile).
// Every thread issues all its loads for a 4096-wide slice of H at once (4
// float4 of the router row, 4 x 8 bytes of each token row), so one memory
// latency covers the slice; then the block reduces the 16 partial sums
// (wave butterfly, then the 4 waves through LDS).  Fixed order ->
// deterministic.
__global__ __launch_bounds__(256) void router_logits_small(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ wr, int T,
                                                           int H, int E,
                                                           float* __restrict__ logits) {
  __shared__ float part[4][16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * 16;
  const int nt = min(16, T - t0);
  const float* wrow = wr + (size_t)e * H;
  const uint16_t* xt = x + (size_t)t0 * H;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int hb = 0; hb < H; hb += 4096) {
    float4 w4[4];
    u32x2 xv[4][16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = hb + j * 1024 + tid * 4;
      const bool ok = h < H;
      w4[j] = ok ? *reinterpret_cast<const float4*>(wrow + h) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        xv[j][i] = (ok && i < nt) ? *reinterpret_cast<const u32x2*>(xt + (size_t)i * H + h) : u32x2{0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float a = acc[i];
        a = fmaf(bf16_to_f32(xv[j][i].x & 0xffffu), w4[j].x, a);
        a = fmaf(bf16_to_f32(xv[j][i].x >> 16), w4[j].y, a);
        a = fmaf(bf16_to_f32(xv[j][i].y & 0xffffu), w4[j].z, a);
        a = fmaf(bf16_to_f32(xv[j][i].y >> 16), w4[j].w, a);
        acc[i] = a;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = acc[i];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if (lane == 0) part[wave][i] = v;
  }
  __syncthreads();
  if (tid < nt) logits[(size_t)(t0 + tid) * E + e] = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
}

// Many tokens (prefill): the product on bf16 MFMA, exactly.  Each fp32
// router weight is split into three bf16 terms, w = hi + mid + lo (hi and mid
// are truncations, lo is the exact remainder: 8 + 8 + 8 significand bits), so
// x * w = x*hi + x*mid + x*lo where every product of the bf16 x with a term
// is exact in fp32; the MFMA accumulates the three products in fp32.  Block
// tile 32 tokens x 64 experts, K step 32, operands staged in double-buffered
// LDS (the split is done once, by the loading thread); wave w owns experts
// 16w..16w+15 of the tile and both 16-token halves (6 MFMAs per K step).
constexpr int RM_TT = 32, RM_TE = 64;

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

__global__ __launch_bounds__(256) void router_logits_mfma(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr, int T,
                                                          int H, int E,
                                                          float* __restrict__ logits) {
  __shared__ u32x4 xs[2][RM_TT * 4];
  __shared__ u32x4 ws[2][3][RM_TE * 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RM_TT, e0 = blockIdx.y * RM_TE;
  // loaders: threads 0..127 -> x (token tid/4, chunk tid%4); all -> wr (expert tid/4, chunk tid%4)
  const int lrow = tid >> 2, lch = tid & 3;
  const uint16_t* xp = x + (size_t)min(t0 + (lrow & 31), T - 1) * H + lch * 8;
  const float* wp = wr + (size_t)min(e0 + lrow, E - 1) * H + lch * 8;
  // two register sets: step k+2 is loaded while step k computes and step k+1
  // waits to be split and stored into the other LDS buffer
  u32x4 rx0, rx1;
  float rw0[8], rw1[8];
  auto gload = [&](u32x4& rx, float* rw, int k0) {
    if (tid < 128) rx = ld16(xp + k0);
    const float4 a = *reinterpret_cast<const float4*>(wp + k0);
    const float4 b = *reinterpret_cast<const float4*>(wp + k0 + 4);
    rw[0] = a.x; rw[1] = a.y; rw[2] = a.z; rw[3] = a.w;
    rw[4] = b.x; rw[5] = b.y; rw[6] = b.z; rw[7] = b.w;
  };
  auto lstore = [&](const u32x4& rx, const float* rw, int buf) {
    if (tid < 128) xs[buf][lrow * 4 + lch] = rx;
    u32x4 h, m, l;
    split3_bf16(rw, h, m, l);
    ws[buf][0][lrow * 4 + lch] = h;
    ws[buf][1][lrow * 4 + lch] = m;
    ws[buf][2][lrow * 4 + lch] = l;
  };
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fc = lane >> 4;
  auto compute = [&](int buf) {
    const u32x4 a0 = xs[buf][fr * 4 + fc];
    const u32x4 a1 = xs[buf][(16 + fr) * 4 + fc];
#pragma unroll
    for (int sp = 0; sp < 3; ++sp) {
      const u32x4 b = ws[buf][sp][(16 * wave + fr) * 4 + fc];
      acc0 = mfma16x16x32(a0, b, acc0);
      acc1 = mfma16x16x32(a1, b, acc1);
    }
  };
  const int nk = H / 32;
  gload(rx0, rw0, 0);
  if (nk > 1) gload(rx1, rw1, 32);
  lstore(rx0, rw0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    if (kt + 2 < nk) gload(rx0, rw0, (kt + 2) * 32);
    compute(0);
    if (kt + 1 < nk) lstore(rx1, rw1, 1);
    __syncthreads();
    if (kt + 1 >= nk) break;
    if (kt + 3 < nk) gload(rx1, rw1, (kt + 3) * 32);
    compute(1);
    if (kt + 2 < nk) lstore(rx0, rw0, 0);
    __syncthreads();
  }
  // D[m][n]: lane holds expert 16*wave + (lane & 15), tokens 4*(lane>>4) + i
  const int e = e0 + 16 * wave + fr;
  if (e < E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ta = t0 + 4 * fc + i, tb = t0 + 16 + 4 * fc + i;
      if (ta < T) logits[(size_t)ta * E + e] = acc0[i];
      if (tb < T) logits[(size_t)tb * E + e] = acc1[i];
    }
  }
}

int launch_router_logits(const uint16_t* x, const float* wr, int T, int H, int E, float* logits,
                         hipStream_t s) {
  if (T <= 64) {
    hipLaunchKernelGGL(router_logits_small, dim3(E, (T + 15) / 16), dim3(256), 0, s, x, wr, T, H,
                       E, logits);
  } else {
    hipLaunchKernelGGL(router_logits_mfma, dim3((T + RM_TT - 1) / RM_TT, (E + RM_TE - 1) / RM_TE),
                       dim3(256), 0, s, x, wr, T, H, E, logits);
  }
  return launch_status();
}

// ---------------------------------------------------------------- S2 ------
// One wave per token.  Lane l holds experts l, l+64, l+128, l+192 (E <= 256).
// Each candidate is an order-preserving unsigned key (the fp32 key in softmax
// mode, the fp64 key in sigmoid mode; -0 folded into +0, NaN treated as
// -inf) plus its id; a candidate beats another on a larger key, then on a
// smaller id.  k rounds of a wave arg-max: each lane's best of its 4, the
// best of each 16-lane row through 4 DPP exchanges (quad xor 1, quad xor 2,
// half-row mirror, row mirror), then the 4 row winners read with readlane;
// the owner retires the winner.  Sigmoid values and weights are fp64.
__device__ __forceinline__ uint64_t ord_key32(float f) {
  f = (f != f) ? -__builtin_inff() : f + 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (uint64_t)((u >> 31) ? ~u : (u | 0x80000000u));
}

__device__ __forceinline__ float unord_key32(uint64_t k) {
  const uint32_t u = (uint32_t)k;
  return __uint_as_float((u >> 31) ? (u & 0x7fffffffu) : ~u);
}

__device__ __forceinline__ uint64_t ord_key64(double d) {
  d = (d != d) ? -__builtin_inf() : d + 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(d);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ bool beats(uint64_t ka, uint32_t ia, uint64_t kb, uint32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ void dpp_keep_best(uint64_t& k, uint32_t& id) {
  const uint32_t lo = dpp32<CTRL>((uint32_t)k), hi = dpp32<CTRL>((uint32_t)(k >> 32));
  const uint32_t oid = dpp32<CTRL>(id);
  const uint64_t ok = ((uint64_t)hi << 32) | lo;
  if (beats(ok, oid, k, id)) {
    k = ok;
    id = oid;
  }
}

__device__ __forceinline__ uint32_t rdlane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Top-k of one token.  L[i] = logit of expert lane + 64 i (ignored past E).
// Writes ids[0..k) and weights[0..k) of the token.
template <int MODE>
__device__ __forceinline__ void gate_token(const float (&L)[4], const float* __restrict__ bias,
                                           int E, int k, float routed_scale, float eps,
                                           int32_t* __restrict__ ids_row,
                                           float* __restrict__ w_row) {
  const int lane = threadIdx.x & 63;
  constexpr uint32_t NO_ID = 0xffffffffu;
  uint64_t key[4];
  uint32_t id[4];
  double sval[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    key[i] = 0;  // below every real key, even -inf
    id[i] = NO_ID;
    sval[i] = 0.0;
    if (e < E) {
      id[i] = (uint32_t)e;
      if (MODE == 0) {
        key[i] = ord_key32(bias ? (L[i] + bias[e]) : L[i]);  // fp32 add, as the oracle
      } else {
        const double sg = 1.0 / (1.0 + exp(-(double)L[i]));
        sval[i] = sg;
        key[i] = ord_key64(bias ? sg + (double)bias[e] : sg);
      }
    }
  }
  uint64_t my_key = 0;
  uint32_t my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t bk = key[0];
    uint32_t bi = id[0];
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (beats(key[i], id[i], bk, bi)) {
        bk = key[i];
        bi = id[i];
      }
    dpp_keep_best<0xB1>(bk, bi);   // quad_perm [1,0,3,2]
    dpp_keep_best<0x4E>(bk, bi);   // quad_perm [2,3,0,1]
    dpp_keep_best<0x141>(bk, bi);  // row_half_mirror
    dpp_keep_best<0x140>(bk, bi);  // row_mirror
    uint64_t wk = ((uint64_t)rdlane((uint32_t)(bk >> 32), 0) << 32) | rdlane((uint32_t)bk, 0);
    uint32_t wi = rdlane(bi, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
      const uint64_t rk =
          ((uint64_t)rdlane((uint32_t)(bk >> 32), 16 * r) << 32) | rdlane((uint32_t)bk, 16 * r);
      const uint32_t ri = rdlane(bi, 16 * r);
      if (beats(rk, ri, wk, wi)) {
        wk = rk;
        wi = ri;
      }
    }
    // wi is wave-uniform; its owner retires it
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (id[i] == wi) {
        key[i] = 0;
        id[i] = NO_ID;
      }
    if (lane == j) {
      my_key = wk;
      my_id = wi;
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
    for (int i = 0; i < 4; ++i) {
      const double o = __shfl(sval[i], src, 64);
      if (slot == i) sv = o;
    }
    v = (lane < k) ? sv : 0.0;
  }
  double sum = v;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
  if (lane < k) {
    double w;
    if (MODE == 0)
      w = v / sum;
    else
      w = v / (sum + (double)eps) * (double)routed_scale;
    ids_row[lane] = (int32_t)my_id;
    w_row[lane] = (float)w;
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void gate_topk_kernel(const float* __restrict__ logits,
                                                        const float* __restrict__ bias, int T,
                                                        int E, int k, float routed_scale,
                                                        float eps, int32_t* __restrict__ ids,
                                                        float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; no barriers
  float L[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    L[i] = e < E ? logits[(size_t)t * E + e] : 0.f;
  }
  gate_token<MODE>(L, bias, E, k, routed_scale, eps, ids + (size_t)t * k, wout + (size_t)t * k);
}

int launch_gate_topk(const float* logits, const float* bias, int T, int E, int k, int mode,
                     float routed_scale, float eps, int32_t* ids, float* w, hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (mode == 0)
    hipLaunchKernelGGL(gate_topk_kernel<0>, grid, block, 0, s, logits, bias, T, E, k,
                       routed_scale, eps, ids, w);
  else
    hipLaunchKernelGGL(gate_topk_kernel<1>, grid, block, 0, s, logits, bias, T, E, k,
                       routed_scale, eps, ids, w);
  return launch_status();
}

}  // namespace moe
