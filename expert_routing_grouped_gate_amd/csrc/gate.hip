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

// Many tokens (prefill): LDS-tiled fp32 product, block tile 64 tokens x 32
// experts, K step 32; each thread owns 4 tokens x 2 experts.
constexpr int RT_TT = 64, RT_TE = 32, RT_BK = 32;

__global__ __launch_bounds__(256) void router_logits_tiled(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ wr, int T,
                                                           int H, int E,
                                                           float* __restrict__ logits) {
  __shared__ float xs[RT_BK][RT_TT + 4];
  __shared__ float ws[RT_BK][RT_TE + 4];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RT_TT;
  const int e0 = blockIdx.y * RT_TE;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][2] = {};
  // load assignments
  const int xl_tok = tid >> 2, xl_h = (tid & 3) * 8;
  const int wl_e = tid >> 3, wl_h = (tid & 7) * 4;
  const int xtok = min(t0 + xl_tok, T - 1);
  const int we = min(e0 + wl_e, E - 1);
  const uint16_t* xp = x + (size_t)xtok * H + xl_h;
  const float* wp = wr + (size_t)we * H + wl_h;
  for (int h0 = 0; h0 < H; h0 += RT_BK) {
    const u32x4 xv = ld16(xp + h0);
    const float4 wv = *reinterpret_cast<const float4*>(wp + h0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[xl_h + 2 * i][xl_tok] = bf16_to_f32(xv[i] & 0xffffu);
      xs[xl_h + 2 * i + 1][xl_tok] = bf16_to_f32(xv[i] >> 16);
    }
    ws[wl_h + 0][wl_e] = wv.x;
    ws[wl_h + 1][wl_e] = wv.y;
    ws[wl_h + 2][wl_e] = wv.z;
    ws[wl_h + 3][wl_e] = wv.w;
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < RT_BK; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&xs[kk][ty * 4]);
      const float2 b = *reinterpret_cast<const float2*>(&ws[kk][tx * 2]);
      acc[0][0] = fmaf(a.x, b.x, acc[0][0]);
      acc[0][1] = fmaf(a.x, b.y, acc[0][1]);
      acc[1][0] = fmaf(a.y, b.x, acc[1][0]);
      acc[1][1] = fmaf(a.y, b.y, acc[1][1]);
      acc[2][0] = fmaf(a.z, b.x, acc[2][0]);
      acc[2][1] = fmaf(a.z, b.y, acc[2][1]);
      acc[3][0] = fmaf(a.w, b.x, acc[3][0]);
      acc[3][1] = fmaf(a.w, b.y, acc[3][1]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + tx * 2 + j;
      if (e < E) logits[(size_t)t * E + e] = acc[i][j];
    }
  }
}

int launch_router_logits(const uint16_t* x, const float* wr, int T, int H, int E, float* logits,
                         hipStream_t s) {
  if (T <= 64) {
    hipLaunchKernelGGL(router_logits_small, dim3(E, (T + 15) / 16), dim3(256), 0, s, x, wr, T, H,
                       E, logits);
  } else {
    hipLaunchKernelGGL(router_logits_tiled, dim3((T + RT_TT - 1) / RT_TT, (E + RT_TE - 1) / RT_TE),
                       dim3(256), 0, s, x, wr, T, H, E, logits);
  }
  return launch_status();
}

// ---------------------------------------------------------------- S2 ------
// One wave per token.  Lane l holds experts l, l+64, l+128, l+192 (E <= 256).
// k rounds of a wave-wide arg-max over (key desc, id asc); the owner lane
// retires the winner.  Keys, sigmoid values and weights are fp64.
struct Cand {
  double key;
  int id;
};

__device__ __forceinline__ bool better(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

template <int MODE>
__global__ __launch_bounds__(256) void gate_topk_kernel(const float* __restrict__ logits,
                                                        const float* __restrict__ bias, int T,
                                                        int E, int k, float routed_scale,
                                                        float eps, int32_t* __restrict__ ids,
                                                        float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  constexpr int NEG_BIG_ID = 0x7fffffff;
  const double NEG_INF = -__builtin_inf();
  double key[4], sval[4];
  int id[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    key[i] = NEG_INF;
    sval[i] = 0.0;
    id[i] = NEG_BIG_ID;
    if (e < E) {
      const float L = logits[(size_t)t * E + e];
      id[i] = e;
      if (MODE == 0) {
        const float kf = bias ? (L + bias[e]) : L;  // fp32 add, as the oracle
        key[i] = (kf != kf) ? NEG_INF : (double)kf;
      } else {
        const double s = 1.0 / (1.0 + exp(-(double)L));
        sval[i] = s;
        const double kk = bias ? s + (double)bias[e] : s;
        key[i] = (kk != kk) ? NEG_INF : kk;
      }
    }
  }
  double my_key = 0.0, my_s = 0.0;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    double bk = key[0];
    int bi = id[0];
    double bs = sval[0];
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (better(key[i], id[i], bk, bi)) {
        bk = key[i];
        bi = id[i];
        bs = sval[i];
      }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const double ok = __shfl_xor(bk, d, 64);
      const int oi = __shfl_xor(bi, d, 64);
      const double os = __shfl_xor(bs, d, 64);
      if (better(ok, oi, bk, bi)) {
        bk = ok;
        bi = oi;
        bs = os;
      }
    }
    // bi is wave-uniform now; retire it at its owner
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (id[i] == bi) {
        key[i] = NEG_INF;
        id[i] = NEG_BIG_ID;
      }
    if (lane == j) {
      my_key = bk;
      my_id = bi;
      my_s = bs;
    }
  }
  double v;
  if (MODE == 0) {
    const double k0 = __shfl(my_key, 0, 64);
    v = (lane < k) ? exp(my_key - k0) : 0.0;
  } else {
    v = (lane < k) ? my_s : 0.0;
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
    ids[(size_t)t * k + lane] = my_id;
    wout[(size_t)t * k + lane] = (float)w;
  }
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
