// The step before the MoE layer: residual add + RMSNorm in one pass, with
// the outputs the layer takes.
//
// [Qwen3] "fused-operator optimisation": residual add, RMSNorm and dynamic
// MXFP8 quantisation are fused so that the intermediate results are not
// written and read back ("fused RMSNorm + MX quant"), and the norm before the
// MoE block returns its result in FP32 for the gate and in BF16 for the
// experts together with the updated residual ("fused RMSNorm + Cast").
// [Notes] section 2, "Add and RMSNorm": z = x + r, then
// y_i = z_i / sqrt(mean_j z_j^2 + eps) * w_i.
//
// One block of 256 threads per row (norm_row in rowops.hpp): the row's
// chunks stay in registers, so x and r are read once and every output is
// written once.  The fused form takes x from the combine of the layer's
// expert rows (combine_chunks), the layer output the next layer's norm reads:
// the combined row is rounded to bf16 exactly as moe_combine stores it, so the
// fusion reproduces moe_combine followed by moe_add_rmsnorm bit for bit while
// the combined row never round-trips through memory (it is stored only if
// asked for).
#include "common.hpp"
#include "launch.hpp"
#include "rowops.hpp"

namespace moe {

template <int NCH>
__global__ __launch_bounds__(kNormThreads) void add_rmsnorm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ res,
    const uint16_t* __restrict__ w, int H, float eps, NormOut o) {
  const size_t row = blockIdx.x;
  const uint16_t* xr = x + row * (size_t)H;
  u32x4 xv[NCH], rv[NCH], wv[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) xv[j] = ld16(xr + 8 * norm_chunk(j, H / 8));
  norm_row_loads<NCH>(res, w, H, row, rv, wv);
  norm_row<NCH>(xv, rv, wv, H, eps, row, o);
}

template <int NCH>
__global__ __launch_bounds__(kNormThreads) void combine_add_rmsnorm_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ pair_pos,
    const float* __restrict__ tw, const uint16_t* __restrict__ shared_y, int k,
    const uint16_t* __restrict__ res, const uint16_t* __restrict__ w, int H, float eps,
    uint16_t* __restrict__ out, NormOut o) {
  const int t = blockIdx.x;
  const int R = (int)gridDim.x * k;
  const int32_t* pp = pair_pos + (size_t)t * k;
  const float* wt = tw + (size_t)t * k;
  const uint16_t* srow = shared_y ? shared_y + (size_t)t * H : nullptr;
  // the norm's residual and weight chunks first, then every chunk of this
  // thread combined (all slot rows in flight at once)
  u32x4 rv[NCH], wv[NCH];
  norm_row_loads<NCH>(res, w, H, t, rv, wv);
  u32x4 xv[NCH];
  const int c0 = 8 * (int)threadIdx.x;
  combine_chunks<NCH>(y, pp, wt, srow, k, R, H, c0, xv);
  if (out) {
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      if (c0 + 2048 * j < H) *reinterpret_cast<u32x4*>(out + (size_t)t * H + c0 + 2048 * j) = xv[j];
  }
  norm_row<NCH>(xv, rv, wv, H, eps, t, o);
}

template <int NCH>
static void launch_norm(const uint16_t* x, const uint16_t* res, const uint16_t* w, int T, int H,
                        float eps, const NormOut& o, hipStream_t s) {
  hipLaunchKernelGGL(add_rmsnorm_kernel<NCH>, dim3(T), dim3(kNormThreads), 0, s, x, res, w, H, eps,
                     o);
}

template <int NCH>
static void launch_fused(const uint16_t* y, const int32_t* pair_pos, const float* tw,
                         const uint16_t* shared_y, int T, int k, const uint16_t* res,
                         const uint16_t* w, int H, float eps, uint16_t* out, const NormOut& o,
                         hipStream_t s) {
  hipLaunchKernelGGL(combine_add_rmsnorm_kernel<NCH>, dim3(T), dim3(kNormThreads), 0, s, y,
                     pair_pos, tw, shared_y, k, res, w, H, eps, out, o);
}

static int norm_chunks(int H) { return (H / 8 + kNormThreads - 1) / kNormThreads; }

// T >= 1, H % 32 == 0, H <= 16384 (checked by the caller).
int launch_add_rmsnorm(const uint16_t* x, const uint16_t* res, const uint16_t* w, int T, int H,
                       float eps, float* yf, uint16_t* yb, uint16_t* rout, uint8_t* q,
                       uint8_t* qs, hipStream_t s) {
  const NormOut o{yf, yb, rout, q, qs};
  const int per = norm_chunks(H);
  if (per <= 1)
    launch_norm<1>(x, res, w, T, H, eps, o, s);
  else if (per <= 2)
    launch_norm<2>(x, res, w, T, H, eps, o, s);
  else if (per <= 4)
    launch_norm<4>(x, res, w, T, H, eps, o, s);
  else
    launch_norm<8>(x, res, w, T, H, eps, o, s);
  return launch_status();
}

// T >= 1, 1 <= k <= 32, H % 256 == 0, H <= 16384 (checked by the caller).
int launch_combine_add_rmsnorm(const uint16_t* y, const int32_t* pair_pos, const float* tw,
                               const uint16_t* shared_y, int T, int k, const uint16_t* res,
                               const uint16_t* w, int H, float eps, uint16_t* out, float* yf,
                               uint16_t* yb, uint16_t* rout, uint8_t* q, uint8_t* qs,
                               hipStream_t s) {
  const NormOut o{yf, yb, rout, q, qs};
  const int per = norm_chunks(H);
  if (per <= 1)
    launch_fused<1>(y, pair_pos, tw, shared_y, T, k, res, w, H, eps, out, o, s);
  else if (per <= 2)
    launch_fused<2>(y, pair_pos, tw, shared_y, T, k, res, w, H, eps, out, o, s);
  else if (per <= 4)
    launch_fused<4>(y, pair_pos, tw, shared_y, T, k, res, w, H, eps, out, o, s);
  else
    launch_fused<8>(y, pair_pos, tw, shared_y, T, k, res, w, H, eps, out, o, s);
  return launch_status();
}

}  // namespace moe
