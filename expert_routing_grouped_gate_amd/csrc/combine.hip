// S7: finalize_routing ([Qwen3] "GMM enablement and routing optimisation":
// expert outputs are put back in token order and summed with the top-k
// weights) plus the always-on shared expert's row ([Hy3] section 1.1).
//
// Grid (T, H / 2048): a block covers 2048 hidden elements of one token, each
// thread 8 consecutive ones (16-byte loads/stores, combine_chunks: the rows
// of up to 8 slots loaded together, then accumulated in slot order in fp32,
// so the result does not depend on scheduling).
#include "common.hpp"
#include "launch.hpp"
#include "rowops.hpp"

namespace moe {

constexpr int CB_COLS = 2048;  // hidden elements per block

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ shared_y, int k,
                                                      int H, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int R = (int)gridDim.x * k;
  const int c = blockIdx.y * CB_COLS + threadIdx.x * 8;
  if (c >= H) return;  // no barriers below
  u32x4 o[1];
  combine_chunks<1>(y, pair_pos + (size_t)t * k, w + (size_t)t * k,
                    shared_y ? shared_y + (size_t)t * H : nullptr, k, R, H, c, o);
  *reinterpret_cast<u32x4*>(out + (size_t)t * H + c) = o[0];
}

int launch_combine(const uint16_t* y, const int32_t* pair_pos, const float* w,
                   const uint16_t* shared_y, int T, int k, int H, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(T, (H + CB_COLS - 1) / CB_COLS), dim3(256), 0, s, y,
                     pair_pos, w, shared_y, k, H, out);
  return launch_status();
}

}  // namespace moe
