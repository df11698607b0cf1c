// S7: finalize_routing ([Qwen3] "GMM enablement and routing optimisation":
// expert outputs are put back in token order and summed with the top-k
// weights) plus the always-on shared expert's row ([Hy3] section 1.1).
//
// One block per token; each thread owns 8 consecutive hidden elements per
// pass (16-byte loads/stores).  The k slots are accumulated in slot order in
// fp32, so the result does not depend on scheduling.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ shared_y, int k,
                                                      int H, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int pos = pair_pos[(size_t)t * k + j];
      if (pos < 0) continue;
      const float wj = w[(size_t)t * k + j];
      const u32x4 v = ld16(y + (size_t)pos * H + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(wj, bf16_to_f32(v[q] & 0xffffu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wj, bf16_to_f32(v[q] >> 16), acc[2 * q + 1]);
      }
    }
    if (shared_y != nullptr) {
      const u32x4 v = ld16(shared_y + (size_t)t * H + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(v[q] & 0xffffu);
        acc[2 * q + 1] += bf16_to_f32(v[q] >> 16);
      }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    *reinterpret_cast<u32x4*>(out + (size_t)t * H + c) = o;
  }
}

int launch_combine(const uint16_t* y, const int32_t* pair_pos, const float* w,
                   const uint16_t* shared_y, int T, int k, int H, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(256), 0, s, y, pair_pos, w, shared_y, k, H,
                     out);
  return launch_status();
}

}  // namespace moe
