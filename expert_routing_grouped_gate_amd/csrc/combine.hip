// S7: finalize_routing ([Qwen3] "GMM enablement and routing optimisation":
// expert outputs are put back in token order and summed with the top-k
// weights) plus the always-on shared expert's row ([Hy3] section 1.1).
//
// Grid (T, H / 2048): a block covers 2048 hidden elements of one token, each
// thread 8 consecutive ones (16-byte loads/stores).  A token's slot
// positions and weights are read once per block; the rows of up to 8 slots
// are loaded together and then accumulated in slot order in fp32, so the
// result does not depend on scheduling.
#include "common.hpp"
#include "launch.hpp"

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
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int32_t* pp = pair_pos + (size_t)t * k;
  const float* wt = w + (size_t)t * k;
  for (int j0 = 0; j0 < k; j0 += 8) {
    int pos[8];
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      pos[u] = j0 + u < k ? pp[j0 + u] : -1;
      if (pos[u] >= R) pos[u] = -1;  // outside the rows of y: treated as dropped
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = pos[u] >= 0 ? ld16(y + (size_t)pos[u] * H + c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (pos[u] < 0) continue;  // a dropped pair (expert id out of range)
      const float wj = wt[j0 + u];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(wj, bf16_to_f32(v[u][q] & 0xffffu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wj, bf16_to_f32(v[u][q] >> 16), acc[2 * q + 1]);
      }
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

int launch_combine(const uint16_t* y, const int32_t* pair_pos, const float* w,
                   const uint16_t* shared_y, int T, int k, int H, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(T, (H + CB_COLS - 1) / CB_COLS), dim3(256), 0, s, y,
                     pair_pos, w, shared_y, k, H, out);
  return launch_status();
}

}  // namespace moe
