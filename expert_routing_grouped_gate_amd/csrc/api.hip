// C ABI of libmoe: host-side argument checks, then stream-ordered kernel
// launches.  Declarations, argument meaning, layouts and error behaviour are
// documented in include/moe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <unordered_map>

#include "moe.h"
#include "launch.hpp"

namespace moe {

int resident_grid(const void* kernel, int block, long long max_tiles) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int grid;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache[dev].find(kernel);
    if (it != cache[dev].end()) {
      grid = it->second;
    } else {
      int cus = 0, occ = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          cus <= 0)
        cus = 256;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, block, 0) != hipSuccess ||
          occ <= 0)
        occ = 1;
      grid = ((cus * occ + 7) / 8) * 8;
      cache[dev][kernel] = grid;
    }
  }
  const long long cap = ((max_tiles + 7) / 8) * 8;
  return (int)(cap < grid ? cap : grid);
}

}  // namespace moe

// The scratch of moe_layer_forward_noalloc: one copy per GPU, in the device
// code object's zero-initialised data (no file space), loaded with the
// library.  Host code never uses this name as an address (on the host it is
// only a stand-in): scratch_device_ptr() asks the runtime for the address on
// the current GPU once and keeps it per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

using moe::GroupedGemm;

// Device address of `scratch` on the GPU that `stream` runs on (the current
// GPU for the null stream), or nullptr when the runtime cannot give it.
// Looked up once per device, with that device current (switched to and back
// when it is not), and kept.
void* scratch_device_ptr(hipStream_t stream) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = -1;
  if (stream != nullptr) {
    hipDevice_t d = -1;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return nullptr;
    dev = d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
    if (e != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_ptrs(std::initializer_list<const void*> required) {
  for (const void* p : required)
    if (p == nullptr) return MOE_ERR_NULL;
  for (const void* p : required)
    if (!al16(p)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

int check_optional(std::initializer_list<const void*> optional) {
  for (const void* p : optional)
    if (p != nullptr && !al16(p)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

int check_dims_HE(int H, int E) {
  if (H <= 0 || E <= 0) return MOE_ERR_SHAPE;
  if (H % 256 != 0 || E > 256) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_k(int E, int k) {
  if (k <= 0) return MOE_ERR_SHAPE;
  if (k > E || k > 32) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_rows(int T, int k) {
  if (T < 0) return MOE_ERR_SHAPE;
  if ((long long)T * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_weights(const MoeFfnWeights* w) {
  if (w == nullptr) return MOE_ERR_NULL;
  int st = check_dims_HE(w->H, w->E);
  if (st) return st;
  if (w->I <= 0 || w->shared_I < 0) return MOE_ERR_SHAPE;
  if (w->I % 128 != 0 || (w->shared_I % 128) != 0) return MOE_ERR_UNSUPPORTED;
  if (w->fmt == MOE_FMT_BF16) {
    if ((st = check_ptrs({w->w13, w->w2}))) return st;
    if (w->shared_I > 0 && (st = check_ptrs({w->shared_w13, w->shared_w2}))) return st;
    return MOE_OK;
  }
  if (w->fmt == MOE_FMT_W4A8) {
    if ((st = check_ptrs({w->w13, w->w13_scales, w->w2, w->w2_scales}))) return st;
    if (w->shared_I > 0 &&
        (st = check_ptrs({w->shared_w13, w->shared_w13_scales, w->shared_w2, w->shared_w2_scales})))
      return st;
    // one expert's E2M1 matrix (2I x H/2 bytes, H x I/2 for w2) is addressed
    // with 32-bit offsets
    const long long big = (long long)(w->I > w->shared_I ? w->I : w->shared_I) * w->H;
    if (big >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
  }
  return MOE_ERR_UNSUPPORTED;
}

// The weight-streaming GEMMs (16-row tiles, weights straight into MFMA
// operands) or the LDS-tiled ones (128-row tiles).  With at most 16 tokens
// no expert holds more than 16 rows, so streaming reads each touched
// expert's weights exactly once.  Above that the choice follows the
// crossover measured on full-size layers (H = 4096, I = 1536, 128 and 192
// experts, top-8; both paths forced, layer time): bf16 streaming is faster
// up to about 3 rows per expert on average and W4A8 streaming up to about 8
// (each 16-row tile re-reads its expert's weights, but a 128-row W4A8 tile
// costs more MFMA time per padded row than the packed weights take to
// stream); with a bf16 shared expert that the tiled launches take in as one
// more group (fold_shared) the tiled path is faster from 17 tokens on.  The
// choice depends on the weights and T, k only, so the folded launches and
// the separate per-GEMM calls always run the same kernels.
inline bool stream_rows(const MoeFfnWeights* w, int T, int k) {
  if (T <= 16) return true;
  const long long rows = (long long)T * k;
  if (w->fmt == MOE_FMT_W4A8) return rows <= 8ll * w->E;
  const bool shared_folds = w->shared_I > 0 && w->shared_I == w->I;
  return !shared_folds && rows <= 3ll * w->E;
}

GroupedGemm routed_gemm(const MoeFfnWeights* w, int T, int k, const int32_t* sorted_pair,
                        const int32_t* offsets) {
  GroupedGemm g{};
  g.sorted_pair = sorted_pair;
  g.topk = k;
  g.offsets = offsets;
  g.G = w->E;
  g.ident_rows = 0;
  g.total_rows = T * k;
  return g;
}

GroupedGemm up_gemm(const MoeFfnWeights* w, const void* x, const uint8_t* x_scales, int T, int k,
                    const int32_t* sorted_pair, const int32_t* offsets, void* act, uint8_t* act_scales) {
  GroupedGemm g = routed_gemm(w, T, k, sorted_pair, offsets);
  g.A = x;
  g.A_scales = x_scales;
  g.gather = 1;
  g.W = w->w13;
  g.W_scales = w->w13_scales;
  g.N = w->I;
  g.K = w->H;
  g.up_off = w->I;
  g.out = act;
  g.out_scales = act_scales;
  if (w->fmt == MOE_FMT_W4A8) {
    g.w_gstride = (long long)w->I * w->H;  // bytes: 2I rows of H/2
    g.ws_gstride = (long long)moe::mx_packed_scales_bytes(2 * w->I, w->H);
  } else {
    g.w_gstride = 2ll * w->I * w->H;
  }
  return g;
}

GroupedGemm down_gemm(const MoeFfnWeights* w, const void* act, const uint8_t* act_scales, int T, int k,
                      const int32_t* offsets, uint16_t* y) {
  GroupedGemm g = routed_gemm(w, T, k, nullptr, offsets);
  g.A = act;
  g.A_scales = act_scales;
  g.gather = 0;
  g.W = w->w2;
  g.W_scales = w->w2_scales;
  g.N = w->H;
  g.K = w->I;
  g.up_off = 0;
  g.out = y;
  if (w->fmt == MOE_FMT_W4A8) {
    g.w_gstride = (long long)w->H * (w->I / 2);
    g.ws_gstride = (long long)moe::mx_packed_scales_bytes(w->H, w->I);
  } else {
    g.w_gstride = (long long)w->H * w->I;
  }
  return g;
}

// The shared expert run inside the routed grouped GEMMs as one more group
// ([Hy3] section 1.1: one always-on shared expert; the survey of this layer
// plans it as an extra group of the grouped matmul): its T rows read x (and
// then its own activations) without gather and its tiles join the routed
// tile list, so no separate, partly empty launch runs after the routed ones.
// Taken for bf16 weights with shared_I == I when both GEMMs run on the
// LDS-tiled kernels (more than 16 tokens); else the caller launches the
// shared expert on its own.  Fills the extra-group fields of up / dn.
bool fold_shared(const MoeFfnWeights* w, int T, int k, const void* x, void* shared_act,
                 uint16_t* shared_y, GroupedGemm& up, GroupedGemm& dn) {
  if (w->fmt != MOE_FMT_BF16 || w->shared_I <= 0 || w->shared_I != w->I) return false;
  if (stream_rows(w, T, k)) return false;
  up.xg_rows = T;
  up.xg_A = x;
  up.xg_W = w->shared_w13;
  up.xg_out = shared_act;
  dn.xg_rows = T;
  dn.xg_A = shared_act;
  dn.xg_W = w->shared_w2;
  dn.xg_out = shared_y;
  if (moe::tiled4_fits(up, true) && moe::tiled4_fits(dn, false)) return true;
  up.xg_rows = dn.xg_rows = 0;
  return false;
}

}  // namespace

extern "C" {

const char* moe_status_string(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is negative or inconsistent";
    case MOE_ERR_UNSUPPORTED: return "outside the supported limits, or unknown mode/format";
    case MOE_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case MOE_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_SCRATCH: return "the call needs more than the library's static scratch";
    default: return "unknown status";
  }
}

size_t moe_router_workspace_size(int T, int H, int E) {
  if (T <= 0 || check_dims_HE(H, E) != MOE_OK) return 0;
  return moe::router_workspace_bytes(T, H, E);
}

int moe_router_logits(const uint16_t* x, const float* wr, int T, int H, int E, float* logits,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int st;
  if ((st = check_dims_HE(H, E))) return st;
  if (T < 0) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if ((st = check_ptrs({x, wr, logits}))) return st;
  const size_t need = moe::router_workspace_bytes(T, H, E);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    if (!al16(workspace)) return MOE_ERR_ALIGN;
  }
  return moe::launch_router_logits(x, wr, T, H, E, logits, static_cast<float*>(workspace),
                                   as_stream(stream));
}

size_t moe_router_f32_workspace_size(int T, int H, int E) {
  if (T <= 0 || check_dims_HE(H, E) != MOE_OK) return 0;
  return moe::router_f32_workspace_bytes(T, H, E);
}

int moe_router_logits_f32(const float* x, const float* wr, int T, int H, int E, float* logits,
                          void* workspace, size_t workspace_bytes, void* stream) {
  int st;
  if ((st = check_dims_HE(H, E))) return st;
  if (T < 0) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if ((long long)T * E >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if ((st = check_ptrs({x, wr, logits}))) return st;
  const size_t need = moe::router_f32_workspace_bytes(T, H, E);
  if (workspace == nullptr || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (!al16(workspace)) return MOE_ERR_ALIGN;
  return moe::launch_router_logits_f32(x, wr, T, H, E, logits, static_cast<float*>(workspace),
                                       as_stream(stream));
}

int moe_gate_topk(const float* logits, const float* bias, int T, int E, int k, int mode,
                  float routed_scale, float eps, int32_t* topk_ids, float* topk_w,
                  void* stream) {
  int st;
  if (E <= 0) return MOE_ERR_SHAPE;
  if (E > 256) return MOE_ERR_UNSUPPORTED;
  if ((st = check_k(E, k))) return st;
  if ((st = check_rows(T, k))) return st;
  if (mode != MOE_GATE_SOFTMAX && mode != MOE_GATE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if ((st = check_ptrs({logits, topk_ids, topk_w}))) return st;
  if ((st = check_optional({bias}))) return st;
  return moe::launch_gate_topk(logits, bias, T, E, k, mode, routed_scale, eps, topk_ids, topk_w,
                               as_stream(stream));
}

size_t moe_route_workspace_size(int T, int k, int E) {
  if (T <= 0 || k <= 0 || E <= 0) return 0;
  return moe::route_workspace_bytes(T, k, E);
}

int moe_route(const int32_t* topk_ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
              int32_t* sorted_pair, int32_t* pair_pos, int32_t* dev_status, void* workspace,
              size_t workspace_bytes, void* stream) {
  int st;
  if (E <= 0) return MOE_ERR_SHAPE;
  if (E > 256) return MOE_ERR_UNSUPPORTED;
  if ((st = check_k(E, k))) return st;
  if ((st = check_rows(T, k))) return st;
  if ((st = check_ptrs({counts, offsets}))) return st;
  if ((st = check_optional({dev_status}))) return st;
  if (T > 0 && (st = check_ptrs({topk_ids, sorted_pair, pair_pos}))) return st;
  const size_t need = moe::route_workspace_bytes(T, k, E);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    if (!al16(workspace)) return MOE_ERR_ALIGN;
  }
  if (T == 0) return MOE_OK;
  return moe::launch_route(topk_ids, T, k, E, counts, offsets, sorted_pair, pair_pos, dev_status,
                           static_cast<int32_t*>(workspace), as_stream(stream));
}

int moe_mx_quantize(const uint16_t* x, int rows, int cols, uint8_t* codes, uint8_t* scales,
                    void* stream) {
  int st;
  if (rows < 0 || cols <= 0) return MOE_ERR_SHAPE;
  if (cols % 32 != 0 || (long long)rows * cols >= (1ll << 40)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if ((st = check_ptrs({x, codes, scales}))) return st;
  return moe::launch_mx_quantize(x, rows, cols, codes, scales, as_stream(stream));
}

size_t moe_mx_packed_scales_bytes(int rows, int K) {
  if (rows <= 0 || K <= 0 || rows % 16 != 0 || K % 128 != 0) return 0;
  return moe::mx_packed_scales_bytes(rows, K);
}

int moe_mx_pack_weight(const uint8_t* codes, const uint8_t* scales, int G, int rows, int K,
                       uint8_t* packed_codes, uint8_t* packed_scales, void* stream) {
  int st;
  if (G < 0 || rows <= 0 || K <= 0) return MOE_ERR_SHAPE;
  if (rows % 16 != 0 || K % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (G == 0) return MOE_OK;
  if ((st = check_ptrs({codes, scales, packed_codes, packed_scales}))) return st;
  return moe::launch_mx_pack(codes, scales, G, rows, K, packed_codes, packed_scales,
                             as_stream(stream));
}

int moe_grouped_ffn_up(const MoeFfnWeights* w, const void* x, const uint8_t* x_scales, int T,
                       int k, const int32_t* sorted_pair, const int32_t* offsets, void* act,
                       uint8_t* act_scales, void* stream) {
  int st;
  if ((st = check_weights(w))) return st;
  if ((st = check_k(w->E, k))) return st;
  if ((st = check_rows(T, k))) return st;
  if (T == 0) return MOE_OK;
  if ((st = check_ptrs({x, sorted_pair, offsets, act}))) return st;
  const bool mx = w->fmt == MOE_FMT_W4A8;
  if (mx && (st = check_ptrs({x_scales, act_scales}))) return st;
  const GroupedGemm g = up_gemm(w, x, x_scales, T, k, sorted_pair, offsets, act, act_scales);
  const bool sm = stream_rows(w, T, k);
  return mx ? moe::launch_ffn_up_w4a8(g, sm, as_stream(stream))
            : moe::launch_ffn_up_bf16(g, sm, as_stream(stream));
}

int moe_grouped_ffn_down(const MoeFfnWeights* w, const void* act, const uint8_t* act_scales,
                         int T, int k, const int32_t* offsets, uint16_t* y, void* stream) {
  int st;
  if ((st = check_weights(w))) return st;
  if ((st = check_k(w->E, k))) return st;
  if ((st = check_rows(T, k))) return st;
  if (T == 0) return MOE_OK;
  if ((st = check_ptrs({act, offsets, y}))) return st;
  const bool mx = w->fmt == MOE_FMT_W4A8;
  if (mx && (st = check_ptrs({act_scales}))) return st;
  const GroupedGemm g = down_gemm(w, act, act_scales, T, k, offsets, y);
  const bool sm = stream_rows(w, T, k);
  return mx ? moe::launch_ffn_down_w4a8(g, sm, as_stream(stream))
            : moe::launch_ffn_down_bf16(g, sm, as_stream(stream));
}

int moe_shared_ffn(const MoeFfnWeights* w, const void* x, const uint8_t* x_scales, int T,
                   void* shared_act, uint8_t* shared_act_scales, uint16_t* shared_y,
                   void* stream) {
  int st;
  if ((st = check_weights(w))) return st;
  if (w->shared_I <= 0) return MOE_ERR_SHAPE;
  if (T < 0) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if ((st = check_ptrs({x, shared_act, shared_y}))) return st;
  const bool mx = w->fmt == MOE_FMT_W4A8;
  if (mx && (st = check_ptrs({x_scales, shared_act_scales}))) return st;
  GroupedGemm g{};
  g.offsets = nullptr;
  g.G = 1;
  g.ident_rows = T;
  g.total_rows = T;
  g.gather = 0;
  g.A = x;
  g.A_scales = x_scales;
  g.W = w->shared_w13;
  g.W_scales = w->shared_w13_scales;
  g.w_gstride = 0;
  g.ws_gstride = 0;
  g.N = w->shared_I;
  g.K = w->H;
  g.up_off = w->shared_I;
  g.out = shared_act;
  g.out_scales = shared_act_scales;
  const bool sm = T <= 16;
  st = mx ? moe::launch_ffn_up_w4a8(g, sm, as_stream(stream)) : moe::launch_ffn_up_bf16(g, sm, as_stream(stream));
  if (st) return st;
  GroupedGemm d = g;
  d.A = shared_act;
  d.A_scales = shared_act_scales;
  d.W = w->shared_w2;
  d.W_scales = w->shared_w2_scales;
  d.N = w->H;
  d.K = w->shared_I;
  d.up_off = 0;
  d.out = shared_y;
  d.out_scales = nullptr;
  return mx ? moe::launch_ffn_down_w4a8(d, sm, as_stream(stream)) : moe::launch_ffn_down_bf16(d, sm, as_stream(stream));
}

int moe_grouped_ffn(const MoeFfnWeights* w, const void* x, const uint8_t* x_scales, int T, int k,
                    const int32_t* sorted_pair, const int32_t* offsets, void* act,
                    uint8_t* act_scales, uint16_t* y, void* shared_act,
                    uint8_t* shared_act_scales, uint16_t* shared_y, void* stream) {
  if (w != nullptr && w->shared_I > 0 && shared_y != nullptr && T > 0 && check_weights(w) == MOE_OK &&
      check_k(w->E, k) == MOE_OK && check_rows(T, k) == MOE_OK &&
      check_ptrs({x, sorted_pair, offsets, act, y, shared_act, shared_y}) == MOE_OK) {
    GroupedGemm up = up_gemm(w, x, x_scales, T, k, sorted_pair, offsets, act, act_scales);
    GroupedGemm dn = down_gemm(w, act, act_scales, T, k, offsets, y);
    if (fold_shared(w, T, k, x, shared_act, shared_y, up, dn)) {
      moe::launch_tiled4(up, true, as_stream(stream));
      int st = moe::launch_status();
      if (st) return st;
      moe::launch_tiled4(dn, false, as_stream(stream));
      return moe::launch_status();
    }
  }
  int st = moe_grouped_ffn_up(w, x, x_scales, T, k, sorted_pair, offsets, act, act_scales, stream);
  if (st) return st;
  st = moe_grouped_ffn_down(w, act, act_scales, T, k, offsets, y, stream);
  if (st) return st;
  if (w->shared_I > 0 && shared_y != nullptr)
    st = moe_shared_ffn(w, x, x_scales, T, shared_act, shared_act_scales, shared_y, stream);
  return st;
}

int moe_add_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* weight, int T,
                    int H, float eps, float* y_f32, uint16_t* y_bf16, uint16_t* residual_out,
                    uint8_t* y_mx, uint8_t* y_mx_scales, void* stream) {
  int st;
  if (T < 0 || H <= 0) return MOE_ERR_SHAPE;
  if (H % 32 != 0 || H > 16384) return MOE_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || eps == __builtin_inff()) return MOE_ERR_SHAPE;  // also rejects NaN
  if (T == 0) return MOE_OK;
  if ((y_mx == nullptr) != (y_mx_scales == nullptr)) return MOE_ERR_NULL;
  if (!y_f32 && !y_bf16 && !residual_out && !y_mx) return MOE_ERR_NULL;
  if ((st = check_ptrs({x, weight}))) return st;
  if ((st = check_optional({residual, y_f32, y_bf16, residual_out, y_mx, y_mx_scales}))) return st;
  return moe::launch_add_rmsnorm(x, residual, weight, T, H, eps, y_f32, y_bf16, residual_out, y_mx,
                                 y_mx_scales, as_stream(stream));
}

int moe_combine_add_rmsnorm(const uint16_t* y, const int32_t* pair_pos, const float* topk_w,
                            const uint16_t* shared_y, int T, int k, int H,
                            const uint16_t* residual, const uint16_t* weight, float eps,
                            uint16_t* out, float* y_f32, uint16_t* y_bf16, uint16_t* residual_out,
                            uint8_t* y_mx, uint8_t* y_mx_scales, void* stream) {
  int st;
  if (H <= 0 || k <= 0) return MOE_ERR_SHAPE;
  if (H % 256 != 0 || H > 16384 || k > 32) return MOE_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || eps == __builtin_inff()) return MOE_ERR_SHAPE;  // also rejects NaN
  if ((st = check_rows(T, k))) return st;
  if (T == 0) return MOE_OK;
  if ((y_mx == nullptr) != (y_mx_scales == nullptr)) return MOE_ERR_NULL;
  if (!out && !y_f32 && !y_bf16 && !residual_out && !y_mx) return MOE_ERR_NULL;
  if ((st = check_ptrs({y, pair_pos, topk_w, weight}))) return st;
  if ((st = check_optional({shared_y, residual, out, y_f32, y_bf16, residual_out, y_mx, y_mx_scales})))
    return st;
  return moe::launch_combine_add_rmsnorm(y, pair_pos, topk_w, shared_y, T, k, residual, weight, H,
                                         eps, out, y_f32, y_bf16, residual_out, y_mx, y_mx_scales,
                                         as_stream(stream));
}

int moe_combine(const uint16_t* y, const int32_t* pair_pos, const float* topk_w,
                const uint16_t* shared_y, int T, int k, int H, uint16_t* out, void* stream) {
  int st;
  if (H <= 0) return MOE_ERR_SHAPE;
  if (H % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (k <= 0) return MOE_ERR_SHAPE;
  if (k > 32) return MOE_ERR_UNSUPPORTED;
  if ((st = check_rows(T, k))) return st;
  if (T == 0) return MOE_OK;
  if ((st = check_ptrs({y, pair_pos, topk_w, out}))) return st;
  if ((st = check_optional({shared_y}))) return st;
  return moe::launch_combine(y, pair_pos, topk_w, shared_y, T, k, H, out, as_stream(stream));
}

// Decode front end: the router's partial sums, then (at the next 256-byte
// boundary) the gate blocks' done counter.
static bool decode_front(int T, int k) { return T <= 16 && T * k <= 1024; }
static size_t decode_counter_offset(int T, const MoeLayerDesc* d) {
  return (moe_router_workspace_size(T, d->H, d->E) + 255) / 256 * 256;
}

size_t moe_layer_workspace_size(const MoeLayerDesc* d, int T) {
  if (d == nullptr || T <= 0) return 0;
  // the router's partial sums and the routing histograms are live at
  // different times and share the space
  const size_t r = decode_front(T, d->k) ? decode_counter_offset(T, d) + 256
                                         : moe_router_workspace_size(T, d->H, d->E);
  const size_t h = moe_route_workspace_size(T, d->k, d->E);
  return r > h ? r : h;
}

size_t moe_workspace_size(const MoeLayerDesc* d, int T) { return moe_layer_workspace_size(d, T); }

int moe_layer_forward(const MoeLayerDesc* d, const uint16_t* x, int T, uint16_t* out,
                      const MoeLayerBuffers* b, void* stream) {
  int st;
  if (d == nullptr || b == nullptr) return MOE_ERR_NULL;
  if ((st = check_weights(&d->ffn))) return st;
  if (d->ffn.H != d->H || d->ffn.E != d->E) return MOE_ERR_SHAPE;
  if ((st = check_k(d->E, d->k))) return st;
  if ((st = check_rows(T, d->k))) return st;
  if (d->gate_mode != MOE_GATE_SOFTMAX && d->gate_mode != MOE_GATE_SIGMOID)
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if ((st = check_ptrs({x, out, d->wr, b->logits, b->topk_ids, b->topk_w, b->counts, b->offsets,
                        b->sorted_pair, b->pair_pos, b->act, b->y}))) return st;
  if ((st = check_optional({d->bias, b->dev_status}))) return st;
  const bool shared = d->ffn.shared_I > 0;
  const bool mx = d->ffn.fmt == MOE_FMT_W4A8;
  if (shared && (st = check_ptrs({b->shared_act, b->shared_y}))) return st;
  if (mx && (st = check_ptrs({b->xq, b->xq_scales, b->act_scales}))) return st;
  if (mx && shared && (st = check_ptrs({b->shared_act_scales}))) return st;
  const size_t need = moe_layer_workspace_size(d, T);
  if (need > 0) {
    if (b->workspace == nullptr || b->workspace_bytes < need) return MOE_ERR_WORKSPACE;
    if (!al16(b->workspace)) return MOE_ERR_ALIGN;
  }
  const int k = d->k;
  const void* xin = mx ? static_cast<const void*>(b->xq) : static_cast<const void*>(x);
  const uint8_t* xin_s = mx ? b->xq_scales : nullptr;
  if (decode_front(T, k)) {
    // decode: router partials (+ MXFP8 x), then a block per token for its
    // top-k, the last one also for the routing
    hipStream_t s = as_stream(stream);
    float* part = static_cast<float*>(b->workspace);
    int32_t* done = reinterpret_cast<int32_t*>(static_cast<char*>(b->workspace) +
                                               decode_counter_offset(T, d));
    if ((st = moe::launch_router_partial(x, d->wr, T, d->H, d->E, part, mx ? b->xq : nullptr,
                                         mx ? b->xq_scales : nullptr, done, s)))
      return st;
    if ((st = moe::launch_gate_route_decode(part, d->H, d->bias, T, d->E, k, d->gate_mode,
                                            d->routed_scale, d->eps, b->logits, b->topk_ids,
                                            b->topk_w, b->counts, b->offsets, b->sorted_pair,
                                            b->pair_pos, b->dev_status, done, s)))
      return st;
  } else {
    // router (+ the MXFP8 codes of x for W4A8) and gate (the router's slice
    // partials are summed inside the gate)
    if ((st = moe::launch_router_gate(x, d->wr, T, d->H, d->E, k, d->gate_mode, d->routed_scale,
                                      d->eps, d->bias, b->logits, b->topk_ids, b->topk_w,
                                      static_cast<float*>(b->workspace), mx ? b->xq : nullptr,
                                      mx ? b->xq_scales : nullptr, as_stream(stream))))
      return st;
    if ((st = moe_route(b->topk_ids, T, k, d->E, b->counts, b->offsets, b->sorted_pair,
                        b->pair_pos, b->dev_status, b->workspace, b->workspace_bytes, stream)))
      return st;
  }
  hipEvent_t ev0 = reinterpret_cast<hipEvent_t>(b->ev_ffn_up_begin);
  hipEvent_t ev1 = reinterpret_cast<hipEvent_t>(b->ev_ffn_up_end);
  const bool timed = ev0 != nullptr && ev1 != nullptr;
  GroupedGemm up = up_gemm(&d->ffn, xin, xin_s, T, k, b->sorted_pair, b->offsets, b->act, b->act_scales);
  GroupedGemm dn = down_gemm(&d->ffn, b->act, b->act_scales, T, k, b->offsets, b->y);
  const bool folded = shared && fold_shared(&d->ffn, T, k, xin, b->shared_act, b->shared_y, up, dn);
  if (timed && hipEventRecord(ev0, as_stream(stream)) != hipSuccess) return MOE_ERR_LAUNCH;
  if (folded) {
    moe::launch_tiled4(up, true, as_stream(stream));
    if ((st = moe::launch_status())) return st;
  } else if ((st = moe_grouped_ffn_up(&d->ffn, xin, xin_s, T, k, b->sorted_pair, b->offsets, b->act,
                                      b->act_scales, stream))) {
    return st;
  }
  if (timed && hipEventRecord(ev1, as_stream(stream)) != hipSuccess) return MOE_ERR_LAUNCH;
  if (folded) {
    moe::launch_tiled4(dn, false, as_stream(stream));
    if ((st = moe::launch_status())) return st;
  } else {
    if ((st = moe_grouped_ffn_down(&d->ffn, b->act, b->act_scales, T, k, b->offsets, b->y, stream)))
      return st;
    if (shared && (st = moe_shared_ffn(&d->ffn, xin, xin_s, T, b->shared_act, b->shared_act_scales,
                                       b->shared_y, stream)))
      return st;
  }
  return moe_combine(b->y, b->pair_pos, b->topk_w, shared ? b->shared_y : nullptr, T, k, d->H,
                     out, stream);
}

int moe_layer_forward_noalloc(const MoeLayerDesc* d, const uint16_t* x, int T, uint16_t* out,
                              const MoeLayerBuffers* b, void* stream) {
  if (d == nullptr || b == nullptr) return MOE_ERR_NULL;
  if (T < 0) return MOE_ERR_SHAPE;
  if (moe_layer_workspace_size(d, T) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  MoeLayerBuffers s = *b;
  s.workspace = nullptr;
  s.workspace_bytes = 0;
  if (T > 0) {
    // moe_layer_forward validates everything else before it enqueues
    void* p = scratch_device_ptr(as_stream(stream));
    if (p == nullptr) return MOE_ERR_LAUNCH;
    s.workspace = p;
    s.workspace_bytes = MOE_NOALLOC_SCRATCH_BYTES;
  }
  return moe_layer_forward(d, x, T, out, &s, stream);
}

}  // extern "C"
