// Host-side launchers of the kernels (one per step); the C ABI in api.hip
// validates arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// MOE_ERR_LAUNCH (-5) if the runtime reports a launch error, else 0.
inline int launch_status() { return hipGetLastError() == hipSuccess ? 0 : -5; }

// Blocks of `kernel` (launched with `block` threads) that are resident at
// once on the current device: CUs x blocks per CU, rounded up to a multiple
// of 8 and capped by max_tiles (rounded the same way).  The occupancy query
// runs once per (kernel, device) and is cached.
int resident_grid(const void* kernel, int block, long long max_tiles);

// Router workspace (bytes) for T tokens: the split-H partial logits of the
// few-token path (T <= 64), else 0.
size_t router_workspace_bytes(int T, int H, int E);
int launch_router_logits(const uint16_t* x, const float* wr, int T, int H, int E, float* logits,
                         float* ws, hipStream_t s);
// Router logits from fp32 hidden states (any T): split-H partials with fp64
// accumulation, summed in slice order; workspace [H/256, T, E] fp32.
size_t router_f32_workspace_bytes(int T, int H, int E);
int launch_router_logits_f32(const float* x, const float* wr, int T, int H, int E, float* logits,
                             float* ws, hipStream_t s);
// Few-token layer front end (T <= 16, T*k <= 1024): partial logits (+ MXFP8
// x when xq != nullptr; done zeroed when not null), then one block per token
// for its logits and top-k, the last of them also for the counts and the
// permutation (done: the counter router_partial zeroed).
int launch_router_partial(const uint16_t* x, const float* wr, int T, int H, int E,
                          float* partial, uint8_t* xq, uint8_t* xq_scales, int32_t* done,
                          hipStream_t s);
int launch_gate_route_decode(const float* partial, int H, const float* bias, int T, int E, int k,
                             int mode, float routed_scale, float eps, float* logits, int32_t* ids,
                             float* w, int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                             int32_t* pair_pos, int32_t* dev_status, int32_t* done,
                             hipStream_t s);
int launch_gate_topk(const float* logits, const float* bias, int T, int E, int k, int mode,
                     float routed_scale, float eps, int32_t* ids, float* w, hipStream_t s);
// S1 + S2 for the layer: the router's slice partials (in ws, of
// router_workspace_bytes) summed inside the gate, logits stored on the way;
// with xq != nullptr the router kernels also write x's MXFP8 codes and
// scales (S0 of the W4A8 layer).
int launch_router_gate(const uint16_t* x, const float* wr, int T, int H, int E, int k, int mode,
                       float routed_scale, float eps, const float* bias, float* logits,
                       int32_t* ids, float* w, float* ws, uint8_t* xq, uint8_t* xq_scales,
                       hipStream_t s);

size_t route_workspace_bytes(int T, int k, int E);
int launch_route(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pair, int32_t* pair_pos, int32_t* dev_status, int32_t* ws,
                 hipStream_t s);

// One grouped GEMM problem.  Rows of group g are [offsets[g], offsets[g+1])
// (or a single identity group of ident_rows rows when offsets == nullptr).
struct GroupedGemm {
  const void* A;              // activations (bf16 or MXFP8 codes)
  const uint8_t* A_scales;    // MXFP8 scales [rows, K/32] (W4A8 only)
  const int32_t* sorted_pair; // gather: A row of sorted row r = A[sorted_pair[r] / topk]
  int topk;
  int gather;                 // 1: gather A rows through sorted_pair; 0: A row = r
  const int32_t* offsets;
  int G;
  int ident_rows;
  int total_rows;             // upper bound of rows over all groups (T*k or T)
  const void* W;              // per-group weights, [N_w, K] each (bf16 or fp4 codes)
  const uint8_t* W_scales;    // per-group E8M0 scales [N_w, K/32] (W4A8 only)
  long long w_gstride;        // elements (bf16) or bytes (fp4 codes) between groups
  long long ws_gstride;       // scale bytes between groups
  int N;                      // output columns
  int K;                      // reduction length
  int up_off;                 // SwiGLU: row offset of the up half in W (= N)
  void* out;                  // [rows, N] bf16, or MXFP8 codes (W4A8 GEMM1)
  uint8_t* out_scales;        // [rows, N/32] (W4A8 GEMM1)
  // One extra group after the G groups of `offsets` (the shared expert in
  // the routed launch; LDS-tiled bf16 kernels only): xg_rows rows that read
  // activation rows 0.. of xg_A without gather, multiply by xg_W (same shape
  // as one group's W) and write rows 0.. of xg_out.  0 rows: none.
  int xg_rows;
  const void* xg_A;
  const void* xg_W;
  void* xg_out;
};

int launch_ffn_up_bf16(const GroupedGemm& g, bool streamed, hipStream_t s);
int launch_ffn_down_bf16(const GroupedGemm& g, bool streamed, hipStream_t s);
int launch_ffn_up_w4a8(const GroupedGemm& g, bool streamed, hipStream_t s);
int launch_ffn_down_w4a8(const GroupedGemm& g, bool streamed, hipStream_t s);
// LDS-tiled W4A8 GEMMs (128 x 256 block tiles) and the shapes they take.
bool mx_tiled_fits(const GroupedGemm& g, bool swiglu);
void launch_mx_tiled(const GroupedGemm& g, bool swiglu, hipStream_t s);
// bf16 GEMMs for many rows per expert on two waves per SIMD (128 x 256 block
// tiles on eight waves, a DMA ring streaming across tiles) and the shapes
// they take.
bool tiled4_fits(const GroupedGemm& g, bool swiglu);
void launch_tiled4(const GroupedGemm& g, bool swiglu, hipStream_t s);


int launch_mx_quantize(const uint16_t* x, int rows, int cols, uint8_t* codes, uint8_t* scales,
                       hipStream_t s);

// Packed W4A8 weights (layout in mx.hip): scale bytes of one matrix, and the
// pack of G matrices of R x K.
size_t mx_packed_scales_bytes(int rows, int K);
int launch_mx_pack(const uint8_t* codes, const uint8_t* scales, int G, int R, int K,
                   uint8_t* packed_codes, uint8_t* packed_scales, hipStream_t s);

// Residual add + RMSNorm (T >= 1, H % 32 == 0, H <= 16384); any output may be
// null (q and qs together).
int launch_add_rmsnorm(const uint16_t* x, const uint16_t* res, const uint16_t* w, int T, int H,
                       float eps, float* yf, uint16_t* yb, uint16_t* rout, uint8_t* q,
                       uint8_t* qs, hipStream_t s);

// combine (S7) of the layer's expert rows + residual add + RMSNorm of the
// combined rows (T >= 1, 1 <= k <= 32, H % 256 == 0, H <= 16384); out (the
// combined rows) and the norm outputs may each be null.
int launch_combine_add_rmsnorm(const uint16_t* y, const int32_t* pair_pos, const float* tw,
                               const uint16_t* shared_y, int T, int k, const uint16_t* res,
                               const uint16_t* w, int H, float eps, uint16_t* out, float* yf,
                               uint16_t* yb, uint16_t* rout, uint8_t* q, uint8_t* qs,
                               hipStream_t s);

int launch_combine(const uint16_t* y, const int32_t* pair_pos, const float* w,
                   const uint16_t* shared_y, int T, int k, int H, uint16_t* out, hipStream_t s);

}  // namespace moe
