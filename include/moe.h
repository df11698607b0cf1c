/*
 * moe.h - C ABI of libmoe, a sparse Mixture-of-Experts layer forward for
 * AMD MI355X (gfx950), written in HIP.
 *
 * Sources.  Page titles are abbreviated:
 *   [Qwen3] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters"
 *           (基于Atlas A3、950训练/推理集群的Qwen3-MoE模型低时延推理性能优化实践)
 *   [Hy3]   "Hy3 295B MoE on Atlas A3: end-to-end inference optimisation"
 *           (cann-recipes-infer：Hy3 295B MoE 大模型在 Atlas A3 平台的端到端推理优化实践)
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     the descriptor structs themselves, which are host memory read during
 *     the call only.  The library allocates and frees nothing.
 *   - bf16 tensors travel as uint16_t bit patterns; ids, counts, offsets and
 *     permutations are int32; MX element codes and E8M0 scales are uint8.
 *   - Every tensor is dense row-major (last index fastest) and every device
 *     pointer must be 16-byte aligned (MOE_ERR_ALIGN otherwise).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues kernels on that stream and returns; no call synchronises, reads
 *     device memory on the host or allocates, so every call can be captured
 *     into a HIP graph.
 *   - Host-side argument checks run before anything is enqueued and return a
 *     negative moe_status; nothing is enqueued on error.  A failed launch
 *     returns MOE_ERR_LAUNCH.  Data errors that only the device can see
 *     (an expert id outside [0, E)) are reported in a device status word.
 *   - T == 0 (no tokens) is valid and enqueues nothing.
 *   - Limits: 1 <= k <= min(E, 32); 1 <= E <= 256; H % 256 == 0;
 *     I % 128 == 0; T * k < 2^31; W4A8: max(I, shared_I) * H < 2^31 (one
 *     expert's E2M1 matrix is addressed with 32-bit offsets).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* a size is negative or inconsistent */
  MOE_ERR_UNSUPPORTED = -3, /* outside the limits above, or unknown mode/format */
  MOE_ERR_ALIGN = -4,       /* a device pointer is not 16-byte aligned */
  MOE_ERR_LAUNCH = -5,      /* the HIP runtime rejected a kernel launch */
  MOE_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required */
  MOE_ERR_SCRATCH = -7      /* the call needs more than the library's static scratch */
} moe_status;

/* Gating modes (S2). */
typedef enum {
  /* [Qwen3] "GMM enablement and routing optimisation": fused gating top-k
   * softmax.  key = logit (+ bias, added in fp32); the k largest keys are
   * selected; weights = softmax over the selected keys. */
  MOE_GATE_SOFTMAX = 0,
  /* [Hy3] section 1.3 and 5.1: s = sigmoid(logit); key = s + bias decides
   * selection only; weight = s / (sum of selected s + eps) * routed_scale.
   * s and key are computed and compared in fp64. */
  MOE_GATE_SIGMOID = 1
} moe_gate_mode;

/* Weight / activation formats. */
typedef enum {
  MOE_FMT_BF16 = 0, /* bf16 weights and activations, fp32 accumulation */
  /* [Qwen3] overview and "MoE EP optimisation (AllGather scheme, W4A8)":
   * MXFP4 (E2M1) weights with one E8M0 scale per 32 along K; activations
   * dynamically quantised to MXFP8 (E4M3FN) per 32 along K. */
  MOE_FMT_W4A8 = 1
} moe_format;

/* Bits of the device status word written by moe_route. */
#define MOE_DEV_BAD_EXPERT_ID 1 /* some topk id was outside [0, E) */

/* Human-readable text for a moe_status value (static storage). */
const char* moe_status_string(int code);

/* ------------------------------------------------------------- S1 -----
 * Router logits ([Qwen3] "fused RMSNorm + Cast": the gate runs in fp32).
 *   logits[t, e] = sum_h float(x[t, h]) * wr[e, h], fp32 accumulation.
 *   x      [T, H] bf16
 *   wr     [E, H] fp32
 *   logits [T, E] fp32 (output)
 *   workspace  device scratch of moe_router_workspace_size(T, H, E) bytes
 *              (few tokens: per-slice partial sums over H; may be NULL when
 *              that size is 0); MOE_ERR_WORKSPACE when too small.
 * Deterministic: the summation order of each output is fixed. */
size_t moe_router_workspace_size(int T, int H, int E);
int moe_router_logits(const uint16_t* x, const float* wr, int T, int H, int E,
                      float* logits, void* workspace, size_t workspace_bytes, void* stream);

/* S1 from fp32 hidden states ([Qwen3] "fused RMSNorm + Cast": the norm before
 * the MoE block gives the gate an FP32 copy of the hidden states, e.g. the
 * y_f32 output of moe_add_rmsnorm).  L[t, e] = sum_h x[t, h] * wr[e, h]; the
 * products and their sums over each 256-column slice of H are taken in
 * fp64 and rounded to fp32 once, the slices are then added in order in fp32.
 *   x      [T, H] fp32
 *   wr     [E, H] fp32
 *   logits [T, E] fp32 (output)
 *   workspace  device scratch of moe_router_f32_workspace_size(T, H, E) bytes
 *              (the per-slice sums, [H/256, T, E] fp32); MOE_ERR_WORKSPACE when
 *              missing or too small.
 * Limits as moe_router_logits (H % 256 == 0, E <= 256), T * E < 2^31.
 * Deterministic: the summation order of each output is fixed. */
size_t moe_router_f32_workspace_size(int T, int H, int E);
int moe_router_logits_f32(const float* x, const float* wr, int T, int H, int E, float* logits,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------- S2 -----
 * Gate top-k ([Qwen3] gating top-k softmax; [Hy3] section 1.3 router call
 * with k, bias, sigmoid norm type, routed_scaling_factor and eps).
 *   logits   [T, E] fp32
 *   bias     [E] fp32 or NULL.  Softmax mode: added to the logits (affects
 *            selection and weights).  Sigmoid mode: added to s for selection
 *            only.
 *   routed_scale  multiplies the sigmoid-mode weights (2.826 for Hy3);
 *            ignored in softmax mode.
 *   eps      added to the sigmoid-mode denominator (1e-20 for Hy3).
 *   topk_ids [T, k] int32 (output); slots ordered by key descending, ties to
 *            the lower expert id.  NaN logits count as -infinity.
 *   topk_w   [T, k] fp32 (output), computed in fp64 and rounded. */
int moe_gate_topk(const float* logits, const float* bias, int T, int E, int k,
                  int mode, float routed_scale, float eps,
                  int32_t* topk_ids, float* topk_w, void* stream);

/* ---------------------------------------------------------- S3, S4 -----
 * init_routing + compute_expert_tokens ([Qwen3] "GMM enablement and routing
 * optimisation"; [Hy3] section 6.2: the grouped matmul's group_list is the
 * per-expert token count).
 *   topk_ids    [T, k] int32
 *   counts      [E]    int32 (output) pairs per expert
 *   offsets     [E+1]  int32 (output) exclusive prefix sum of counts;
 *               offsets[E] = number of valid pairs
 *   sorted_pair [T*k]  int32 (output) pair indices p = t*k + j grouped by
 *               expert, ascending p within an expert (stable sort)
 *   pair_pos    [T*k]  int32 (output) inverse: pair_pos[sorted_pair[r]] = r;
 *               -1 for a pair whose id is out of range
 *   dev_status  [1] int32 or NULL (output): MOE_DEV_BAD_EXPERT_ID if any id
 *               is outside [0, E), else 0.  Pairs with such ids are dropped
 *               (not counted, not placed).
 *   workspace   device scratch of moe_route_workspace_size(T, k, E) bytes
 *               (may be NULL when that size is 0). */
size_t moe_route_workspace_size(int T, int k, int E);
int moe_route(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
              int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
              int32_t* dev_status, void* workspace, size_t workspace_bytes,
              void* stream);

/* ----------------------------------------------- before the layer -----
 * Residual add + RMSNorm in one pass, with the outputs the MoE layer takes
 * ([Qwen3] "fused-operator optimisation": "fused RMSNorm + MX quant" and
 * "fused RMSNorm + Cast" (FP32 for the gate, BF16 for the experts, plus the
 * updated residual); the formula as written in the "LLM inference
 * optimisation study note", section 2, "Add and RMSNorm").  Per row:
 *   z = x + residual (x alone when residual is NULL), in fp32;
 *   y_i = z_i / sqrt(mean_j z_j^2 + eps) * weight_i (sum of squares in
 *   fp32, the reciprocal root in fp64, the products in fp32).
 *   x            [T, H] bf16
 *   residual     [T, H] bf16, or NULL (first layer)
 *   weight       [H] bf16 (the norm's gamma)
 *   eps          >= 0 and finite (variance epsilon)
 * Outputs, each may be NULL (at least one must be given):
 *   y_f32        [T, H] fp32: y (the gate's input)
 *   y_bf16       [T, H] bf16: y rounded to nearest even (the experts' input)
 *   residual_out [T, H] bf16: z rounded to nearest even (the next layer's
 *                residual)
 *   y_mx, y_mx_scales  [T, H] uint8 E4M3 codes + [T, H/32] uint8 E8M0 scales
 *                of y quantised with the rule of moe_mx_quantize (both or
 *                neither)
 * No output may overlap an input.  Limits: H % 32 == 0, H <= 16384.  T == 0
 * enqueues nothing.  Errors: MOE_ERR_NULL (x or weight NULL, no output, or
 * only one of y_mx / y_mx_scales), MOE_ERR_SHAPE (T < 0, H <= 0, eps negative
 * or not finite), MOE_ERR_UNSUPPORTED (H outside the limits), MOE_ERR_ALIGN. */
int moe_add_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* weight, int T,
                    int H, float eps, float* y_f32, uint16_t* y_bf16, uint16_t* residual_out,
                    uint8_t* y_mx, uint8_t* y_mx_scales, void* stream);

/* S7 fused with the next step's residual add + RMSNorm: the layer's output
 * feeds the next norm without a round trip through memory ([Qwen3]
 * "fused-operator optimisation": fusing to avoid writing and re-reading
 * intermediate results).  Per token row: out = moe_combine's row (fp32 slot
 * order, + shared row, rounded to bf16), then moe_add_rmsnorm of out with
 * `residual`.  Every output equals moe_combine followed by moe_add_rmsnorm
 * bit for bit.
 *   y, pair_pos, topk_w, shared_y, T, k, H   as moe_combine
 *   residual, weight, eps                    as moe_add_rmsnorm (x = out)
 *   out          [T, H] bf16 layer output, or NULL (not stored)
 *   y_f32, y_bf16, residual_out, y_mx, y_mx_scales   as moe_add_rmsnorm
 * At least one output must be given.  No output may overlap an input.
 * Limits: H % 256 == 0, H <= 16384, 1 <= k <= 32.  T == 0 enqueues nothing. */
int moe_combine_add_rmsnorm(const uint16_t* y, const int32_t* pair_pos, const float* topk_w,
                            const uint16_t* shared_y, int T, int k, int H,
                            const uint16_t* residual, const uint16_t* weight, float eps,
                            uint16_t* out, float* y_f32, uint16_t* y_bf16, uint16_t* residual_out,
                            uint8_t* y_mx, uint8_t* y_mx_scales, void* stream);

/* ------------------------------------------------------------- S0 -----
 * Dynamic MXFP8 quantisation ([Qwen3] "MoE EP optimisation": hidden_states
 * -> MXFP8 data + scale; round_mode rint, dst_type float8_e4m3fn).  Per
 * block of 32 consecutive elements of a row: shared exponent
 * e = floor(log2(amax)) - 8 clamped to [-127, 127] (amax 0 -> -127),
 * scale code = e + 127, element = E4M3 round-to-nearest-even of x / 2^e,
 * saturated to +-448.
 *   x      [rows, cols] bf16, cols % 32 == 0
 *   codes  [rows, cols] uint8 (output)
 *   scales [rows, cols/32] uint8 (output) */
int moe_mx_quantize(const uint16_t* x, int rows, int cols, uint8_t* codes,
                    uint8_t* scales, void* stream);

/* ------------------------------------------------ W4A8 weight layout -----
 * One-time re-layout of MX weights at load time ([Hy3] section 6.2, "GMM
 * and weight layout": the expert weight layout is settled when the weights
 * are loaded, so the decode step never re-arranges them).  Input: G matrices
 * of rows x K (rows % 16 == 0, K % 128 == 0), E2M1 codes [G, rows, K/2] (low
 * nibble = even k) and E8M0 scales [G, rows, K/32].  Output, per matrix
 * (ns = K/128, nq = ceil(ns/4)):
 *   packed_codes  (rows*K/2 bytes): 1 KB block (q, s) at (q*ns + s)*1024,
 *                 q = group of 16 rows, s = 128-wide K step; its 16-byte
 *                 lane l = 16*b + i is bytes [64s + 16b, +16) of row 16q + i.
 *   packed_scales (moe_mx_packed_scales_bytes(rows, K) bytes): 256-byte
 *                 block (q, c) at (q*nq + c)*256; its dword lane l = 16*b + i
 *                 has in byte u the scale of row 16q + i, 32-block
 *                 4*(4c + u) + b (zero beyond the last step).
 * The inputs are only read; outputs are caller-owned device memory.
 * moe_mx_packed_scales_bytes returns 0 for unsupported shapes. */
size_t moe_mx_packed_scales_bytes(int rows, int K);
int moe_mx_pack_weight(const uint8_t* codes, const uint8_t* scales, int G, int rows, int K,
                       uint8_t* packed_codes, uint8_t* packed_scales, void* stream);

/* ---------------------------------------------------------- S5, S6 -----
 * Expert weights.  [out, in] layout, K-contiguous ([Hy3] section 6.2 keeps
 * the checkpoint layout and multiplies through a transposed view).
 *   bf16: w13 [E, 2I, H]  rows [0, I) = gate_proj, [I, 2I) = up_proj
 *         ([Qwen3] compute decomposition: gate and up concatenated; the
 *         SwiGLU takes SiLU of the first half times the second half)
 *         w2  [E, H, I]
 *   W4A8: the matrices above as E2M1 codes (low nibble = even k) with one
 *         E8M0 scale per 32 consecutive k, in the packed layout written by
 *         moe_mx_pack_weight: w13 = packed codes of [E, 2I, H/2] (same size),
 *         w13_scales = E x moe_mx_packed_scales_bytes(2I, H) bytes; w2 =
 *         packed codes of [E, H, I/2], w2_scales = E x
 *         moe_mx_packed_scales_bytes(H, I) bytes.
 *   The optional shared expert ([Hy3] section 1.1: one per MoE layer, added
 *   to every token) uses the same format with intermediate shared_I
 *   (shared_I == 0: none; W4A8: packed as one matrix each). */
typedef struct {
  int H, I, E;
  int fmt; /* moe_format */
  const void* w13;
  const uint8_t* w13_scales;
  const void* w2;
  const uint8_t* w2_scales;
  int shared_I;
  const void* shared_w13;
  const uint8_t* shared_w13_scales;
  const void* shared_w2;
  const uint8_t* shared_w2_scales;
} MoeFfnWeights;

/* Grouped GEMM over w13 with SwiGLU in the epilogue ([Qwen3] grouped matmul
 * + fused swiglu; [Hy3] section 5.2: swiglu with group quant on the
 * quantised path), one launch over all experts; tiles are scheduled on the
 * device from `offsets` (no host read of the counts).
 *   x        bf16: [T, H] bf16.  W4A8: MXFP8 codes [T, H] (from
 *            moe_mx_quantize) with x_scales [T, H/32].
 *   sorted_pair, offsets: from moe_route (k = experts per token).
 *   act      [T*k, I] in sorted-row order (output): bf16 a = SiLU(g) * u
 *            rounded to bf16; W4A8: MXFP8 codes of a with act_scales
 *            [T*k, I/32].
 * Rows r >= offsets[E] are not written.  Kernels: weight-streaming 16-row
 * tiles with at most 16 tokens, or with at most 3 (bf16) / 8 (W4A8) rows per
 * expert on average when no bf16 shared expert with shared_I == I is
 * attached; LDS-tiled 128-row tiles otherwise (the same choice in every
 * entry point, so their outputs agree bit for bit). */
int moe_grouped_ffn_up(const MoeFfnWeights* w, const void* x, const uint8_t* x_scales,
                       int T, int k, const int32_t* sorted_pair, const int32_t* offsets,
                       void* act, uint8_t* act_scales, void* stream);

/* Grouped GEMM over w2: y[r, :] = act[r, :] . w2[e(r)]^T, fp32 accumulate,
 * stored bf16.  y [T*k, H] in sorted-row order (output). */
int moe_grouped_ffn_down(const MoeFfnWeights* w, const void* act, const uint8_t* act_scales,
                         int T, int k, const int32_t* offsets, uint16_t* y, void* stream);

/* The shared expert over all T tokens (no routing): shared_act [T, shared_I]
 * (+ shared_act_scales [T, shared_I/32] for W4A8), shared_y [T, H] bf16.
 * Requires w->shared_I > 0. */
int moe_shared_ffn(const MoeFfnWeights* w, const void* x, const uint8_t* x_scales, int T,
                   void* shared_act, uint8_t* shared_act_scales, uint16_t* shared_y,
                   void* stream);

/* moe_grouped_ffn_up followed by moe_grouped_ffn_down (and moe_shared_ffn
 * when w->shared_I > 0 and shared_y is not NULL).  With bf16 weights,
 * shared_I == I and more than 16 tokens, the shared expert runs as one more
 * group inside the two routed launches; every output equals the separate
 * calls' bit for bit. */
int moe_grouped_ffn(const MoeFfnWeights* w, const void* x, const uint8_t* x_scales,
                    int T, int k, const int32_t* sorted_pair, const int32_t* offsets,
                    void* act, uint8_t* act_scales, uint16_t* y,
                    void* shared_act, uint8_t* shared_act_scales, uint16_t* shared_y,
                    void* stream);

/* ------------------------------------------------------------- S7 -----
 * finalize_routing ([Qwen3]: re-order expert outputs back to tokens and take
 * the weighted sum) plus the shared expert's row ([Hy3] section 1.1):
 *   out[t, :] = bf16_rne( sum_{j<k} w[t,j] * y[pair_pos[t*k+j], :]
 *                         + shared_y[t, :] )
 * fp32 accumulation in slot order j; pairs with pair_pos < 0 are skipped.
 *   y [T*k, H] bf16, pair_pos [T*k], topk_w [T, k] fp32,
 *   shared_y [T, H] bf16 or NULL, out [T, H] bf16 (output). */
int moe_combine(const uint16_t* y, const int32_t* pair_pos, const float* topk_w,
                const uint16_t* shared_y, int T, int k, int H, uint16_t* out,
                void* stream);

/* ------------------------------------------------------ whole layer -----
 * S0..S7 in one call on one stream.  The router launch also writes the
 * MXFP8 x of the W4A8 path (no separate quantiser).  With T <= 16 and
 * T*k <= 1024 (decode) the front end is two launches: router partial sums,
 * then one block per token for its logits and top-k, the last of them to
 * finish also for the counts and the permutation; the shared expert runs
 * inside the routed GEMM launches as moe_grouped_ffn describes; the buffers
 * receive the same values as the per-step calls. */
typedef struct {
  int H, E, k;
  int gate_mode;        /* moe_gate_mode */
  float routed_scale;   /* sigmoid mode weight scale (2.826 for Hy3) */
  float eps;            /* sigmoid mode denominator eps (1e-20 for Hy3) */
  const float* wr;      /* [E, H] fp32 router weight */
  const float* bias;    /* [E] fp32 or NULL */
  MoeFfnWeights ffn;    /* ffn.H and ffn.E must equal H and E */
} MoeLayerDesc;

/* Caller-owned buffers for the intermediates; all are written. */
typedef struct {
  float* logits;          /* [T, E] */
  int32_t* topk_ids;      /* [T, k] */
  float* topk_w;          /* [T, k] */
  int32_t* counts;        /* [E] */
  int32_t* offsets;       /* [E+1] */
  int32_t* sorted_pair;   /* [T*k] */
  int32_t* pair_pos;      /* [T*k] */
  int32_t* dev_status;    /* [1] or NULL */
  uint8_t* xq;            /* W4A8: [T, H] MXFP8 codes of x; else unused */
  uint8_t* xq_scales;     /* W4A8: [T, H/32] */
  void* act;              /* [T*k, I] bf16 (W4A8: uint8 codes) */
  uint8_t* act_scales;    /* W4A8: [T*k, I/32] */
  uint16_t* y;            /* [T*k, H] bf16 */
  void* shared_act;       /* [T, shared_I] when the layer has a shared expert */
  uint8_t* shared_act_scales;
  uint16_t* shared_y;     /* [T, H] */
  void* workspace;        /* moe_layer_workspace_size(desc, T) bytes (router
                             partial sums or routing histograms; with at most
                             16 tokens also the gate blocks' done counter,
                             which the call zeroes itself; one call at a time
                             per workspace) */
  size_t workspace_bytes;
  /* Optional hipEvent_t handles, recorded on `stream` right before and right
   * after the grouped GEMM1 (w13 + SwiGLU) launch so that a caller can time
   * that kernel inside a full layer call; NULL to skip. */
  void* ev_ffn_up_begin;
  void* ev_ffn_up_end;
} MoeLayerBuffers;

/* Device scratch moe_layer_forward needs for T tokens (bytes; 0 when none or
 * for invalid arguments).  moe_workspace_size is the same function under the
 * name the layer's scratch query carries in the routing operator split
 * (init_routing / grouped matmul / finalize_routing, [Qwen3] "GMM enablement
 * and routing optimisation"); either may be called. */
size_t moe_layer_workspace_size(const MoeLayerDesc* d, int T);
size_t moe_workspace_size(const MoeLayerDesc* d, int T);
int moe_layer_forward(const MoeLayerDesc* d, const uint16_t* x, int T, uint16_t* out,
                      const MoeLayerBuffers* b, void* stream);

/* ------------------------------------------- whole layer, no allocation -----
 * moe_layer_forward for callers that cannot allocate device memory or hand
 * the library a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, kernels and
 * results as moe_layer_forward, except that b->workspace and
 * b->workspace_bytes are ignored: the router's partial sums and the routing
 * histograms live in one static device array of the library,
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the library's first
 * use on that GPU until the process ends.  The call allocates nothing.
 *   Limit: moe_layer_workspace_size(d, T) <= MOE_NOALLOC_SCRATCH_BYTES (the
 *   router part never exceeds 64 MiB; the routing part does only beyond
 *   about 66 million routed pairs at E = 256), else MOE_ERR_SCRATCH and
 *   nothing is enqueued.  The array used is the one of the GPU that `stream`
 *   runs on (the current GPU for the null stream).
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents (every byte a call reads from it, that call wrote
 *   first, so nothing needs to start at zero).  Calls that overlap on one
 *   GPU (different streams or host threads, or a second call enqueued
 *   before the first finished on another stream) RACE on it: order them on
 *   one stream.  MOE_ERR_LAUNCH if the array's device address cannot be
 *   obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_forward_noalloc(const MoeLayerDesc* d, const uint16_t* x, int T, uint16_t* out,
                              const MoeLayerBuffers* b, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
