/*
 * moe.h -- C ABI of the sparse-MoE FFN layer forward for AMD MI355X (gfx950).
 *
 * The layer (Step-3.5-Flash MoE block) as the pages state it:
 *   sglang-jax issue "[Feature] Support Step 3.5 Flash (StepFun) Model",
 *   section "Model configuration" (MoE and clamped-SwiGLU bullets) and
 *   "Key difficulties" item 1; llm-atlas Step-3.5-Flash model card, "Raw
 *   config fields" (hidden_size, moe_num_experts, moe_top_k,
 *   moe_intermediate_size, share_expert_dim, norm_expert_weight,
 *   moe_router_activation = sigmoid, moe_router_scaling_factor = 3,
 *   use_moe_router_bias, need_fp32_gate, swiglu_limits, swiglu_limits_shared).
 *
 * Per token t with activation x_t (bf16, length H):
 *   z_e   = x_t . Wg_e                    fp32 router logits, e in [0, E)
 *   s_e   = 1 / (1 + exp(-z_e))           sigmoid scores
 *   key_e = s_e + b_e                     the bias only decides selection
 *   ids   = the k experts of largest key, equal keys -> lower index first,
 *           listed in that rank order
 *   w_j   = routed_scaling * s_{ids_j} / sum_j' s_{ids_j'}   (renormalize != 0)
 *         = routed_scaling * s_{ids_j}                        (renormalize == 0)
 *   f_e(x) = W_down_e (SiLU(g) * u),  g = W_gate_e x,  u = W_up_e x, where
 *           for limit L > 0: g = min(g, L), u = clamp(u, -L, L)
 *   y_t   = f_shared(x_t) + sum_j w_j f_{ids_j}(x_t)   (shared weight 1.0)
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major and live in device memory of the
 *     current HIP device, unless stated otherwise.  bf16 is passed as raw
 *     uint16_t bits.  Weights are stored out x in: w_gate/w_up [E][I][H],
 *     w_down [E][H][I], ws_gate/ws_up [Is][H], ws_down [H][Is],
 *     router_w [E][H] (fp32), router_bias [E] (fp32).
 *   - Pair id p = t * k + j names slot j of token t.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no state between calls except the per-thread error text and
 *     the fixed scratch of moe_forward_noalloc (a device array per GPU, sized
 *     at build time, allocated by the runtime when the library is loaded).
 *   - Every call only enqueues work on `stream` (0 = the null stream) and
 *     returns without synchronising; results are ready when the stream is.
 *   - Arguments are validated before anything is enqueued: an error return
 *     means that nothing was launched.  `moe_last_error()` then describes it.
 *   - tokens == 0 is valid: MOE_OK; moe_permute then writes the E+1 zero
 *     offsets, the other entry points launch nothing.  Per-token buffers
 *     (x, y, ids, weights, pair arrays) may then be NULL.
 *   - Limits: 1 <= top_k <= min(num_experts, 32); num_experts <= 1024;
 *     hidden % 128 == 0; inter % 64 == 0; inter_shared % 64 == 0 (0 = no
 *     shared expert); tokens * top_k < 2^31 and tokens * top_k *
 *     max(hidden, inter, inter_shared) < 2^32; every pointer 16-byte aligned.
 *   - Preconditions not checked: inputs are finite; outputs do not alias
 *     inputs or the workspace; ids given to moe_permute are in [0, E).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null required pointer, negative or zero size, k > E */
  MOE_ERR_UNSUPPORTED = 2, /* a size or alignment outside the limits above */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4          /* a HIP launch failed; moe_last_error() has the HIP text */
} moe_status;

/* Layer configuration; the names follow the model's config fields. */
typedef struct {
  int64_t tokens;            /* T >= 0                                            */
  int32_t hidden;            /* H, hidden_size (4096)                             */
  int32_t num_experts;       /* E, moe_num_experts (288)                          */
  int32_t top_k;             /* k, moe_top_k (8)                                  */
  int32_t inter;             /* I, moe_intermediate_size (1280)                   */
  int32_t inter_shared;      /* Is, share_expert_dim (1280); 0 = no shared expert */
  float routed_scaling;      /* moe_router_scaling_factor (3.0)                   */
  int32_t renormalize;       /* norm_expert_weight (1)                            */
  float swiglu_limit;        /* swiglu_limits[layer] for routed experts; <= 0: none */
  float swiglu_limit_shared; /* swiglu_limits_shared[layer]; <= 0: none           */
} moe_config;

/* Bytes of device workspace that moe_forward, moe_route and moe_permute need
 * for this configuration (one size serves all three).  Returns 0 for an
 * invalid configuration.  These three take the workspace with any contents:
 * each call writes every word of it that it reads (work-queue counters
 * included) before reading it, so one workspace serves calls of different
 * batch sizes in turn (calls on it must not overlap). */
size_t moe_workspace_size(const moe_config* cfg);

/* Text of the last error on the calling thread ("" if none).  Valid until
 * the next call on this thread. */
const char* moe_last_error(void);

/* Router: fp32 logits, sigmoid, bias-for-selection, top-k, gating weights.
 * Follows "Key difficulties" item 1 of the sglang-jax issue (scores in fp32;
 * bias only selects; weights gathered from the bias-free scores, then
 * normalised and multiplied by 3.0).
 *   x           [T][H] bf16 activations
 *   router_w    [E][H] fp32 router weight
 *   router_bias [E] fp32, or NULL for no bias
 *   topk_ids    out [T][k] int32, rank order (key desc, ties -> lower index)
 *   topk_w      out [T][k] fp32 gating weights aligned with topk_ids
 *   ws          device workspace of ws_bytes >= moe_workspace_size(cfg) */
moe_status moe_route(const moe_config* cfg, const uint16_t* x, const float* router_w,
                     const float* router_bias, int32_t* topk_ids, float* topk_w, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* Token permutation by expert, the grouping a grouped GEMM over experts
 * needs (sglang-jax issue, "Implementation strategy": GMM over experts).
 * A stable counting sort of the pairs by expert id:
 *   topk_ids        [T][k] int32 in [0, E)
 *   expert_offsets  out [E+1] int32: exclusive prefix of per-expert pair
 *                   counts; expert_offsets[E] == T*k
 *   sorted_pairs    out [T*k] int32: pair ids grouped by expert, ascending
 *                   pair id within an expert
 *   pair_pos        out [T*k] int32: inverse, sorted_pairs[pair_pos[p]] == p
 *   ws              device workspace (as for moe_route) */
moe_status moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t* expert_offsets,
                       int32_t* sorted_pairs, int32_t* pair_pos, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Whole layer forward: route, permute, grouped SwiGLU experts (gate/up and
 * down), shared expert, and a deterministic combine (fixed summation order,
 * no floating-point atomics).  Covers the MoE bullet of "Model
 * configuration" and the clamped SwiGLU of the "Reuse map" in the sglang-jax
 * issue.
 *   y             out [T][H] bf16 layer output
 *   topk_ids_out  optional out [T][k] int32 (NULL: kept in the workspace)
 *   topk_w_out    optional out [T][k] fp32  (NULL: kept in the workspace)
 *   ws_gate/ws_up/ws_down may be NULL when inter_shared == 0. */
moe_status moe_forward(const moe_config* cfg, const uint16_t* x, const float* router_w,
                       const float* router_bias, const uint16_t* w_gate, const uint16_t* w_up,
                       const uint16_t* w_down, const uint16_t* ws_gate, const uint16_t* ws_up,
                       const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                       float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward that also records `n_events` caller-created HIP events on
 * `stream` around its kernels, for per-kernel timing.  Event i is recorded
 * before stage i and event n_events-1 after the last stage; stages are
 * MOE_STAGE_* below.  n_events must be MOE_NUM_STAGES + 1. */
enum {
  MOE_STAGE_ROUTER_GEMM = 0, /* router logits (partials)             */
  MOE_STAGE_TOPK = 1,        /* sigmoid, bias, top-k, gating weights  */
  MOE_STAGE_RANK = 2,        /* per-chunk ranks and histograms        */
  MOE_STAGE_SCAN = 3,        /* expert offsets and GEMM tile lists    */
  MOE_STAGE_SCATTER = 4,     /* sorted pairs and their inverse        */
  MOE_STAGE_GATEUP = 5,      /* grouped gate/up GEMM + SwiGLU         */
  MOE_STAGE_DOWN = 6,        /* grouped down GEMM, weighted           */
  MOE_STAGE_COMBINE = 7,     /* shared + weighted routed sum -> y     */
  MOE_NUM_STAGES = 8
};
moe_status moe_forward_timed(const moe_config* cfg, const uint16_t* x, const float* router_w,
                             const float* router_bias, const uint16_t* w_gate,
                             const uint16_t* w_up, const uint16_t* w_down,
                             const uint16_t* ws_gate, const uint16_t* ws_up,
                             const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                             float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream,
                             hipEvent_t* events, int n_events);

/* moe_forward with the routed experts' weights in FP8.  The sglang-jax issue
 * "[Feature] Support Step 3.5 Flash (StepFun) Model", section "Model
 * configuration", lists FP8 among the model's official weight formats beside
 * BF16 and says nothing more about it; the layout below (OCP E4M3 codes with
 * one fp32 scale per output row) is this library's reading of that format.
 * Each routed weight is decode(code) * scale of its output row, code an OCP
 * FP8 E4M3 ("e4m3fn": bias 7, no infinities, max 448) byte:
 *   w8_gate, w8_up  [E][I][H] uint8 codes;  scale_gate, scale_up  [E][I] fp32
 *   w8_down         [E][H][I] uint8 codes;  scale_down            [E][H] fp32
 * The shared expert stays bf16 (ws_gate/ws_up/ws_down as in moe_forward).
 * Products are formed exactly (every e4m3 value is a bf16 value) and
 * accumulated in fp32; the row scale multiplies each accumulated sum.  Same
 * workspace size, conventions and limits as moe_forward. */
moe_status moe_forward_fp8(const moe_config* cfg, const uint16_t* x, const float* router_w,
                           const float* router_bias, const uint8_t* w8_gate, const uint8_t* w8_up,
                           const uint8_t* w8_down, const float* scale_gate,
                           const float* scale_up, const float* scale_down,
                           const uint16_t* ws_gate, const uint16_t* ws_up,
                           const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                           float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* The same layer forward as moe_forward in ONE kernel launch, for small
 * batches (decoding): tokens <= 256 and tokens * top_k <= 2048, else
 * MOE_ERR_UNSUPPORTED (checked before anything is enqueued).  It is the
 * fused expert backend that the sglang-jax issue names as the performance
 * switch to follow the grouped-matmul path ("Reuse map", "Implementation
 * strategy").  On an MI355X it is slower than moe_forward at every measured
 * batch size; it serves callers that want a single launch per layer.
 * Arguments, layouts and outputs are those of moe_forward, and so are the
 * results, bit for bit: every output is formed in the same arithmetic order.
 *
 * Workspace: moe_workspace_size(cfg) bytes, as for moe_forward.  Its
 * control words (MOE_WS_FUSED_CTL below, under 5 KB) must be zero before
 * the first moe_forward_fused call on that workspace -- zero-fill the
 * workspace once after allocating it; every call leaves them zero again,
 * and no other entry point writes them.  Calls that share a workspace must
 * be ordered (one stream).  The status word (MOE_WS_FUSED_STATUS) stays
 * zero unless an internal wait gave up (about a second, only possible if
 * the launch was starved), which marks the outputs invalid; it is sticky
 * until the caller clears it. */
moe_status moe_forward_fused(const moe_config* cfg, const uint16_t* x, const float* router_w,
                             const float* router_bias, const uint16_t* w_gate,
                             const uint16_t* w_up, const uint16_t* w_down,
                             const uint16_t* ws_gate, const uint16_t* ws_up,
                             const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                             float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- Layer forward that allocates nothing ----------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same forward as moe_forward (same kernels, same results bit
 * for bit), with its workspace in a fixed scratch array inside the library:
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) of device memory on each GPU the
 * library runs on, held from the library's load there until the process
 * ends.  That covers the full-shape layer (hidden 4096, 288 experts, top 8,
 * intermediate 1280) up to about 630 tokens; a configuration whose
 * moe_workspace_size() exceeds it returns MOE_ERR_WORKSPACE before anything
 * is enqueued.  The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); on its first call on a device it looks up
 * that device's scratch address.  The scratch used is the current HIP
 * device's, so the stream must belong to the current device (as the buffers
 * of every entry point do).
 * Every call on one GPU uses that GPU's one scratch array, which keeps the
 * last call's contents (each call writes what it reads first): calls that
 * overlap on one GPU -- on different streams or host threads without
 * ordering -- race on it and must not be issued.  Arguments, outputs and
 * errors are those of moe_forward; no workspace argument. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_noalloc(const moe_config* cfg, const uint16_t* x, const float* router_w,
                               const float* router_bias, const uint16_t* w_gate,
                               const uint16_t* w_up, const uint16_t* w_down,
                               const uint16_t* ws_gate, const uint16_t* ws_up,
                               const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                               float* topk_w_out, hipStream_t stream);

/* Where an intermediate of moe_forward lives inside the workspace, for
 * inspection after the stream has finished (tests, debugging).  Writes the
 * byte offset and size; returns MOE_ERR_INVALID_ARG for an unknown id. */
enum {
  MOE_WS_TOPK_IDS = 0,       /* [T][k] int32 (when topk_ids_out was NULL)  */
  MOE_WS_TOPK_W = 1,         /* [T][k] fp32  (when topk_w_out was NULL)    */
  MOE_WS_EXPERT_OFFSETS = 2, /* [E+1] int32                                */
  MOE_WS_SORTED_PAIRS = 3,   /* [T*k] int32                                */
  MOE_WS_PAIR_POS = 4,       /* [T*k] int32                                */
  MOE_WS_H = 5,              /* [T*k][I] bf16 routed SwiGLU activations in
                                sorted order, then [T][Is] shared          */
  MOE_WS_O = 6,              /* [T*k][H] bf16 weighted routed expert outputs
                                in sorted order, then [T][H] shared        */
  MOE_WS_FUSED_CTL = 7,      /* uint32 control words of moe_forward_fused  */
  MOE_WS_FUSED_STATUS = 8    /* uint32: nonzero = a fused wait gave up     */
};
moe_status moe_workspace_view(const moe_config* cfg, int which, size_t* offset, size_t* bytes);

/* ---- Dense SwiGLU FFN ----------------------------------------------------
 * The FFN of Step-3.5-Flash's first three layers, which are dense (sglang-jax
 * issue, "Model configuration", MLP bullet: intermediate 11264; "Reuse map":
 * first-k dense + MoE layers; llm-atlas model card, "Raw config fields":
 * intermediate_size).  The same clamped SwiGLU MLP as one expert above, applied to every
 * token:  y_t = W_down (SiLU(g) * u),  g = W_gate x_t,  u = W_up x_t, with
 * g = min(g, L), u = clamp(u, -L, L) for L > 0.  It runs on the grouped
 * expert GEMMs with a single group of all T tokens.
 *   x      [T][H] bf16;  w_gate, w_up [I][H] bf16;  w_down [H][I] bf16
 *   y      out [T][H] bf16
 *   ws     device workspace of ws_bytes >= moe_dense_workspace_size(cfg)
 * Limits: hidden % 128 == 0; inter % 64 == 0, inter >= 64; tokens *
 * max(hidden, inter) < 2^32; pointers 16-byte aligned.  Conventions as above
 * (tokens == 0 launches nothing; x and y may then be NULL). */
typedef struct {
  int64_t tokens;     /* T >= 0                                    */
  int32_t hidden;     /* H, hidden_size (4096)                     */
  int32_t inter;      /* I, intermediate_size (11264)              */
  float swiglu_limit; /* swiglu_limits[layer] (0.0 for these layers); <= 0: none */
  int32_t reserved;   /* must be 0                                 */
} moe_dense_config;

/* Workspace bytes for moe_dense_forward; 0 for an invalid configuration. */
size_t moe_dense_workspace_size(const moe_dense_config* cfg);

moe_status moe_dense_forward(const moe_dense_config* cfg, const uint16_t* x,
                             const uint16_t* w_gate, const uint16_t* w_up,
                             const uint16_t* w_down, uint16_t* y, void* ws, size_t ws_bytes,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
