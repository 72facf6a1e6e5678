/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse MoE-layer forward.
 *
 * One MoE layer of the Step-3.5-Flash / Step-5-Preview decoders:
 *   out = routed_moe(x) + shared_expert(x)
 * with sigmoid router scores, a per-expert routing bias used only for the
 * top-k choice, expert weights taken from the raw scores, optional
 * renormalisation, a router scaling factor, clipped-SwiGLU experts and an
 * always-on shared expert (page "MAX 中 Step-3.5-Flash 架构解析：混合注意力、MoE
 * 与 TP/EP/DP 并行实现指南", section "MoE：共享专家、sigmoid 路由与激活裁剪";
 * configuration fields from its section "Step3p5Config配置项全解").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every tensor pointer is a DEVICE pointer, row-major, contiguous,
 *   16-byte aligned, owned by the caller.  The library never allocates or
 *   frees device memory; scratch memory comes in through (ws, ws_bytes),
 *   sized by moe_workspace_size().
 * bf16: raw IEEE bfloat16 (uint16 storage).  FP8: OCP E4M3FN codes (uint8).
 * Weights use the [out_features, in_features] layout of the stacked
 *   checkpoint tensors (layers.{i}.moe.{proj}.weight [num_experts, ...]).
 *   The fused first projection holds the gate rows 0..I-1, then the up rows
 *   I..2I-1.
 * Streams: all work is enqueued on `stream`, and only there; no call waits
 *   for the device, so a HIP graph can capture any call.
 * Errors: arguments are checked before anything is launched; on an argument
 *   error nothing is written.  MOE_ERR_HIP reports a launch failure (the
 *   launches before it stay queued on `stream`); faults inside kernels
 *   surface on the stream.
 * Threads: the library keeps no global mutable state; calls are thread-safe.
 *   Calls that share a workspace must be ordered on one stream.
 * Shapes: H % 64 == 0, I % 64 == 0, Is % 64 == 0 (or Is == 0), 1 <= k <= 32,
 *   k <= E <= 1024, T >= 0 (T == 0 is a no-op), T * k < 2^31, and, as x and
 *   one expert's fused first-projection weights are addressed with 32-bit
 *   byte offsets, T * H < 2^31, 2 I * H < 2^31 and 2 Is * H < 2^31.  FP8
 *   experts also need H % 128 == 0 and I % 128 == 0.  Other shapes return
 *   MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,  /* null pointer, negative size, bad enum, k > E, negative limit */
    MOE_ERR_UNSUPPORTED = 2,       /* a shape or dtype combination the kernels do not cover */
    MOE_ERR_WORKSPACE = 3,         /* ws_bytes smaller than moe_workspace_size() */
    MOE_ERR_HIP = 4                /* a HIP launch or runtime call failed */
} moe_status_t;

typedef enum {
    MOE_BF16 = 0,
    MOE_FP32 = 1,
    MOE_FP8_E4M3_B128 = 2          /* E4M3FN codes + one fp32 scale per 128x128 block */
} moe_dtype_t;

/* One layer's configuration.  Field meanings follow Step3p5Config (config
 * table of the MAX page): moe_num_experts, moe_top_k, moe_intermediate_size,
 * share_expert_dim, moe_router_scaling_factor, norm_expert_weight, and one
 * layer's entries of swiglu_limits / swiglu_limits_shared (0 = no clipping). */
typedef struct {
    int32_t hidden_size;            /* H */
    int32_t num_experts;            /* E, routed experts */
    int32_t top_k;                  /* k, experts per token */
    int32_t moe_intermediate_size;  /* I, routed expert width */
    int32_t share_expert_dim;       /* Is, shared expert width; 0 = no shared expert */
    float   router_scaling_factor;  /* multiplies the k weights (3.0 on both models) */
    int32_t norm_expert_weight;     /* 1: divide the k raw scores by their sum first */
    float   swiglu_limit;           /* routed experts' clip; 0 = none; < 0 invalid */
    float   swiglu_limit_shared;    /* shared expert's clip; 0 = none; < 0 invalid */
    int32_t expert_dtype;           /* moe_dtype_t: MOE_BF16 or MOE_FP8_E4M3_B128 (routed experts) */
    int32_t out_dtype;              /* moe_dtype_t: MOE_FP32 or MOE_BF16 (layer output) */
} moe_config_t;

/* Bytes of scratch memory moe_layer_forward needs for T tokens (it also
 * covers each step's own entry point).  Writes *bytes; pure host function. */
moe_status_t moe_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes);

/* Router (MAX page, MoE section, Step3p5MoEGate paragraph): logits in fp32
 * from bf16 x [T,H] and w_router [E,H]; s = sigmoid(logit); the k experts
 * with the largest s + router_bias (fp32 [E]) are chosen, ordered by
 * corrected score descending, ties to the lower index, NaN last; every id is
 * in [0, E-1] even for NaN/Inf inputs.  topk_w [T,k] fp32 = raw s of the
 * chosen experts, divided by their sum if norm_expert_weight, times
 * router_scaling_factor.  topk_ids [T,k] int32.  Uses ws for the logits. */
moe_status_t moe_route(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                       const float* router_bias, int32_t* topk_ids, float* topk_w,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Permutation of the T*k (token, slot) pairs by expert (the grouping the
 * routed experts run on; pages describe it only through EP dispatch).
 * expert_counts [E]: pairs per expert.  expert_offsets [E+1]: exclusive
 * prefix sum.  row_to_pair [T*k]: rows are expert-major and ascending in
 * token inside an expert; row r holds pair p = t*k + j.  pair_to_row [T*k]:
 * the inverse.  All int32; results are deterministic. */
moe_status_t moe_permute(const moe_config_t* cfg, int64_t T, const int32_t* topk_ids,
                         int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* row_to_pair, int32_t* pair_to_row,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Routed experts (MAX page, MoE section: clipped SwiGLU built on the
 * concatenated gate|up projection, limit = swiglu_limit): for every row r of
 * expert e (rows expert_offsets[e] .. expert_offsets[e+1]-1), with
 * t = row_to_pair[r] / k:
 *   [g|u] = W13[e] x[t];  h = act(g, u, L);  y_rows[r] = W2[e] h
 * act = silu(g)*u if L == 0, else min(silu(g), L) * clamp(u, -L, L).
 * w13 [E,2I,H], w2 [E,H,I]: bf16, or E4M3FN codes with w13_scale
 * [E,2I/128,H/128] and w2_scale [E,H/128,I/128] fp32 (multiplying) when
 * expert_dtype is MOE_FP8_E4M3_B128 (miles page "Step-5-Preview", section
 * 1 Model Introduction); scales must be NULL for bf16 and both non-NULL for
 * FP8.  In FP8 mode x (per token) and h (per row) are quantised per 128
 * columns to E4M3FN (round to nearest even) with scale amax/448, or 1 for an
 * all-zero group, and both projections accumulate the exact code products
 * of each 128-wide block in fp32 before applying the two scales.
 * y_rows: T*k expert output rows, unweighted, in row order, each in the
 * scaled-fp16 row format: H fp16 values (round to nearest even), then one
 * int8 exponent e per 128 columns, then zero bytes up to a multiple of 16; the
 * value is fp16 * 2^e.  The library picks e so that the group's largest
 * magnitude scales into [2^14, 2^15) (rounding may carry it to 2^15), so no
 * finite result overflows and every
 * value keeps fp16's 11 significant bits relative to its group's largest
 * (for the same bytes as bf16 rows plus 1/256).  moe_expert_rows_bytes()
 * gives the size of n rows. */
moe_status_t moe_grouped_swiglu(const moe_config_t* cfg, int64_t T, const void* x,
                                const int32_t* expert_offsets, const int32_t* row_to_pair,
                                const void* w13, const float* w13_scale,
                                const void* w2, const float* w2_scale,
                                void* y_rows, void* ws, size_t ws_bytes, hipStream_t stream);

/* The two halves of moe_grouped_swiglu, for callers that schedule them
 * apart (and for timing the first projection on its own).
 * moe_expert_up: h = act(W13[e] x[row_to_pair[r] / k], L) for every row r.
 *   h is [T*k, I] bf16 for bf16 experts; for FP8 experts it is [T*k, I]
 *   E4M3FN codes, then, at the next multiple of 256 bytes, fp32 scales laid
 *   out block-major as [I/128][T*k] (moe_hidden_bytes() covers both).
 * moe_expert_down: y_rows[r] = W2[e] h[r] (h dequantised in FP8 mode).
 * Shared expert in the same launches (optional): with bf16 experts and
 * share_expert_dim == moe_intermediate_size, ws13 / ws2 (bf16 [2Is,H] /
 * [H,Is], MAX page, MoE section) may be passed; the shared expert then runs
 * as T more rows after the T*k routed ones -- h[T*k + t] = act(Ws13 x[t],
 * swiglu_limit_shared) and y_rows[T*k + t] = Ws2 h[T*k + t], so h holds
 * (T*k + T) rows (moe_hidden_bytes() covers them whenever the shared expert
 * can run this way) and y_rows [T*k + T, H].  Pass ws13 and ws2 together or
 * not at all; otherwise both are NULL.  Any other configuration with a
 * non-NULL ws13/ws2 is MOE_ERR_INVALID_ARGUMENT. */
moe_status_t moe_expert_up(const moe_config_t* cfg, int64_t T, const void* x,
                           const int32_t* expert_offsets, const int32_t* row_to_pair,
                           const void* w13, const float* w13_scale, const void* ws13, void* h,
                           void* ws, size_t ws_bytes, hipStream_t stream);
moe_status_t moe_expert_down(const moe_config_t* cfg, int64_t T, const void* h,
                             const int32_t* expert_offsets, const void* w2, const float* w2_scale,
                             const void* ws2, void* y_rows, void* ws, size_t ws_bytes, hipStream_t stream);
/* Bytes of the h buffer moe_expert_up writes for T tokens (with room for
 * the shared expert's rows when it can run in the same launches). */
moe_status_t moe_hidden_bytes(const moe_config_t* cfg, int64_t T, size_t* bytes);
/* Bytes of `rows` expert output rows in the scaled-fp16 row format of
 * moe_grouped_swiglu (2 H + 16 ceil(H / 2048) bytes per row).  Pure host
 * function. */
moe_status_t moe_expert_rows_bytes(const moe_config_t* cfg, int64_t rows, size_t* bytes);

/* Shared expert (MAX page, MoE section: always-on MLP of width
 * share_expert_dim, clipped with swiglu_limit_shared):
 *   y_shared[t] = Ws2 act(Ws13 x[t], L_shared)
 * ws13 [2Is,H] bf16 (gate rows first), ws2 [H,Is] bf16, y_shared [T,H] fp32.
 * Requires share_expert_dim > 0. */
moe_status_t moe_shared_ffn(const moe_config_t* cfg, int64_t T, const void* x,
                            const void* ws13, const void* ws2, float* y_shared,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Weighted combine (MAX page, MoE section: routed output plus the shared
 * expert's): out[t] = sum_j topk_w[t,j] * y_rows[pair_to_row[t*k+j]] + s[t]
 * accumulated in fp32 in slot order; y_rows: T*k rows in the scaled-fp16
 * row format, as written by the routed experts.  The shared term s is
 * y_shared (fp32 [T,H], from moe_shared_ffn) or shared_rows (T rows in the
 * same scaled format: the shared expert's rows written by moe_expert_down,
 * i.e. y_rows + T*k rows), or absent when both are NULL; passing both is
 * MOE_ERR_INVALID_ARGUMENT.  residual (fp32
 * [T,H], optional): the block's fp32 residual stream (AutoModel page,
 * benchmark table), added last, out[t] = residual[t] + (the sum above); out
 * may then be the residual buffer itself when out_dtype is fp32 (in-place
 * update; with bf16 output that aliasing is MOE_ERR_INVALID_ARGUMENT).
 * out [T,H] in out_dtype (fp32 or bf16). */
moe_status_t moe_combine(const moe_config_t* cfg, int64_t T, const void* y_rows,
                         const int32_t* pair_to_row, const float* topk_w,
                         const float* y_shared, const void* shared_rows, const float* residual,
                         void* out, hipStream_t stream);

/* Zero-centred RMSNorm in front of the layer (MAX page: the block's norms
 * are zero-centred RMSNorms with weight_offset 1, the stored weight g scaling
 * by 1 + g; AutoModel page, benchmark table: norms in FP32):
 *   x[t,h] = bf16_rne( resid[t,h] / sqrt(mean_h resid[t,:]^2 + eps) * (1 + g[h]) )
 * computed in fp32.  resid [T,H] fp32, norm_weight g [H] fp32, x [T,H] bf16
 * (the layer's input).  eps >= 0 and finite (the pages print no value). */
moe_status_t moe_rmsnorm(const moe_config_t* cfg, int64_t T, const float* resid, const float* norm_weight,
                         float eps, void* x, hipStream_t stream);

/* moe_rmsnorm followed by moe_route on its output, as one pass where it
 * pays (MAX page, model overview: the norm feeds the MoE block's router):
 * x [T,H] bf16 as moe_rmsnorm writes it, topk_ids / topk_w as moe_route
 * gives for that x, bit for bit.  From 512 tokens (H <= 4096, H % 256 == 0,
 * E <= 384) the norm and the router logits run in one kernel that feeds the
 * normalised rows to the router from on-chip memory; otherwise the two steps
 * run in turn (moe_block_forward always takes the two steps).  Uses ws for the
 * logits (moe_workspace_size covers it); errors as for moe_route and
 * moe_rmsnorm. */
moe_status_t moe_rmsnorm_route(const moe_config_t* cfg, int64_t T, const float* resid, const float* norm_weight,
                               float eps, const void* w_router, const float* router_bias, void* x,
                               int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* The whole layer: route, permute, routed experts, shared expert, combine.
 * Inputs as above (ws13/ws2 may be NULL when share_expert_dim == 0).  With
 * bf16 experts and share_expert_dim == moe_intermediate_size the shared
 * expert runs as one more group of the routed experts' launches, else in
 * launches of its own after them.
 * out [T,H] in out_dtype.  Optional outputs (NULL to skip): topk_ids_out
 * [T,k], topk_w_out [T,k], expert_counts_out [E]. */
moe_status_t moe_layer_forward(const moe_config_t* cfg, int64_t T, const void* x,
                               const void* w_router, const float* router_bias,
                               const void* w13, const float* w13_scale,
                               const void* w2, const float* w2_scale,
                               const void* ws13, const void* ws2, void* out,
                               int32_t* topk_ids_out, float* topk_w_out,
                               int32_t* expert_counts_out,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments less (ws, ws_bytes), the same kernels and results.  Its
 * workspace is a device array inside the library, moe_noalloc_max_bytes()
 * (64 MiB) per GPU, held until the process ends; a call whose
 * moe_workspace_size() exceeds it returns MOE_ERR_WORKSPACE before
 * anything is launched (at the Step-5 shapes with bf16 experts that is
 * above 609 tokens).  The call allocates nothing.  All calls on one GPU share that
 * array: calls that overlap on one GPU (other streams, other threads)
 * race; order them on one stream. */
moe_status_t moe_layer_forward_noalloc(const moe_config_t* cfg, int64_t T, const void* x,
                                       const void* w_router, const float* router_bias,
                                       const void* w13, const float* w13_scale,
                                       const void* w2, const float* w2_scale,
                                       const void* ws13, const void* ws2, void* out,
                                       int32_t* topk_ids_out, float* topk_w_out,
                                       int32_t* expert_counts_out, hipStream_t stream);
/* Bytes of the array moe_layer_forward_noalloc works in. */
size_t moe_noalloc_max_bytes(void);

/* The MoE sub-block of a decoder layer (MAX page: each layer has a norm in
 * front of the MLP/MoE and a residual connection around it; AutoModel page,
 * benchmark table: FP32 norms and residual stream):
 *   x = moe_rmsnorm(resid_in);  resid_out = resid_in + moe_layer_forward(x)
 * with the add fused into the combine.  resid_in, resid_out [T,H] fp32;
 * resid_out may be resid_in (in-place).  cfg->out_dtype must be MOE_FP32.
 * Other arguments as for moe_layer_forward and moe_rmsnorm; x lives in the
 * workspace (moe_workspace_size covers it). */
moe_status_t moe_block_forward(const moe_config_t* cfg, int64_t T, const float* resid_in,
                               const float* norm_weight, float eps,
                               const void* w_router, const float* router_bias,
                               const void* w13, const float* w13_scale,
                               const void* w2, const float* w2_scale,
                               const void* ws13, const void* ws2, float* resid_out,
                               int32_t* topk_ids_out, float* topk_w_out,
                               int32_t* expert_counts_out,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Routing replay (miles page "Step-5-Preview", section 5.2 Algorithm: the
 * trainer reruns the expert choices its rollout made).  topk_ids [T,k] int32
 * is an INPUT: the replayed choice, each id clamped to [0, E-1] (callers
 * should pass ids in range; the clamp only keeps every access in bounds).
 * Duplicate ids in a row are allowed; each slot is treated on its own.
 * topk_w [T,k] fp32 = the raw sigmoid scores of those experts under the
 * current router (x, w_router as for moe_route), divided by their sum if
 * norm_expert_weight, times router_scaling_factor.  That the weights come
 * from the current router is this library's reading; the page says only
 * that the choices are replayed.  Replaying moe_route's own ids gives back
 * its weights bit for bit.  There is no routing bias: it only steers the
 * choice.  Uses ws for the logits (moe_workspace_size covers it). */
moe_status_t moe_route_replay(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                              const int32_t* topk_ids, float* topk_w,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Static balanced routing for benchmarks (AutoModel page, benchmark table:
 * the Step-5 benchmark replaces the router's choice with a fake, balanced,
 * static one).  Writes topk_ids [T,k] int32 with pair p = t*k + j sent to
 * expert p mod E: every expert gets floor(T*k/E) or one more pair, and the
 * k experts of a token are distinct.  The rule is this library's reading;
 * the page names the mode only.  Feed the result to
 * moe_layer_forward_routed. */
moe_status_t moe_balanced_ids(const moe_config_t* cfg, int64_t T, int32_t* topk_ids, hipStream_t stream);

/* The whole layer with the expert choice supplied by the caller (routing
 * replay, or the static balanced routing above): the weights as in
 * moe_route_replay, then the same permute, routed and shared experts and
 * combine as moe_layer_forward.  topk_ids [T,k] int32 is an input (clamped
 * to [0, E-1]); the other arguments are those of moe_layer_forward, less
 * router_bias and topk_ids_out.  Same workspace size. */
moe_status_t moe_layer_forward_routed(const moe_config_t* cfg, int64_t T, const void* x,
                                      const void* w_router, const int32_t* topk_ids,
                                      const void* w13, const float* w13_scale,
                                      const void* w2, const float* w2_scale,
                                      const void* ws13, const void* ws2, void* out,
                                      float* topk_w_out, int32_t* expert_counts_out,
                                      void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- training: forward that keeps its state, and the backward ----------
 *
 * The trainer's side of the method (AutoModel page, benchmark table: BF16
 * forward, backward and optimizer over the whole backbone; miles page: a BF16
 * trainer that replays the rollout's expert choices).  bf16 experts only, and
 * the shared expert, if any, must have the routed experts' width (Is == I,
 * as in both models); other configurations return MOE_ERR_UNSUPPORTED. */

/* Bytes of the state moe_layer_forward_train keeps for T tokens, and of the
 * scratch moe_layer_backward needs.  Pure host functions. */
moe_status_t moe_saved_bytes(const moe_config_t* cfg, int64_t T, size_t* bytes);
moe_status_t moe_backward_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes);

/* moe_layer_forward for training: the same layer, and in `saved` (caller-
 * owned device memory of moe_saved_bytes, to be passed unchanged to
 * moe_layer_backward) the expert choice, the weights, the chosen raw scores,
 * the permutation, the first projection's pre-activations (bf16), h (bf16)
 * and the expert output rows (scaled fp16).  The activation is applied to the
 * bf16-rounded pre-activations it keeps, so the backward differentiates the
 * function that ran.  topk_ids_in [T,k] int32 (optional): a replayed choice
 * (see moe_route_replay; router_bias may then be NULL).  ws: moe_workspace_size. */
moe_status_t moe_layer_forward_train(const moe_config_t* cfg, int64_t T, const void* x,
                                     const void* w_router, const float* router_bias,
                                     const int32_t* topk_ids_in,
                                     const void* w13, const void* w2,
                                     const void* ws13, const void* ws2, void* out,
                                     void* saved, size_t saved_bytes,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Gradients of the loss sum(out * dout) through the layer that
 * moe_layer_forward_train ran on the same x and weights:
 *   dout [T,H] fp32 in;  dx [T,H], dw_router [E,H], dw13 [E,2I,H],
 *   dw2 [E,H,I], dws13 [2Is,H], dws2 [H,Is] fp32 out (overwritten; experts
 *   without tokens get zeros; dws13/dws2 may be NULL without a shared expert).
 * The expert choice passes no gradient and the routing bias gets none.  Each
 * clamp of the clipped SwiGLU passes the gradient where its input lies in its
 * range, ends included.  Products run on bf16 operands (dout times the
 * weights rounded to bf16, the saved activations) with fp32 accumulation.
 * ws: moe_backward_workspace_size bytes. */
moe_status_t moe_layer_backward(const moe_config_t* cfg, int64_t T, const void* x,
                                const void* w_router, const void* w13, const void* w2,
                                const void* ws13, const void* ws2,
                                const void* saved, size_t saved_bytes, const float* dout,
                                float* dx, float* dw_router, float* dw13, float* dw2,
                                float* dws13, float* dws2,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
