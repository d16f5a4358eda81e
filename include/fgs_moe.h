/*
 * fgs_moe.h - C ABI of the fine-grained MoE feed-forward layer for MI355X
 * (gfx950).  Plain pointers and sizes only; no C++ or framework types.
 *
 * The layer (one call = one MoE sublayer over N flattened tokens):
 *
 *   "Inside Kolibri 1: Hybrid RNoPE Attention, Sparse MoE, and FP8 Serving"
 *   (flozi.net), section "Routing: selection bias and mixture weights are
 *   separate":
 *     1. logits h = x W_r^T in FP32, x [N, d], W_r [E, d];
 *     2. the learned correction bias b is added, s = h + b, and the top_k
 *        expert ids with the largest s are selected;
 *     3. mixture weights are sigmoid(h) of the selected ids, from the
 *        UNBIASED logits, not renormalised to sum one;
 *     4. every selected (token, expert) pair is processed; there is no
 *        per-expert capacity and no token is dropped;
 *     5. each routed or shared expert is a SwiGLU MLP
 *        W_down (SiLU(W_gate x) * (W_up x)), without biases.
 *   Same page, section "The released stack": one shared expert is evaluated
 *   for every token besides the routed ones.  Same page, section "The FP8 path
 *   is explicitly mixed precision": FP8 E4M3 weights with FP32 scales, which
 *   are applied exactly (never rounded to powers of two).
 *   "Kolibri 1 Deep Dive" (abrarakhunji.com), "Mathematical Routing & Load
 *   Balancing Formulation": the output is the gate-weighted sum of the
 *   selected experts' outputs, added to the residual stream (the residual add
 *   is the caller's, or MOE_FLAG_ACCUMULATE).
 *
 *   out[t] = S(x_t) + sum_{j<k} w[t,j] * E_{ids[t,j]}(x_t)
 *
 * Conventions fixed by this library where the pages are silent:
 *   - equal scores select the lower expert id; the k ids of a token are
 *     stored in ascending id order (slot j = j-th smallest id);
 *   - the shared expert has coefficient 1;
 *   - FP8 is OCP E4M3FN (bias 7, max 448, no infinities); a weight is
 *     code * scale with one FP32 scale per output channel (row), or per
 *     128 x 128 block with MOE_FLAG_FP8_BLOCK128;
 *   - the expert matmuls take bfloat16 activations (an FP32 x is rounded to
 *     bfloat16 for the experts; the router always uses x as given);
 *   - dispatch is a stable counting sort of pairs by (expert, token).
 *
 * Memory: every pointer is device memory owned by the caller.  The library
 * allocates nothing and frees nothing.  Its only mutable global state is set
 * once per device on the first call there: a cache of the device architecture
 * check and the raised LDS limit of the GEMM kernels, and the address of the
 * static scratch array behind moe_forward_noalloc; plus the thread-local code
 * of the last HIP error.
 *
 * Execution: all work is enqueued on `stream` (a hipStream_t; NULL = the
 * default stream) without host synchronisation; results are valid once the
 * stream reaches that point.  `stream` must belong to the calling thread's
 * current device (hipSetDevice), which is the device that is checked and
 * configured.  Device faults surface at the caller's next
 * synchronisation.  Calls that share a workspace must be ordered on one
 * stream.  Calls can be captured in a HIP graph (no memset or host work is
 * enqueued); make the first call on each device outside a capture, since it
 * queries the device and sets kernel attributes.
 */
#ifndef FGS_MOE_H
#define FGS_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK               0
#define MOE_ERR_ARG         -1   /* null pointer, bad size, misaligned pointer, bad flag */
#define MOE_ERR_UNSUPPORTED -2   /* dtype combination, or the device is not gfx950 */
#define MOE_ERR_WORKSPACE   -3   /* workspace smaller than moe_workspace_size() */
#define MOE_ERR_HIP         -4   /* a HIP call failed; see moe_last_hip_error() */

/* element types */
#define MOE_DTYPE_F32       0
#define MOE_DTYPE_BF16      1
#define MOE_DTYPE_FP8_E4M3  2

/* flags */
#define MOE_FLAG_ACCUMULATE  (1u << 0)  /* out = round(out + y) instead of out = round(y) */
#define MOE_FLAG_RENORMALIZE (1u << 1)  /* mixture weights = softmax of the selected unbiased
                                           logits (sum to one), the gate of "Kolibri 1 Deep
                                           Dive", "Mathematical Routing & Load Balancing
                                           Formulation"; default off (sigmoid, not
                                           renormalised) */

#define MOE_FLAG_FP8_BLOCK128 (1u << 2) /* FP8 weights carry one FP32 scale per 128 x 128 block
                                           instead of one per output channel: the released
                                           checkpoint's layout, "Inside Kolibri 1" (flozi.net),
                                           section "The FP8 path is explicitly mixed precision".
                                           Requires w_dtype FP8_E4M3 and d_model, d_ff,
                                           d_ff_shared multiples of 128 (else MOE_ERR_ARG). */

#define MOE_FLAG_FP8_ACT_QUANT (1u << 3) /* FP8 x FP8 expert matmuls: the experts' input x and each
                                           expert's hidden activations are quantised on the fly in
                                           1 x 128 groups (moe_quantize_groups) and multiplied on the
                                           FP8 matrix cores; same page and section.  The router
                                           still reads x unquantised.  Requires w_dtype FP8_E4M3,
                                           x_dtype BF16 and d_model, d_ff, d_ff_shared multiples
                                           of 128 (else MOE_ERR_ARG). */

/* pipeline stages, for optional timing events */
#define MOE_STAGE_ROUTER    0   /* router logits */
#define MOE_STAGE_TOPK      1   /* bias-corrected top-k, sigmoid weights */
#define MOE_STAGE_DISPATCH  2   /* histogram, scan, scatter */
#define MOE_STAGE_GATE_UP   3   /* routed + shared gate/up projections and SwiGLU */
#define MOE_STAGE_DOWN      4   /* routed + shared down projections */
#define MOE_STAGE_COMBINE   5   /* weighted unpermute into out */
#define MOE_NUM_STAGES      6

/* Problem description.
 * Limits: n_tokens >= 0 (0 is a no-op); 1 <= top_k <= min(n_experts, 8);
 * 1 <= n_experts <= 1024; d_model, d_ff and d_ff_shared positive multiples
 * of 64; n_tokens * top_k < 2^31.
 * x_dtype: MOE_DTYPE_F32 or MOE_DTYPE_BF16 (out has the same type).
 * w_dtype: MOE_DTYPE_BF16 or MOE_DTYPE_FP8_E4M3 (routed and shared experts). */
typedef struct moe_desc {
    int32_t  n_tokens;     /* N */
    int32_t  d_model;      /* d (2560 in the pages' layer) */
    int32_t  n_experts;    /* E routed experts (384) */
    int32_t  top_k;        /* k (6) */
    int32_t  d_ff;         /* routed expert width f (512) */
    int32_t  d_ff_shared;  /* shared expert width f_s (512) */
    int32_t  x_dtype;
    int32_t  w_dtype;
    uint32_t flags;
} moe_desc;

/* Expert weights, row-major [out][in], element type desc->w_dtype.
 * Scales (FP32) are required for FP8 and must be NULL for bfloat16.  By
 * default there is one scale per output channel (the shapes below); with
 * MOE_FLAG_FP8_BLOCK128 one per 128 x 128 block, row-major over blocks:
 * s_gate, s_up [E][f/128][d/128], s_down [E][d/128][f/128], ss_gate, ss_up
 * [f_s/128][d/128], ss_down [d/128][f_s/128]; weight (o, i) then uses scale
 * (o/128, i/128).  All weight pointers 16-byte aligned. */
typedef struct moe_weights {
    const void  *w_gate;   /* [E][f][d] */
    const void  *w_up;     /* [E][f][d] */
    const void  *w_down;   /* [E][d][f] */
    const float *s_gate;   /* [E][f]   FP8 only */
    const float *s_up;     /* [E][f]   FP8 only */
    const float *s_down;   /* [E][d]   FP8 only */
    const void  *ws_gate;  /* [f_s][d] shared expert */
    const void  *ws_up;    /* [f_s][d] */
    const void  *ws_down;  /* [d][f_s] */
    const float *ss_gate;  /* [f_s]    FP8 only */
    const float *ss_up;    /* [f_s]    FP8 only */
    const float *ss_down;  /* [d]      FP8 only */
} moe_weights;

/* Optional outputs (every member may be NULL; the struct pointer may be NULL).
 * They expose the intermediate results of the call for inspection. */
typedef struct moe_aux {
    float   *logits;          /* [N][E] FP32 router logits h (unbiased) */
    int32_t *topk_ids;        /* [N][k] selected ids, ascending per token */
    float   *topk_w;          /* [N][k] sigmoid(h) at those ids */
    float   *gap;             /* [N] k-th minus (k+1)-th best biased score (+inf if k == E) */
    int32_t *expert_offsets;  /* [E+1] start row of each expert in the sorted buffer */
    int32_t *pair_of_row;     /* [N*k] pair t*k+j stored at each sorted row */
    int32_t *row_of_pair;     /* [N*k] sorted row of each pair t*k+j */
    void   **stage_events;    /* [2*MOE_NUM_STAGES] hipEvent_t or NULL each: recorded on
                                 `stream` before (2s) and after (2s+1) stage s */
} moe_aux;

/* Workspace bytes moe_forward needs for this description (0 on a bad
 * description).  Pure host function; touches no device. */
size_t moe_workspace_size(const moe_desc *desc);

/* One MoE sublayer:  out[t] = S(x_t) + sum_j w[t,j] E_{ids[t,j]}(x_t)
 * (plus the old out[t] with MOE_FLAG_ACCUMULATE), rounded once to x_dtype.
 *   x           [N][d]  x_dtype, 16-byte aligned
 *   router_w    [E][d]  FP32
 *   router_bias [E]     FP32 expert-correction bias
 *   weights     expert and shared-expert weights (above)
 *   out         [N][d]  x_dtype; must not overlap x unless ACCUMULATE is set
 *               and x == out (in-place residual)
 *   workspace   >= moe_workspace_size(desc) bytes, 256-byte aligned; its
 *               contents need no initialisation and are clobbered
 *   aux         optional intermediate outputs, may be NULL
 *   stream      hipStream_t
 * Returns MOE_OK or a negative status; on an error nothing is enqueued
 * except for MOE_ERR_HIP, where a launch failed part-way. */
int moe_forward(const moe_desc *desc, const void *x, const float *router_w,
                const float *router_bias, const moe_weights *weights, void *out,
                void *workspace, size_t workspace_bytes, const moe_aux *aux,
                void *stream);

/* Bytes of the per-GPU device array behind moe_forward_noalloc: the full
 * layer (d 2560, 384 experts, top-6, f 512) fits it up to 256 tokens in every
 * weight format. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The intermediates live in a library-owned device
 * array of MOE_NOALLOC_SCRATCH_BYTES per GPU (static storage of the code
 * object, held until the process ends); no call allocates or frees memory.
 * Arguments, semantics and errors as moe_forward, with the array as the
 * workspace: a description whose moe_workspace_size() exceeds
 * MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE before anything is
 * enqueued.  Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (no part of it needs to start at zero): calls that can
 * overlap on one GPU (several streams, or threads without ordering) race and
 * give undefined results, so order them on one stream.  The first call on each
 * device resolves the array's address; make it outside a graph capture. */
int moe_forward_noalloc(const moe_desc *desc, const void *x, const float *router_w,
                        const float *router_bias, const moe_weights *weights, void *out,
                        const moe_aux *aux, void *stream);

/* Workspace bytes moe_block_forward needs (0 on a bad description): the
 * moe_forward workspace plus room for the normalised input. */
size_t moe_block_workspace_size(const moe_desc *desc);

/* The MoE sublayer of a sandwich-normalised block, updating the residual
 * stream in place.  "Inside Kolibri 1" (flozi.net), section "The released
 * stack": RMSNorm before and after the MoE, residual addition after it.
 *   x     = RMSNorm(resid; norm_pre), rounded to x_dtype
 *   y     = the layer of moe_forward applied to x (FP32, before rounding)
 *   resid = round(resid + RMSNorm(y; norm_post))
 * with RMSNorm(v; g)_i = v_i / sqrt(mean_j v_j^2 + eps) * g_i (statistics in
 * FP32).  The post-norm and the residual add are fused into the combine.
 *   resid      [N][d] x_dtype, read and written (16-byte aligned)
 *   norm_pre   [d] FP32, norm_post [d] FP32 (16-byte aligned); eps >= 0
 *   workspace  >= moe_block_workspace_size(desc) bytes, 256-byte aligned
 * Other arguments and errors as moe_forward; MOE_FLAG_ACCUMULATE is rejected
 * (the residual add is part of this call). */
int moe_block_forward(const moe_desc *desc, void *resid, const float *norm_pre, const float *norm_post,
                      float eps, const float *router_w, const float *router_bias,
                      const moe_weights *weights, void *workspace, size_t workspace_bytes,
                      const moe_aux *aux, void *stream);

/* Dynamic FP8 quantisation in 1 x 128 groups, the activation format of
 * MOE_FLAG_FP8_ACT_QUANT ("Inside Kolibri 1", section "The FP8 path is
 * explicitly mixed precision": activations quantised dynamically in groups
 * of 1 x 128).  For each row r and group g of 128 consecutive columns:
 *   scale[r][g] = amax / 448 in FP32 (1 if the group is all zero),
 *   q[r][c]     = E4M3FN(v[r][c] / scale) with IEEE FP32 division, clamped to
 *                 +-448, rounded to nearest even.
 *   v       [rows][cols] v_dtype (MOE_DTYPE_F32 or MOE_DTYPE_BF16), row-major,
 *           16-byte aligned; cols a positive multiple of 128
 *   q       [rows][cols] uint8 codes, 8-byte aligned
 *   scales  [rows][cols/128] FP32, 4-byte aligned
 * rows == 0 is a no-op.  Device pointers owned by the caller; enqueued on
 * `stream`.  Returns MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED or MOE_ERR_HIP. */
int moe_quantize_groups(const void *v, int v_dtype, int64_t rows, int32_t cols, uint8_t *q, float *scales,
                        void *stream);

/* Static text for a status code. */
const char *moe_status_string(int status);

/* The hipError_t of the most recent MOE_ERR_HIP on the calling thread (0 if none). */
int moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FGS_MOE_H */
