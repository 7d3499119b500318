/*
 * moe.h -- C ABI of the MI355X (gfx950) trainable sparse mixture-of-experts layer.
 *
 * The layer (sources: the "Trainable MoE in CUDA" course outline, Parts 1-7;
 * "AI Infra Kernel Lab" README, sections "Project status" and "Numerical
 * contracts"):
 *
 *   logits  l = X Wg^T                                   (outline Part 3)
 *   scores  softmax over experts, or elementwise sigmoid  (outline Part 3; Infra Lab grouped gate)
 *   select  group-limited top-k on the logits; groups are consecutive blocks
 *           of E/n_groups experts scored by their largest member; ties go to
 *           the smaller group / expert id                 (Infra Lab "Project status")
 *           Variants of the DeepSeek gate: an optional correction bias that
 *           enters selection only, and a group score equal to the sum of the
 *           group's two largest members; selection then ranks the fp32
 *           scores plus the bias             (Infra Lab "Numerical contracts")
 *   gates   g = c * w_sel / sum(w_sel), w = the selected unbiased scores,
 *           c = route_scale (default 1)    (outline Part 2)
 *   dispatch per-expert histogram, exclusive scan, stable slots in ascending
 *           token order, gather into expert-major rows    (outline Part 4)
 *   experts ReLU/GELU MLP with biases, or SwiGLU W2(silu(W1 x) * W3 x)
 *                                                          (outline Part 5; Infra Lab "Numerical contracts")
 *   combine Y_t = sum_i g_ti EO[slot(t,i)]                (outline Part 4)
 *   aux     E * sum_e f_e P_e with f_e = count_e/(T k), P_e = mean_t q_te
 *                                                          (outline Part 6)
 *   loss    MSE (mean over T*d) + aux_coef * aux; SGD      (outline Part 7)
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer on the current HIP device,
 *     except the struct pointers themselves (host memory, read during the call).
 *   - Row-major, densely packed tensors.  "dtype" tensors are float32 when
 *     cfg->dtype == MOE_DTYPE_F32 and bfloat16 when MOE_DTYPE_BF16.
 *   - Device pointers must be 16-byte aligned.
 *   - The caller owns and allocates every buffer, the workspace included.
 *     The library never allocates, frees, or synchronises the stream, and
 *     keeps no state between calls.  All work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream).
 *   - Inputs are never written.  Outputs are overwritten completely
 *     (gradients of experts that received no rows are written as zeros).
 *   - All validation happens before the first launch; on an error nothing is
 *     written.  A launch failure returns MOE_ERR_HIP.
 *   - Results are deterministic: the same inputs give bitwise identical
 *     outputs (no floating-point atomics anywhere).
 *   - T == 0 is valid and returns MOE_OK after writing only zero-sized outputs
 *     (gradients of the weights are still written, as zeros).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK                 0
#define MOE_ERR_INVALID_ARG   -1  /* shape/config rule broken (see moe_config) */
#define MOE_ERR_NULL_PTR      -2  /* a required pointer is NULL */
#define MOE_ERR_MISALIGNED    -3  /* a device pointer is not 16-byte aligned */
#define MOE_ERR_WORKSPACE     -4  /* workspace NULL or smaller than moe_workspace_bytes() */
#define MOE_ERR_UNSUPPORTED   -5  /* valid layer, but outside what the kernels support */
#define MOE_ERR_HIP           -6  /* a HIP launch failed */
#define MOE_ERR_SCRATCH       -7  /* moe_route_noalloc: the shape needs more scratch than
                                     MOE_ROUTE_SCRATCH_BYTES */

/* ---- enums ------------------------------------------------------------- */
#define MOE_SCORE_SOFTMAX   0
#define MOE_SCORE_SIGMOID   1
#define MOE_EXPERT_RELU     0     /* MLP with biases, ReLU */
#define MOE_EXPERT_GELU     1     /* MLP with biases, exact-erf GELU */
#define MOE_EXPERT_SWIGLU   2     /* W2 (silu(W1 x) * W3 x), no biases */
#define MOE_DTYPE_F32       0
#define MOE_DTYPE_BF16      1     /* bf16 storage and MFMA inputs, fp32 accumulation */
#define MOE_GROUP_MAX       0     /* group score = largest member logit */
#define MOE_GROUP_TOP2_SUM  1     /* group score = sum of the two largest member values */

#define MOE_MAX_EXPERTS   256
#define MOE_MAX_K          16

/*
 * Layer shape.  Rules (MOE_ERR_INVALID_ARG when broken): T >= 0; d, E, ffn,
 * k, n_groups, topk_groups >= 1; k <= E; E % n_groups == 0;
 * topk_groups <= n_groups; k <= topk_groups * (E / n_groups);
 * T * k < 2^31; group_score is MOE_GROUP_MAX or MOE_GROUP_TOP2_SUM, and
 * MOE_GROUP_TOP2_SUM with n_groups > 1 needs E / n_groups >= 2; route_scale
 * is finite and >= 0 (0 stands for 1, so that a zeroed struct is the plain
 * layer).
 * Selection values: the logits when group_score == MOE_GROUP_MAX and no
 * correction bias is given (exact); otherwise the fp32 scores (softmax
 * probabilities or sigmoid values) plus the correction bias, added in fp32.
 * n_shared >= 0 and n_shared * ffn <= 2^24: the shared-experts branch, one
 * SwiGLU over every token with hidden width Hs = n_shared * ffn (0 = none).
 * fused_dispatch is 0 or 1 ("AI Infra Kernel Lab" README, "Project status": the
 * fused native path, whose private histogram/scan/scatter pack and weighted
 * down-projection epilogue cut the intermediate bytes; "Validation evidence":
 * its byte inventory).  0, the staged path: the token rows are gathered into
 * expert-major copies (Xp), the expert outputs are combined with their gates,
 * and the combine backward writes dEO = gate * dY rows.  1, fused: the up
 * projection and both weight gradients read the token rows of X and dY through
 * token_of (no Xp, no dEO); the up projection stores each row's A scaled by its
 * gate, so the down projection's outputs come gate-weighted and the combine is
 * a plain sum; the down-projection dgrad applies the gate to dY W2 and computes
 * the gate gradient <dY_t, EO> there as <dY_t W2, silu(H1) * H3>.  Same
 * results within rounding; bf16 SwiGLU only (else MOE_ERR_UNSUPPORTED).  In the
 * fused path the saved A and EO hold the gate-scaled rows and MOE_WS_XP has no
 * buffer.
 * Kernel limits (MOE_ERR_UNSUPPORTED): E <= 256, k <= 16; float32: d and ffn
 * multiples of 4; bfloat16: d and ffn multiples of 64, E a multiple of 8, and
 * T * max(d, hcols, 2 Hs) * 2 < 2^31 (hcols = 2 ffn for SwiGLU, else ffn): an
 * expert's rows of a k-strided GEMM operand, up to T of them, must span less
 * than 2 GiB; and max(ffn, Hs) * d * 4 < 2^31: one expert's (or the shared
 * branch's) weight matrix, as float32 masters, must span less than 2 GiB.
 */
typedef struct moe_config {
    int32_t T;            /* tokens */
    int32_t d;            /* model width */
    int32_t E;            /* experts */
    int32_t ffn;          /* expert hidden width */
    int32_t k;            /* experts per token */
    int32_t n_groups;     /* expert groups (1 = no group limit) */
    int32_t topk_groups;  /* groups kept per token */
    int32_t score;        /* MOE_SCORE_* */
    int32_t expert;       /* MOE_EXPERT_* */
    int32_t dtype;        /* MOE_DTYPE_* */
    int32_t group_score;  /* MOE_GROUP_* */
    float   route_scale;  /* gate multiplier after renormalisation; 0 = 1 */
    int32_t n_shared;     /* shared experts (hidden Hs = n_shared * ffn); 0 = none */
    int32_t fused_dispatch; /* 0: staged dispatch; 1: fused dispatch (below) */
} moe_config;

/*
 * Weights in the working dtype.  Wg [E,d]; W1 [E,ffn,d]; b1 [E,ffn];
 * W2 [E,d,ffn]; b2 [E,d]; W3 [E,ffn,d].  b1/b2 are required for the MLP
 * kinds and ignored (may be NULL) for SwiGLU; W3 is required for SwiGLU only.
 * e_bias float [E] is the optional correction bias of the DeepSeek gate (NULL
 * = none; only with MOE_SCORE_SIGMOID, else MOE_ERR_INVALID_ARG): it is added
 * to the scores for selection only; gates and every gradient use the unbiased
 * scores, and no gradient is computed for it.
 * Shared-experts branch ("AI Infra Kernel Lab", the benchmark's shared branch:
 * one replicated SwiGLU whose output is added to the routed combine with no
 * gate): Ws1, Ws3 [Hs,d] and Ws2 [d,Hs] in the working dtype, required when
 * n_shared > 0 and ignored otherwise.
 */
typedef struct moe_weights {
    const void* Wg;
    const void* W1;
    const void* b1;
    const void* W2;
    const void* b2;
    const void* W3;
    const float* e_bias;
    const void* Ws1;
    const void* Ws3;
    const void* Ws2;
} moe_weights;

/*
 * Routing outputs of the forward (all written by moe_forward / moe_route):
 *   logits   float [T,E]   router logits in fp32 (moe_route: ignored, may be NULL)
 *   topk_idx int32 [T,k]   selected experts, in (-selection value, id) order
 *   gates    float [T,k]   renormalised gates times route_scale, same order
 *   counts   int32 [E]     rows per expert
 *   offsets  int32 [E+1]   exclusive scan of counts
 *   slot_of  int32 [T,k]   expert-major row of (t, i)
 *   token_of int32 [T*k]   token of each expert-major row
 *   aux      float [1]     aux load-balancing loss (unscaled)
 *   src_k    int32 [T*k]   pick index i of each expert-major row, so that
 *                          slot_of[token_of[p], src_k[p]] == p; optional: NULL
 *                          leaves it unwritten (no kernel of this library reads it)
 * token_of and src_k are the inverse of slot_of ("Trainable MoE in CUDA" outline
 * Part 4, the packed dispatch tables).
 * moe_backward reads logits, topk_idx, gates, counts, slot_of and token_of.
 */
typedef struct moe_routing {
    float*   logits;
    int32_t* topk_idx;
    float*   gates;
    int32_t* counts;
    int32_t* offsets;
    int32_t* slot_of;
    int32_t* token_of;
    float*   aux;
    int32_t* src_k;
} moe_routing;

/*
 * Gradients written by moe_backward / moe_train_step.  dX is dtype [T,d]
 * (expert path plus router path plus shared branch); the rest are float32
 * with the shapes of the weights.  db1/db2 are required for the MLP kinds,
 * dW3 for SwiGLU, dWs1/dWs3/dWs2 when n_shared > 0.
 */
typedef struct moe_grads {
    void*  dX;
    float* dWg;
    float* dW1;
    float* db1;
    float* dW2;
    float* db2;
    float* dW3;
    float* dWs1;
    float* dWs3;
    float* dWs2;
} moe_grads;

/*
 * Parameters updated in place by moe_train_step: float32 masters and the
 * working copies (dtype).  For MOE_DTYPE_F32 a working pointer may equal its
 * master.  For bf16 the working copy is rewritten as the round-to-nearest-
 * even conversion of the updated master.  e_bias is the optional correction
 * bias (as in moe_weights); it is read, never updated.
 */
typedef struct moe_params {
    float* Wg;  float* W1;  float* b1;  float* W2;  float* b2;  float* W3;
    void*  Wg_w; void* W1_w; void* b1_w; void* W2_w; void* b2_w; void* W3_w;
    const float* e_bias;
    float* Ws1; float* Ws3; float* Ws2;        /* shared branch (n_shared > 0) */
    void*  Ws1_w; void* Ws3_w; void* Ws2_w;
} moe_params;

/* Workspace buffers whose byte offsets moe_workspace_offset() reports.
 * They hold the forward's saved activations, read back by moe_backward:
 *   XP    dtype [T*k, d]    gathered expert-major rows (none with fused dispatch)
 *   H     dtype [T*k, hcols] pre-activations; hcols = 2*ffn for SwiGLU
 *                           ([H1 | H3] per row), ffn for the MLP kinds
 *   A     dtype [T*k, ffn]  activations fed to the down projection
 *   EO    dtype [T*k, d]    expert outputs, expert-major
 */
#define MOE_WS_XP   0
#define MOE_WS_H    1
#define MOE_WS_A    2
#define MOE_WS_EO   3

/* Bytes of workspace every entry point needs for this shape (0 on an invalid
 * shape).  The same workspace must be passed to moe_forward and then to
 * moe_backward: it carries the saved activations between them. */
size_t moe_workspace_bytes(const moe_config* cfg);

/* Byte offset of a saved-activation buffer (MOE_WS_*) inside the workspace,
 * or -1 for an invalid shape or buffer id, and for MOE_WS_XP with fused
 * dispatch.  For inspection only. */
int64_t moe_workspace_offset(const moe_config* cfg, int32_t which);

/*
 * Routing only, from caller-supplied fp32 logits [T,E]: scores, group-limited
 * top-k, gates, histogram, scan and slot maps, and the aux value (steps of
 * outline Parts 2, 3, 4 and 6).  e_bias: the optional correction bias
 * (float [E] or NULL, as in moe_weights).  Writes every field of *r except
 * r->logits.
 */
int moe_route(const moe_config* cfg, const float* logits, const float* e_bias,
              moe_routing* r, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and outputs as moe_route, minus the workspace:
 * the kernels' scratch (per-64-token-chunk histograms, scan bases and aux
 * partial sums, and the GEMM tile prefixes) lives in one static device array
 * of MOE_ROUTE_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends.  Nothing is allocated or freed, and no scratch entry needs
 * clearing (each is written before it is read within the call).
 * Limit: 3 * align256(E * ceil(T / 64) * 4) + align256(4 * 257 * 4) bytes must
 * fit in MOE_ROUTE_SCRATCH_BYTES (T up to 174,656 tokens at E = 256), else
 * MOE_ERR_SCRATCH before any launch.  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams or host threads) race
 * and must be serialised by the caller.  The first call on a device resolves
 * the array's address there (MOE_ERR_HIP if that fails).
 */
#define MOE_ROUTE_SCRATCH_BYTES  (8u << 20)
int moe_route_noalloc(const moe_config* cfg, const float* logits, const float* e_bias,
                      moe_routing* r, void* stream);

/*
 * Forward of the layer: router GEMM, routing, gather, expert up and down
 * projections, combine (outline Parts 3-6).  X dtype [T,d] in; Y dtype [T,d]
 * and every field of *r out; saved activations go to the workspace.
 */
int moe_forward(const moe_config* cfg, const void* X, const moe_weights* w,
                void* Y, moe_routing* r,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of the layer (outline Parts 1-6 backward passes): from the
 * caller's dY (dtype [T,d], the gradient of the loss with respect to Y) and
 * aux_coef (the weight of the aux loss in the total loss), writes every
 * gradient in *g.  Must follow moe_forward with the same cfg, X, w, *r and
 * workspace, with no other call on that workspace in between.
 */
int moe_backward(const moe_config* cfg, const void* X, const moe_weights* w,
                 const moe_routing* r, const void* dY, float aux_coef,
                 moe_grads* g, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One training step (outline Part 7): forward, loss = MSE(Y, Y_target) +
 * aux_coef * aux, backward, then SGD with learning rate lr on every
 * parameter (masters, then working copies).  Y_target dtype [T,d].
 * Writes Y, *r, *g and loss_out (device float[3] = {mse, aux, loss}).
 *
 * The expert weight gradients g->dW1, g->dW2 (g->dW3 for SwiGLU; g->dWs1,
 * g->dWs3, g->dWs2 when n_shared > 0) are either all given or all NULL; a
 * mix fails with MOE_ERR_NULL_PTR.  When they are NULL, nothing is stored
 * for them: the weight-gradient contractions apply the SGD step to those
 * weights and their working copies directly, which saves writing and
 * re-reading the gradients (about 8 bytes per expert parameter).  Each
 * updated value is the same in both modes: master = fma(-lr, grad, master)
 * in float32, with grad the same float32 sum.  The other gradients (dX, dWg,
 * db1, db2) are always written.
 */
int moe_train_step(const moe_config* cfg, const void* X, const void* Y_target,
                   moe_params* p, float lr, float aux_coef,
                   void* Y, moe_routing* r, moe_grads* g, float* loss_out,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Stages of one training step, in launch order (moe_train_step_profiled). */
#define MOE_STAGE_ROUTER_LOGITS   0   /* l = X Wg^T                               */
#define MOE_STAGE_ROUTE           1   /* top-k, gates, histogram, scan, slots, aux */
#define MOE_STAGE_GATHER          2   /* Xp = X[token_of]                         */
#define MOE_STAGE_UP_FWD          3   /* H = Xp W1^T (|W3^T), A = act(H)          */
#define MOE_STAGE_DOWN_FWD        4   /* EO = A W2^T (+ b2)                       */
#define MOE_STAGE_SHARED_FWD      5   /* shared branch Ys = SwiGLU(X) (n_shared > 0) */
#define MOE_STAGE_COMBINE_LOSS    6   /* Y (+ Ys), MSE, dY, loss scalars          */
#define MOE_STAGE_COMBINE_BWD     7   /* dgate, dEO                               */
#define MOE_STAGE_DOWN_DGRAD      8   /* dA = dEO W2, activation backward         */
#define MOE_STAGE_DOWN_WGRAD      9   /* dW2 = dEO^T A (fused: + SGD on W2)        */
#define MOE_STAGE_UP_DGRAD       10   /* dXp = dH W1 (+ dH3 W3)                   */
#define MOE_STAGE_UP_WGRAD       11   /* dW1 (| dW3) = dH^T Xp (fused: + SGD)      */
#define MOE_STAGE_SHARED_BWD     12   /* shared branch dgrad and wgrad (fused: + SGD) */
#define MOE_STAGE_BIAS_GRADS     13   /* db1, db2 (MLP kinds)                     */
#define MOE_STAGE_ROUTER_BWD     14   /* dlogits                                  */
#define MOE_STAGE_ROUTER_DWG     15   /* dWg = dl^T X                             */
#define MOE_STAGE_ROUTER_DX      16   /* router part of dX = dl Wg                */
#define MOE_STAGE_SCATTER        17   /* dX = sum of dXp rows + router part (+ shared) */
#define MOE_STAGE_SGD            18   /* masters and working copies (fused: Wg and
                                         the biases only)                          */
#define MOE_NUM_STAGES           19

/*
 * moe_train_step with timing marks: the same launches, plus
 * hipEventRecord(events[i], stream) right before the launches of stage i and
 * hipEventRecord(events[MOE_NUM_STAGES], stream) after the last one.
 * `events` holds MOE_NUM_STAGES + 1 hipEvent_t created by the caller
 * (hipEventCreate); stage i took hipEventElapsedTime(events[i], events[i+1]).
 * For measurement tools; identical results to moe_train_step.
 */
int moe_train_step_profiled(const moe_config* cfg, const void* X, const void* Y_target,
                            moe_params* p, float lr, float aux_coef,
                            void* Y, moe_routing* r, moe_grads* g, float* loss_out,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events);

/* Static text for a status code. */
const char* moe_status_string(int status);

/* ABI version (incremented on any incompatible change). */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
