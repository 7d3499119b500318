// Argument blocks and host launchers of the gfx950 kernels (internal to libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---- routing ------------------------------------------------------------------
struct RouteArgs {
    const float* logits;   // [T,E]
    int32_t* topk_idx;     // [T,k]
    float* gates;          // [T,k]
    int32_t* hist;         // [E][nchunk]
    float* qpart;          // [nchunk][E]
    int T, E, k, n_groups, topk_groups, score, nchunk;
    const float* bias;     // [E] correction bias (selection only) or NULL
    int group_score;       // MOE_GROUP_*
    float route_scale;     // gate multiplier after renormalisation
};
struct ScanArgs {
    const int32_t* hist;   // [E][nchunk]
    int32_t* cbase;        // [E][nchunk] exclusive prefix within each expert
    int32_t* counts;       // [E]
    int nchunk;
};
struct SlotArgs {
    const int32_t* counts;
    const int32_t* cbase;
    const int32_t* topk_idx;
    const float* gates;
    int32_t* offsets;      // [E+1]
    int32_t* tile_prefix;  // [3][MOE_MAX_EXPERTS+1]: m-tile prefix for 64/128/256-row tiles,
                           // then [MOE_MAX_EXPERTS+1]: the experts by rows, most first
    int32_t* slot_of;      // [T,k]
    int32_t* token_of;     // [T*k]
    float* gate_of;        // [T*k] gate of each expert-major row, or NULL
    int32_t* src_k;        // [T*k] pick index of each row, or NULL
    int T, E, k, nchunk;
};
struct FinalizeArgs {
    const float* qpart;
    const int32_t* counts;
    const float* lpart;    // NULL: no MSE
    int nlpart;
    float* aux_out;        // may be NULL
    float* loss_out;       // may be NULL; [mse, aux, mse + aux_coef*aux]
    float aux_coef;
    int T, d, E, k, nchunk;
};
struct RouterBwdArgs {
    const float* logits;
    const int32_t* topk_idx;
    const float* gates;
    const float* dgate;    // [T,k], or NULL: the gate gradient is summed from dgate_part
    const float* dgate_part;  // [nparts][rows] partial gate gradients of the expert-major rows
    const int32_t* slot_of;   // [T,k] (with dgate_part)
    int nparts; long part_ld;
    const int32_t* counts;
    void* dlogits;         // [T,E] dtype
    float aux_coef;
    int T, E, k, score;
    float route_scale;     // the gates passed in already carry it
};

hipError_t launch_route_topk(const RouteArgs& a, hipStream_t s);
hipError_t launch_expert_scan(const ScanArgs& a, int E, hipStream_t s);
hipError_t launch_slot_assign(const SlotArgs& a, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);
hipError_t launch_router_bwd(const RouterBwdArgs& a, int dtype, hipStream_t s);

// ---- dispatch / combine / elementwise ------------------------------------------
struct GatherArgs {
    const void* X; const int32_t* slot_of; void* Xp;
    int T, k, vec;         // vec = 16-byte vectors per row
};
struct CombineArgs {
    const void* EO; const int32_t* slot_of;
    const float* gates;    // [T,k], or NULL when EO rows already carry their gates
    void* Y;
    const void* Ys;        // shared-branch output [T, d] added to Y, or NULL
    const void* Yt;        // NULL: no loss
    void* dY;              // written when Yt != NULL: 2 (Y - Yt) / (T d)
    float* lpart;          // per-workgroup sum of squared residuals
    float inv_n2;          // 2 / (T d)
    int T, k, vec;
};
struct CombineBwdArgs {
    const void* dY; const void* EO; const int32_t* slot_of; const float* gates;
    float* dgate; void* dEO;
    int T, k, vec;
};
struct ScatterArgs {
    const void* dXp; const int32_t* slot_of; const float* dXr; void* dX;
    const void* dXs;       // shared-branch part of dX [T, d] added last, or NULL
    int T, k, vec;
};
struct ColSumArgs {
    const void* src; long ld; const int32_t* offsets; float* dst; int ncols, E;
};
// One SGD launch updates up to MOE_SGD_MAX_SEG parameter tensors; segment s owns
// workgroups [blk0[s], blk0[s+1]).
constexpr int MOE_SGD_MAX_SEG = 9;
struct SgdSeg {
    float* master; const float* grad; void* work; long n;
};
struct SgdArgs {
    SgdSeg seg[MOE_SGD_MAX_SEG];
    int blk0[MOE_SGD_MAX_SEG + 1];
    int nseg;
    float lr;
};

hipError_t launch_gather(const GatherArgs& a, int dtype, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t s);
hipError_t launch_combine_bwd(const CombineBwdArgs& a, int dtype, hipStream_t s);
hipError_t launch_scatter(const ScatterArgs& a, int dtype, hipStream_t s);
hipError_t launch_colsum(const ColSumArgs& a, int dtype, hipStream_t s);
// Fills blk0 from the segment sizes and launches one SGD kernel over all segments.
hipError_t launch_sgd(SgdArgs& a, int dtype, hipStream_t s);
int combine_loss_blocks(int T);
// Tables of the shared-experts branch as one expert segment of all T rows:
// offsets {0, T} in tab[0..1], then the m-tile prefix per tile height (64, 128,
// 256 rows) at tab + 2 + b * (MOE_MAX_EXPERTS + 1), as the routing writes it.
hipError_t launch_shared_table(int32_t* tab, int T, hipStream_t s);

// ---- expert / router contractions -------------------------------------------------
enum GemmEpi {
    EPI_STORE = 0,         // C = acc, dtype or fp32
    EPI_UP_SWIGLU = 1,     // H1|H3 and A = silu(H1) * H3
    EPI_UP_RELU = 2,       // H = acc + b1, A = relu(H)
    EPI_UP_GELU = 3,       // H = acc + b1, A = gelu(H)
    EPI_DN_SWIGLU = 4,     // dH1 = dA*H3*silu'(H1), dH3 = dA*silu(H1)
    EPI_DN_RELU = 5,       // dH = dA * relu'(H)
    EPI_DN_GELU = 6,       // dH = dA * gelu'(H)
    EPI_SGD = 7,           // weight gradient applied as an SGD step instead of stored:
                           // master = fma(-lr, acc, master), working copy = bf16(master)
    EPI_STORE_BIAS = 8,    // bf16 C = acc + bias per column (MLP down projection)
    EPI_UP_SWIGLU_G = 9,   // EPI_UP_SWIGLU with A scaled by the gate of its row
    EPI_DN_SWIGLU_G = 10,  // EPI_DN_SWIGLU from dA = gate * acc, plus the row partials
                           // of <acc, silu(H1) * H3> (the gate gradient)
    EPI_SCATTER = 11,      // router dX: bf16 dX = sum of the token's k expert rows + acc
                           // (+ the shared branch's part), the scatter's order and rounding
};

// Expert contractions of the layer.  All row-major; see each field.
struct ExpertGemmArgs {
    int T, d, E, ffn, k, rows;       // rows = T*k
    const int32_t* offsets;          // [E+1]
    const int32_t* tile_prefix;      // [3][MOE_MAX_EXPERTS+1] m-tile prefixes, then the
                                     // experts by rows, most first [MOE_MAX_EXPERTS+1]
    int32_t* queue;                  // [8] tile counters of the persistent weight gradients
    const void* Xp; const void* W1; const void* W3; const void* b1;
    const void* W2; const void* b2;
    void* H; void* A; void* EO;      // forward outputs / saved
    const void* dEO; void* dH; void* dXp;  // backward
    float* dW1; float* dW3; float* dW2;
    int expert;                      // MOE_EXPERT_*
    // SGD fused into the weight-gradient contractions (training step without stored
    // expert gradients): when W1m is set, the up-projection wgrad updates W1m/W1w (and
    // W3m/W3w) in place of writing dW1 (dW3); when W2m is set, the down-projection wgrad
    // updates W2m/W2w in place of writing dW2.  m = fp32 masters, w = working copies.
    float* W1m; float* W3m; float* W2m;
    void* W1w; void* W3w; void* W2w;
    float lr;
    // Fused dispatch (SwiGLU, bf16), when token_of is set: the expert-major rows of the
    // layer input and of dY are read from the token-major X and dY through token_of
    // instead of from gathered copies; A is stored scaled by each row's gate (so EO
    // comes out gate-weighted); the down dgrad takes dA = gate * (dY W2) and writes each
    // row's partial gate gradient per 256-column tile into dgate_part [tiles][rows].
    const int32_t* token_of;         // [rows] token of each expert-major row
    const float* gate_of;            // [rows] gate of each expert-major row
    const void* X;                   // [T, d] layer input
    const void* dY;                  // [T, d] gradient of Y
    float* dgate_part;               // [ceil(ffn / 256)][rows]
};
// float32 layer (gemm_simple.hip): one thread per output element, fp32 accumulate.
hipError_t simple_up_fwd(const ExpertGemmArgs& a, hipStream_t s);
hipError_t simple_down_fwd(const ExpertGemmArgs& a, hipStream_t s);
hipError_t simple_down_dgrad(const ExpertGemmArgs& a, hipStream_t s);
hipError_t simple_up_dgrad(const ExpertGemmArgs& a, hipStream_t s);
hipError_t simple_down_wgrad(const ExpertGemmArgs& a, hipStream_t s);
hipError_t simple_up_wgrad(const ExpertGemmArgs& a, hipStream_t s);
// bfloat16 layer (gemm_mfma.hip): grouped MFMA tiles scheduled on the device.
hipError_t mfma_up_fwd(const ExpertGemmArgs& a, hipStream_t s);
// whether mfma_up_fwd takes 128-row tiles for this shape (then it runs in this build, not kt64)
bool mfma_up_fwd_short(const ExpertGemmArgs& a);
namespace kt64 {
// the up projection with 64-deep k-tiles and register-staged loads (gemm_mfma_kt64.hip)
hipError_t mfma_up_fwd(const ExpertGemmArgs& a, hipStream_t s);
}
hipError_t mfma_down_fwd(const ExpertGemmArgs& a, hipStream_t s);
hipError_t mfma_down_dgrad(const ExpertGemmArgs& a, hipStream_t s);
hipError_t mfma_up_dgrad(const ExpertGemmArgs& a, hipStream_t s);
hipError_t mfma_down_wgrad(const ExpertGemmArgs& a, hipStream_t s);
hipError_t mfma_up_wgrad(const ExpertGemmArgs& a, hipStream_t s);

struct RouterGemmArgs {
    int T, d, E;
    const void* X; const void* Wg; const void* dl;
    float* logits; float* dXr; float* dWg;
    float* dwg_part;       // bf16 path: router_dwg_splits(T, E, d) x [E,d] fp32 partials, or NULL
    float* logit_part;     // bf16 path: router_logit_splits(T, E, d) x [T,E] fp32 partials, or NULL
};
int router_dwg_splits(int T, int E, int d);
int router_dwg_kchunk(int T, int E, int d);
int router_logit_splits(int T, int E, int d);
hipError_t simple_router_logits(const RouterGemmArgs& a, hipStream_t s);
hipError_t simple_router_dx(const RouterGemmArgs& a, hipStream_t s);
hipError_t simple_router_dwg(const RouterGemmArgs& a, hipStream_t s);
hipError_t mfma_router_logits(const RouterGemmArgs& a, hipStream_t s);
hipError_t mfma_router_dx(const RouterGemmArgs& a, hipStream_t s);
// The router dX contraction with the scatter in its epilogue (bf16, k = MOE_SCATTER_FUSED_K):
// writes sa.dX = sum over the token's k rows of sa.dXp + dl Wg (+ sa.dXs) and no dXr.
constexpr int MOE_SCATTER_FUSED_K = 8;
hipError_t mfma_router_dx_scatter(const RouterGemmArgs& a, const ScatterArgs& sa, hipStream_t s);
hipError_t mfma_router_dwg(const RouterGemmArgs& a, hipStream_t s);

}  // namespace moe
