// C ABI of the sparse MoE layer: validation, workspace layout and the launch
// sequence of each entry point (declared in include/moe.h).
//
// Sources: "Trainable MoE in CUDA" outline Parts 1-7 (the steps, in order:
// router, top-k gating, dispatch/combine, expert MLP, aux loss, loss and SGD);
// "AI Infra Kernel Lab" README "Quick start" (one public call that routes,
// packs, computes experts and combines; explicit native paths fail rather
// than fall back) and "Project status".
//
// Every call validates all of its arguments before the first launch, then
// enqueues its kernels on the caller's stream with no host synchronisation:
// counts, offsets and the expert GEMM tile schedule never leave the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.hpp"

using namespace moe;

// The scratch of moe_route_noalloc: one static device array, which each GPU the library
// runs on holds until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory; its device address on each GPU comes from hipGetSymbolAddress (taken
// once per device, with that device current, in scratch_ptr below) and only that address
// is ever passed on.
static __device__ __align__(256) unsigned char scratch[MOE_ROUTE_SCRATCH_BYTES];

namespace {

constexpr int kChunk = 64;

enum WsBuf {
    B_XP = 0, B_H, B_A, B_EO, B_DEO, B_DH, B_DXP, B_DY, B_DXR, B_DL, B_DGATE, B_GATEOF, B_DGPART,
    B_HIST, B_CBASE, B_QPART, B_LPART, B_TPREFIX, B_QUEUE, B_DWGPART, B_LOGPART,
    // shared-experts branch: [H1 | H3] [T, 2 Hs], A [T, Hs], Ys [T, d], dH [T, 2 Hs],
    // dX part [T, d], and its one-segment tables (offsets {0, T}, tile prefixes)
    B_HS, B_AS, B_YS, B_DHS, B_DXS, B_STAB,
    B_COUNT
};
constexpr int kTabs = 4 * (MOE_MAX_EXPERTS + 1);            // m-tile prefixes (3) and segment order
constexpr int kSharedTab = 2 + kTabs;                       // int32 entries of B_STAB

struct Layout {
    size_t off[B_COUNT];
    size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
template <class P> inline bool aligned16(const P* p) { return ((uintptr_t)p & 15u) == 0; }

bool shape_ok(const moe_config* c) {
    if (!c) return false;
    if (c->T < 0 || c->d < 1 || c->E < 1 || c->ffn < 1 || c->k < 1 || c->n_groups < 1 ||
        c->topk_groups < 1)
        return false;
    if (c->k > c->E || c->E % c->n_groups != 0 || c->topk_groups > c->n_groups) return false;
    if ((int64_t)c->k > (int64_t)c->topk_groups * (c->E / c->n_groups)) return false;
    if ((int64_t)c->T * c->k >= (int64_t(1) << 31)) return false;
    if (c->score != MOE_SCORE_SOFTMAX && c->score != MOE_SCORE_SIGMOID) return false;
    if (c->expert < MOE_EXPERT_RELU || c->expert > MOE_EXPERT_SWIGLU) return false;
    if (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16) return false;
    if (c->group_score != MOE_GROUP_MAX && c->group_score != MOE_GROUP_TOP2_SUM) return false;
    if (c->group_score == MOE_GROUP_TOP2_SUM && c->n_groups > 1 && c->E / c->n_groups < 2) return false;
    if (!std::isfinite(c->route_scale) || c->route_scale < 0.f) return false;
    if (c->n_shared < 0 || (int64_t)c->n_shared * c->ffn > (int64_t(1) << 24)) return false;
    if (c->fused_dispatch != 0 && c->fused_dispatch != 1) return false;
    return true;
}

inline bool fused(const moe_config* c) { return c->fused_dispatch == 1; }
// bf16 with k = MOE_SCATTER_FUSED_K: the scatter runs in the router dX contraction's epilogue
inline bool scatter_in_router_dx(const moe_config* c) {
    return c->dtype != MOE_DTYPE_F32 && c->k == MOE_SCATTER_FUSED_K;
}
// tiles of 256 columns of the down-projection dgrad: partial gate gradients per row
inline int dgate_parts(const moe_config* c) { return (c->ffn + 255) / 256; }

inline int shared_hidden(const moe_config* c) { return c->n_shared * c->ffn; }

inline float route_scale(const moe_config* c) { return c->route_scale == 0.f ? 1.f : c->route_scale; }

// The correction bias is optional, sigmoid scoring only, and read as fp32 [E].
int check_bias(const moe_config* c, const float* e_bias) {
    if (!e_bias) return MOE_OK;
    if (c->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
    return aligned16(e_bias) ? MOE_OK : MOE_ERR_MISALIGNED;
}

int supported(const moe_config* c) {
    if (c->E > MOE_MAX_EXPERTS || c->k > MOE_MAX_K || c->n_groups > 128) return MOE_ERR_UNSUPPORTED;
    // fused dispatch: the bf16 SwiGLU contractions only
    if (fused(c) && (c->dtype != MOE_DTYPE_BF16 || c->expert != MOE_EXPERT_SWIGLU)) return MOE_ERR_UNSUPPORTED;
    if (c->dtype == MOE_DTYPE_F32) {
        if (c->d % 4 || c->ffn % 4) return MOE_ERR_UNSUPPORTED;
    } else {
        if (c->d % 64 || c->ffn % 64 || c->E % 8) return MOE_ERR_UNSUPPORTED;
        // The grouped GEMMs address an expert's rows of a k-strided operand (up to T rows of
        // up to max(d, hcols) bf16) through one buffer descriptor with 32-bit offsets.
        const int64_t widest = std::max<int64_t>({(int64_t)c->d,
                                                  c->expert == MOE_EXPERT_SWIGLU ? 2 * (int64_t)c->ffn : c->ffn,
                                                  2 * (int64_t)c->n_shared * c->ffn});
        if ((int64_t)c->T * widest * 2 >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
        // One expert's weight block (and the shared branch's) is addressed through one
        // descriptor too, as fp32 masters in the fused SGD step: ffn x d (Hs x d) floats.
        const int64_t wrows = std::max<int64_t>(c->ffn, (int64_t)c->n_shared * c->ffn);
        if (wrows * c->d * 4 >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

inline int esize(const moe_config* c) { return c->dtype == MOE_DTYPE_F32 ? 4 : 2; }
inline int hcols(const moe_config* c) { return c->expert == MOE_EXPERT_SWIGLU ? 2 * c->ffn : c->ffn; }
inline int nchunk(const moe_config* c) { return (c->T + kChunk - 1) / kChunk; }

Layout layout(const moe_config* c) {
    Layout L;
    const size_t s = esize(c), T = c->T, rows = (size_t)c->T * c->k, d = c->d, E = c->E;
    const size_t nc = nchunk(c);
    size_t sz[B_COUNT];
    // fused dispatch: no gathered rows and no dEO (read through token_of from X and dY)
    sz[B_XP] = fused(c) ? 0 : rows * d * s;
    sz[B_H] = rows * hcols(c) * s;
    sz[B_A] = rows * c->ffn * s;
    sz[B_EO] = rows * d * s;
    sz[B_DEO] = fused(c) ? 0 : rows * d * s;
    sz[B_DH] = rows * hcols(c) * s;
    sz[B_DXP] = rows * d * s;
    sz[B_DY] = T * d * s;
    // the fp32 router part of dX: not stored when the scatter runs in the router dX
    // contraction's epilogue (bf16, k = MOE_SCATTER_FUSED_K)
    sz[B_DXR] = scatter_in_router_dx(c) ? 0 : T * d * 4;
    sz[B_DL] = T * E * s;
    sz[B_DGATE] = fused(c) ? 0 : T * c->k * 4;       // fused dispatch: partials in B_DGPART
    sz[B_GATEOF] = fused(c) ? rows * 4 : 0;          // read only by the fused-dispatch GEMMs
    sz[B_DGPART] = fused(c) ? (size_t)dgate_parts(c) * rows * 4 : 0;
    sz[B_HIST] = E * nc * 4;
    sz[B_CBASE] = E * nc * 4;
    sz[B_QPART] = nc * E * 4;
    sz[B_LPART] = (size_t)combine_loss_blocks(c->T) * 4;
    sz[B_TPREFIX] = kTabs * 4;
    sz[B_QUEUE] = 8 * 4;
    // split-K partials of the router weight gradient (bf16 path only)
    const int nsplit = c->dtype == MOE_DTYPE_F32 ? 0 : router_dwg_splits(c->T, c->E, c->d);
    sz[B_DWGPART] = nsplit > 1 ? (size_t)nsplit * E * d * 4 : 0;
    // split-K partials of the router logits (bf16 path only)
    const int lsplit = c->dtype == MOE_DTYPE_F32 ? 0 : router_logit_splits(c->T, c->E, c->d);
    sz[B_LOGPART] = lsplit > 1 ? (size_t)lsplit * T * E * 4 : 0;
    const size_t hs = shared_hidden(c);
    sz[B_HS] = T * 2 * hs * s;
    sz[B_AS] = T * hs * s;
    sz[B_YS] = hs ? T * d * s : 0;
    sz[B_DHS] = T * 2 * hs * s;
    sz[B_DXS] = hs ? T * d * s : 0;
    sz[B_STAB] = hs ? kSharedTab * 4 : 0;
    size_t o = 0;
    for (int b = 0; b < B_COUNT; ++b) {
        L.off[b] = o;
        o += align256(sz[b] > 0 ? sz[b] : 1);
    }
    L.total = o;
    return L;
}


// Device pointers of one call.  Token-sized tensors (tok = true) may be NULL
// when T == 0, since they then hold no elements.
struct Ptrs {
    static constexpr int kMax = 64;
    const void* list[kMax];
    bool tok[kMax];
    int n = 0;
    bool overflow = false;
    bool misaligned_opt = false;
    void add(const void* p, bool t = false) {
        if (n == kMax) { overflow = true; return; }
        list[n] = p; tok[n] = t; ++n;
    }
    // an optional output: NULL skips it, otherwise it must be aligned like the rest
    void add_optional(const void* p) {
        if (p && !aligned16(p)) misaligned_opt = true;
    }
    int check(int T) const {
        if (overflow) return MOE_ERR_INVALID_ARG;
        if (misaligned_opt) return MOE_ERR_MISALIGNED;
        for (int i = 0; i < n; ++i) {
            if (!list[i]) {
                if (tok[i] && T == 0) continue;
                return MOE_ERR_NULL_PTR;
            }
            if (!aligned16(list[i])) return MOE_ERR_MISALIGNED;
        }
        return MOE_OK;
    }
};

int check_common(const moe_config* c, void* ws, size_t ws_bytes) {
    if (!shape_ok(c)) return MOE_ERR_INVALID_ARG;
    int st = supported(c);
    if (st != MOE_OK) return st;
    if (!ws || ws_bytes < layout(c).total) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_MISALIGNED;
    return MOE_OK;
}

void add_weights(Ptrs& P, const moe_config* c, const moe_weights* w) {
    P.add(w->Wg); P.add(w->W1); P.add(w->W2);
    if (c->expert == MOE_EXPERT_SWIGLU) P.add(w->W3);
    else { P.add(w->b1); P.add(w->b2); }
    if (c->n_shared > 0) { P.add(w->Ws1); P.add(w->Ws3); P.add(w->Ws2); }
}

void add_routing(Ptrs& P, const moe_routing* r, bool logits) {
    if (logits) P.add(r->logits, true);
    P.add(r->topk_idx, true); P.add(r->gates, true); P.add(r->counts); P.add(r->offsets);
    P.add(r->slot_of, true); P.add(r->token_of, true); P.add(r->aux);
    P.add_optional(r->src_k);
}

// experts = false: the expert weight gradients (dW1, dW2, dW3) are not stored.
void add_grads(Ptrs& P, const moe_config* c, const moe_grads* g, bool experts = true) {
    P.add(g->dX, true); P.add(g->dWg);
    if (experts) {
        P.add(g->dW1); P.add(g->dW2);
        if (c->expert == MOE_EXPERT_SWIGLU) P.add(g->dW3);
        if (c->n_shared > 0) { P.add(g->dWs1); P.add(g->dWs3); P.add(g->dWs2); }
    }
    if (c->expert != MOE_EXPERT_SWIGLU) { P.add(g->db1); P.add(g->db2); }
}

struct Ctx {
    const moe_config* c;
    char* ws;
    Layout L;
    hipStream_t s;
    void* const* ev = nullptr;    // optional stage events (moe_train_step_profiled)
    template <class T> T* buf(int b) const { return reinterpret_cast<T*>(ws + L.off[b]); }
    hipError_t mark(int stage) const {
        return ev ? hipEventRecord((hipEvent_t)ev[stage], s) : hipSuccess;
    }
};

#define TRY(x)                                   \
    do {                                         \
        hipError_t _e = (x);                     \
        if (_e != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

// Scratch of the routing kernels: per-chunk histograms, their scan bases, per-chunk aux
// partial sums, the GEMM tile prefixes, and (optionally) the gate of each expert-major row.
struct RouteScratch {
    int32_t* hist; int32_t* cbase; float* qpart; int32_t* tprefix; float* gate_of;
};

// Routing from logits: top-k, gates, histogram, scan, slots, aux.  Every scratch entry
// the kernels read was written earlier in the same sequence, so nothing needs clearing.
int run_routing(const moe_config* c, hipStream_t s, const RouteScratch& sc, const float* logits,
                const float* e_bias, moe_routing* r) {
    RouteArgs ra = {logits, r->topk_idx, r->gates, sc.hist, sc.qpart,
                    c->T, c->E, c->k, c->n_groups, c->topk_groups, c->score, nchunk(c),
                    e_bias, c->group_score, route_scale(c)};
    TRY(launch_route_topk(ra, s));
    ScanArgs sa = {sc.hist, sc.cbase, r->counts, nchunk(c)};
    TRY(launch_expert_scan(sa, c->E, s));
    SlotArgs sl = {r->counts, sc.cbase, r->topk_idx, r->gates, r->offsets, sc.tprefix,
                   r->slot_of, r->token_of, sc.gate_of, r->src_k, c->T, c->E, c->k, nchunk(c)};
    TRY(launch_slot_assign(sl, s));
    FinalizeArgs fa = {sc.qpart, r->counts, nullptr, 0, r->aux, nullptr, 0.f,
                       c->T, c->d, c->E, c->k, nchunk(c)};
    TRY(launch_finalize(fa, s));
    return MOE_OK;
}

int run_routing(const Ctx& x, const float* logits, const float* e_bias, moe_routing* r) {
    RouteScratch sc = {x.buf<int32_t>(B_HIST), x.buf<int32_t>(B_CBASE), x.buf<float>(B_QPART),
                       x.buf<int32_t>(B_TPREFIX), fused(x.c) ? x.buf<float>(B_GATEOF) : nullptr};
    return run_routing(x.c, x.s, sc, logits, e_bias, r);
}

// ---- routing with no workspace -------------------------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Bytes of scratch a routing call needs: histograms, scan bases and aux partials of every
// 64-token chunk, and the tile prefixes (each part 256-byte aligned).
size_t route_scratch_bytes(const moe_config* c, size_t* off) {
    const size_t ne = (size_t)c->E * (size_t)nchunk(c) * 4;
    const size_t sz[4] = {ne, ne, ne, (size_t)kTabs * 4};
    size_t o = 0;
    for (int i = 0; i < 4; ++i) {
        if (off) off[i] = o;
        o += align256(sz[i] > 0 ? sz[i] : 1);
    }
    return o;
}

// Device address of this GPU's scratch array, resolved on the first call on the device.
int scratch_ptr(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

ExpertGemmArgs expert_args(const Ctx& x, const moe_weights* w, const moe_routing* r) {
    const moe_config* c = x.c;
    ExpertGemmArgs a = {};
    a.T = c->T; a.d = c->d; a.E = c->E; a.ffn = c->ffn; a.k = c->k; a.rows = c->T * c->k;
    a.offsets = r->offsets;
    a.tile_prefix = x.buf<int32_t>(B_TPREFIX);
    a.queue = x.buf<int32_t>(B_QUEUE);
    a.Xp = x.buf<void>(B_XP);
    a.W1 = w->W1; a.W3 = w->W3; a.W2 = w->W2;
    a.b1 = c->expert == MOE_EXPERT_SWIGLU ? nullptr : w->b1;
    a.b2 = c->expert == MOE_EXPERT_SWIGLU ? nullptr : w->b2;
    a.H = x.buf<void>(B_H); a.A = x.buf<void>(B_A); a.EO = x.buf<void>(B_EO);
    a.dEO = x.buf<void>(B_DEO); a.dH = x.buf<void>(B_DH); a.dXp = x.buf<void>(B_DXP);
    a.expert = c->expert;
    return a;
}

// Fused dispatch: the expert contractions read X and dY through token_of, apply the gates
// themselves, and leave the gate gradient in per-tile partials.
void set_fused(const Ctx& x, ExpertGemmArgs& a, const void* X, const moe_routing* r, const void* dY) {
    a.token_of = r->token_of;
    a.gate_of = x.buf<float>(B_GATEOF);
    a.X = X;
    a.dY = dY;
    a.dgate_part = x.buf<float>(B_DGPART);
}

// The shared-experts branch as one expert segment of all T rows: the expert
// contractions run it with E = 1 and the token rows themselves in place of the
// gathered rows.  Its tables (offsets {0, T}, tile prefixes) are in B_STAB.
ExpertGemmArgs shared_args(const Ctx& x, const void* X, const moe_weights* w) {
    const moe_config* c = x.c;
    ExpertGemmArgs a = {};
    a.T = c->T; a.d = c->d; a.E = 1; a.ffn = shared_hidden(c); a.k = 1; a.rows = c->T;
    a.offsets = x.buf<int32_t>(B_STAB);
    a.tile_prefix = x.buf<int32_t>(B_STAB) + 2;
    a.queue = x.buf<int32_t>(B_QUEUE);
    a.Xp = X;
    a.W1 = w->Ws1; a.W3 = w->Ws3; a.W2 = w->Ws2;
    a.H = x.buf<void>(B_HS); a.A = x.buf<void>(B_AS); a.EO = x.buf<void>(B_YS);
    a.dH = x.buf<void>(B_DHS); a.dXp = x.buf<void>(B_DXS);
    a.expert = MOE_EXPERT_SWIGLU;
    return a;
}

int run_forward(const Ctx& x, const void* X, const moe_weights* w, void* Y, moe_routing* r,
                const void* Yt, float aux_coef, float* loss_out) {
    const moe_config* c = x.c;
    const bool f32 = c->dtype == MOE_DTYPE_F32;
    const int vec = c->d * esize(c) / 16;
    RouterGemmArgs rg = {c->T, c->d, c->E, X, w->Wg, nullptr, r->logits, nullptr, nullptr, nullptr,
                         !f32 && router_logit_splits(c->T, c->E, c->d) > 1 ? x.buf<float>(B_LOGPART) : nullptr};
    TRY(x.mark(MOE_STAGE_ROUTER_LOGITS));
    TRY(f32 ? simple_router_logits(rg, x.s) : mfma_router_logits(rg, x.s));
    TRY(x.mark(MOE_STAGE_ROUTE));
    int st = run_routing(x, r->logits, w->e_bias, r);
    if (st != MOE_OK) return st;
    TRY(x.mark(MOE_STAGE_GATHER));
    if (!fused(c)) {                // fused dispatch: the up projection reads X through token_of
        GatherArgs ga = {X, r->slot_of, x.buf<void>(B_XP), c->T, c->k, vec};
        TRY(launch_gather(ga, c->dtype, x.s));
    }
    ExpertGemmArgs ea = expert_args(x, w, r);
    if (fused(c)) set_fused(x, ea, X, r, nullptr);
    TRY(x.mark(MOE_STAGE_UP_FWD));
    TRY(f32 ? simple_up_fwd(ea, x.s) : (mfma_up_fwd_short(ea) ? mfma_up_fwd(ea, x.s) : kt64::mfma_up_fwd(ea, x.s)));
    TRY(x.mark(MOE_STAGE_DOWN_FWD));
    TRY(f32 ? simple_down_fwd(ea, x.s) : mfma_down_fwd(ea, x.s));
    TRY(x.mark(MOE_STAGE_SHARED_FWD));
    const bool shared = c->n_shared > 0;
    if (shared) {
        TRY(launch_shared_table(x.buf<int32_t>(B_STAB), c->T, x.s));
        ExpertGemmArgs sa = shared_args(x, X, w);
        TRY(f32 ? simple_up_fwd(sa, x.s) : kt64::mfma_up_fwd(sa, x.s));
        TRY(f32 ? simple_down_fwd(sa, x.s) : mfma_down_fwd(sa, x.s));
    }
    TRY(x.mark(MOE_STAGE_COMBINE_LOSS));
    CombineArgs ca = {x.buf<void>(B_EO), r->slot_of, fused(c) ? nullptr : r->gates, Y,
                      shared ? x.buf<void>(B_YS) : nullptr, Yt, x.buf<void>(B_DY),
                      x.buf<float>(B_LPART), c->T > 0 ? 2.0f / ((float)c->T * (float)c->d) : 0.f,
                      c->T, c->k, vec};
    TRY(launch_combine(ca, c->dtype, x.s));
    if (loss_out) {                 // the training step; Yt may be NULL only when T = 0
        FinalizeArgs fa = {x.buf<float>(B_QPART), r->counts, x.buf<float>(B_LPART),
                           combine_loss_blocks(c->T), nullptr, loss_out, aux_coef,
                           c->T, c->d, c->E, c->k, nchunk(c)};
        TRY(launch_finalize(fa, x.s));
    }
    return MOE_OK;
}

// sgd != NULL: the expert weight gradients are not stored; the weight-gradient
// contractions apply the SGD step (rate lr) to sgd's masters and working copies.
int run_backward(const Ctx& x, const void* X, const moe_weights* w, const moe_routing* r,
                 const void* dY, float aux_coef, moe_grads* g,
                 const moe_params* sgd = nullptr, float lr = 0.f) {
    const moe_config* c = x.c;
    const bool f32 = c->dtype == MOE_DTYPE_F32;
    const int vec = c->d * esize(c) / 16;
    TRY(x.mark(MOE_STAGE_COMBINE_BWD));
    if (!fused(c)) {                // fused dispatch: the down dgrad applies the gates itself
        CombineBwdArgs cb = {dY, x.buf<void>(B_EO), r->slot_of, r->gates, x.buf<float>(B_DGATE),
                             x.buf<void>(B_DEO), c->T, c->k, vec};
        TRY(launch_combine_bwd(cb, c->dtype, x.s));
    }
    ExpertGemmArgs ea = expert_args(x, w, r);
    if (fused(c)) set_fused(x, ea, X, r, dY);
    ea.dW1 = g->dW1; ea.dW2 = g->dW2; ea.dW3 = g->dW3;
    if (sgd) {
        const bool glu = c->expert == MOE_EXPERT_SWIGLU;
        ea.dW1 = ea.dW2 = ea.dW3 = nullptr;
        ea.W1m = sgd->W1; ea.W1w = sgd->W1_w;
        ea.W2m = sgd->W2; ea.W2w = sgd->W2_w;
        ea.W3m = glu ? sgd->W3 : nullptr; ea.W3w = glu ? sgd->W3_w : nullptr;
        ea.lr = lr;
    }
    TRY(x.mark(MOE_STAGE_DOWN_DGRAD));
    TRY(f32 ? simple_down_dgrad(ea, x.s) : mfma_down_dgrad(ea, x.s));
    TRY(x.mark(MOE_STAGE_DOWN_WGRAD));
    TRY(f32 ? simple_down_wgrad(ea, x.s) : mfma_down_wgrad(ea, x.s));
    TRY(x.mark(MOE_STAGE_UP_DGRAD));
    TRY(f32 ? simple_up_dgrad(ea, x.s) : mfma_up_dgrad(ea, x.s));
    TRY(x.mark(MOE_STAGE_UP_WGRAD));
    TRY(f32 ? simple_up_wgrad(ea, x.s) : mfma_up_wgrad(ea, x.s));
    TRY(x.mark(MOE_STAGE_SHARED_BWD));
    const bool shared = c->n_shared > 0;
    if (shared) {
        // its output enters Y with no gate: the upstream gradient is dY itself; each
        // dgrad reads a working copy before the wgrad that may update it
        ExpertGemmArgs sa = shared_args(x, X, w);
        sa.dEO = dY;
        sa.dW1 = g->dWs1; sa.dW3 = g->dWs3; sa.dW2 = g->dWs2;
        if (sgd) {
            sa.dW1 = sa.dW3 = sa.dW2 = nullptr;
            sa.W1m = sgd->Ws1; sa.W1w = sgd->Ws1_w;
            sa.W3m = sgd->Ws3; sa.W3w = sgd->Ws3_w;
            sa.W2m = sgd->Ws2; sa.W2w = sgd->Ws2_w;
            sa.lr = lr;
        }
        TRY(f32 ? simple_down_dgrad(sa, x.s) : mfma_down_dgrad(sa, x.s));
        TRY(f32 ? simple_down_wgrad(sa, x.s) : mfma_down_wgrad(sa, x.s));
        TRY(f32 ? simple_up_dgrad(sa, x.s) : mfma_up_dgrad(sa, x.s));
        TRY(f32 ? simple_up_wgrad(sa, x.s) : mfma_up_wgrad(sa, x.s));
    }
    TRY(x.mark(MOE_STAGE_BIAS_GRADS));
    if (c->expert != MOE_EXPERT_SWIGLU) {
        ColSumArgs b2 = {x.buf<void>(B_DEO), c->d, r->offsets, g->db2, c->d, c->E};
        TRY(launch_colsum(b2, c->dtype, x.s));
        ColSumArgs b1 = {x.buf<void>(B_DH), c->ffn, r->offsets, g->db1, c->ffn, c->E};
        TRY(launch_colsum(b1, c->dtype, x.s));
    }
    RouterBwdArgs rb = {r->logits, r->topk_idx, r->gates, fused(c) ? nullptr : x.buf<float>(B_DGATE),
                        x.buf<float>(B_DGPART), r->slot_of, dgate_parts(c), (long)c->T * c->k,
                        r->counts, x.buf<void>(B_DL), aux_coef, c->T, c->E, c->k, c->score,
                        route_scale(c)};
    TRY(x.mark(MOE_STAGE_ROUTER_BWD));
    TRY(launch_router_bwd(rb, c->dtype, x.s));
    const bool fused_scatter = scatter_in_router_dx(c);
    RouterGemmArgs rg = {c->T, c->d, c->E, X, w->Wg, x.buf<void>(B_DL), nullptr,
                         fused_scatter ? nullptr : x.buf<float>(B_DXR), g->dWg,
                         router_dwg_splits(c->T, c->E, c->d) > 1 ? x.buf<float>(B_DWGPART) : nullptr};
    TRY(x.mark(MOE_STAGE_ROUTER_DWG));
    TRY(f32 ? simple_router_dwg(rg, x.s) : mfma_router_dwg(rg, x.s));
    TRY(x.mark(MOE_STAGE_ROUTER_DX));
    ScatterArgs sa = {x.buf<void>(B_DXP), r->slot_of, fused_scatter ? nullptr : x.buf<float>(B_DXR), g->dX,
                      shared ? x.buf<void>(B_DXS) : nullptr, c->T, c->k, vec};
    if (fused_scatter) {
        // the scatter runs in the router dX contraction's epilogue (same sums, same order)
        TRY(mfma_router_dx_scatter(rg, sa, x.s));
        TRY(x.mark(MOE_STAGE_SCATTER));
        return MOE_OK;
    }
    TRY(f32 ? simple_router_dx(rg, x.s) : mfma_router_dx(rg, x.s));
    TRY(x.mark(MOE_STAGE_SCATTER));
    TRY(launch_scatter(sa, c->dtype, x.s));
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return 5; }

const char* moe_status_string(int st) {
    switch (st) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument: layer shape or config rule broken";
        case MOE_ERR_NULL_PTR: return "a required pointer is NULL";
        case MOE_ERR_MISALIGNED: return "a device pointer is not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "workspace missing or smaller than moe_workspace_bytes()";
        case MOE_ERR_UNSUPPORTED: return "shape outside what the gfx950 kernels support";
        case MOE_ERR_HIP: return "a HIP kernel launch failed";
        case MOE_ERR_SCRATCH: return "the call needs more scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

size_t moe_workspace_bytes(const moe_config* cfg) {
    if (!shape_ok(cfg)) return 0;
    return layout(cfg).total;
}

int64_t moe_workspace_offset(const moe_config* cfg, int32_t which) {
    if (!shape_ok(cfg)) return -1;
    Layout L = layout(cfg);
    switch (which) {
        case MOE_WS_XP: return fused(cfg) ? -1 : (int64_t)L.off[B_XP];
        case MOE_WS_H: return (int64_t)L.off[B_H];
        case MOE_WS_A: return (int64_t)L.off[B_A];
        case MOE_WS_EO: return (int64_t)L.off[B_EO];
        default: return -1;
    }
}

int moe_route(const moe_config* cfg, const float* logits, const float* e_bias, moe_routing* r,
              void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_common(cfg, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    if ((st = check_bias(cfg, e_bias)) != MOE_OK) return st;
    if (!r) return MOE_ERR_NULL_PTR;
    Ptrs P;
    P.add(logits, true);
    add_routing(P, r, false);
    if ((st = P.check(cfg->T)) != MOE_OK) return st;
    Ctx x{cfg, (char*)workspace, layout(cfg), (hipStream_t)stream};
    return run_routing(x, logits, e_bias, r);
}

int moe_route_noalloc(const moe_config* cfg, const float* logits, const float* e_bias,
                      moe_routing* r, void* stream) {
    if (!shape_ok(cfg)) return MOE_ERR_INVALID_ARG;
    int st = supported(cfg);
    if (st != MOE_OK) return st;
    if ((st = check_bias(cfg, e_bias)) != MOE_OK) return st;
    if (!r) return MOE_ERR_NULL_PTR;
    size_t off[4];
    if (route_scratch_bytes(cfg, off) > (size_t)MOE_ROUTE_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    Ptrs P;
    P.add(logits, true);
    add_routing(P, r, false);
    if ((st = P.check(cfg->T)) != MOE_OK) return st;
    void* base = nullptr;
    if ((st = scratch_ptr(&base)) != MOE_OK) return st;
    char* b = static_cast<char*>(base);
    RouteScratch sc = {reinterpret_cast<int32_t*>(b + off[0]), reinterpret_cast<int32_t*>(b + off[1]),
                       reinterpret_cast<float*>(b + off[2]), reinterpret_cast<int32_t*>(b + off[3]),
                       nullptr};
    return run_routing(cfg, (hipStream_t)stream, sc, logits, e_bias, r);
}

int moe_forward(const moe_config* cfg, const void* X, const moe_weights* w, void* Y,
                moe_routing* r, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_common(cfg, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    if (!w || !r) return MOE_ERR_NULL_PTR;
    if ((st = check_bias(cfg, w->e_bias)) != MOE_OK) return st;
    Ptrs P;
    P.add(X, true); P.add(Y, true);
    add_weights(P, cfg, w);
    add_routing(P, r, true);
    if ((st = P.check(cfg->T)) != MOE_OK) return st;
    Ctx x{cfg, (char*)workspace, layout(cfg), (hipStream_t)stream};
    return run_forward(x, X, w, Y, r, nullptr, 0.f, nullptr);
}

int moe_backward(const moe_config* cfg, const void* X, const moe_weights* w, const moe_routing* r,
                 const void* dY, float aux_coef, moe_grads* g, void* workspace,
                 size_t workspace_bytes, void* stream) {
    int st = check_common(cfg, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    if (!w || !r || !g) return MOE_ERR_NULL_PTR;
    Ptrs P;
    P.add(X, true); P.add(dY, true);
    add_weights(P, cfg, w);
    add_routing(P, r, true);
    add_grads(P, cfg, g);
    if ((st = P.check(cfg->T)) != MOE_OK) return st;
    Ctx x{cfg, (char*)workspace, layout(cfg), (hipStream_t)stream};
    return run_backward(x, X, w, r, dY, aux_coef, g);
}

static int train_step_impl(const moe_config* cfg, const void* X, const void* Y_target,
                           moe_params* p, float lr, float aux_coef, void* Y, moe_routing* r,
                           moe_grads* g, float* loss_out, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* events) {
    int st = check_common(cfg, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    if (!p || !r || !g) return MOE_ERR_NULL_PTR;
    if ((st = check_bias(cfg, p->e_bias)) != MOE_OK) return st;
    const bool glu = cfg->expert == MOE_EXPERT_SWIGLU;
    // expert weight gradients: all given (stored, then SGD over every parameter) or all
    // NULL (SGD fused into the weight-gradient contractions, nothing stored)
    const bool shared = cfg->n_shared > 0;
    const int n_null = !g->dW1 + !g->dW2 + (glu ? !g->dW3 : 0) +
                       (shared ? !g->dWs1 + !g->dWs3 + !g->dWs2 : 0);
    const bool fused = n_null == (glu ? 3 : 2) + (shared ? 3 : 0);
    if (n_null && !fused) return MOE_ERR_NULL_PTR;
    Ptrs P;
    P.add(X, true); P.add(Y_target, true); P.add(Y, true); P.add(loss_out);
    P.add(p->Wg); P.add(p->W1); P.add(p->W2); P.add(p->Wg_w); P.add(p->W1_w); P.add(p->W2_w);
    if (glu) { P.add(p->W3); P.add(p->W3_w); }
    else { P.add(p->b1); P.add(p->b2); P.add(p->b1_w); P.add(p->b2_w); }
    if (shared) {
        P.add(p->Ws1); P.add(p->Ws3); P.add(p->Ws2); P.add(p->Ws1_w); P.add(p->Ws3_w); P.add(p->Ws2_w);
    }
    add_routing(P, r, true);
    add_grads(P, cfg, g, !fused);
    if ((st = P.check(cfg->T)) != MOE_OK) return st;
    if (events) {
        for (int i = 0; i <= MOE_NUM_STAGES; ++i)
            if (!events[i]) return MOE_ERR_NULL_PTR;
    }
    Ctx x{cfg, (char*)workspace, layout(cfg), (hipStream_t)stream, events};
    moe_weights w = {p->Wg_w, p->W1_w, glu ? nullptr : p->b1_w, p->W2_w, glu ? nullptr : p->b2_w,
                     glu ? p->W3_w : nullptr, p->e_bias,
                     shared ? p->Ws1_w : nullptr, shared ? p->Ws3_w : nullptr, shared ? p->Ws2_w : nullptr};
    st = run_forward(x, X, &w, Y, r, Y_target, aux_coef, loss_out);
    if (st != MOE_OK) return st;
    st = run_backward(x, X, &w, r, x.buf<void>(B_DY), aux_coef, g, fused ? p : nullptr, lr);
    if (st != MOE_OK) return st;
    const long E = cfg->E, d = cfg->d, ffn = cfg->ffn;
    const long hs = shared_hidden(cfg);
    // (the expert and shared weights were already updated when the step is fused)
    struct { float* m; const float* g; void* w; long n; } upd[MOE_SGD_MAX_SEG] = {
        {p->Wg, g->dWg, p->Wg_w, E * d},
        {fused ? nullptr : p->W1, g->dW1, p->W1_w, E * ffn * d},
        {fused ? nullptr : p->W2, g->dW2, p->W2_w, E * d * ffn},
        {glu && !fused ? p->W3 : nullptr, g->dW3, p->W3_w, E * ffn * d},
        {glu ? nullptr : p->b1, g->db1, p->b1_w, E * ffn},
        {glu ? nullptr : p->b2, g->db2, p->b2_w, E * d},
        {shared && !fused ? p->Ws1 : nullptr, g->dWs1, p->Ws1_w, hs * d},
        {shared && !fused ? p->Ws3 : nullptr, g->dWs3, p->Ws3_w, hs * d},
        {shared && !fused ? p->Ws2 : nullptr, g->dWs2, p->Ws2_w, d * hs},
    };
    TRY(x.mark(MOE_STAGE_SGD));
    SgdArgs sa = {};
    sa.lr = lr;
    for (auto& u : upd) {
        if (!u.m || u.n == 0) continue;
        sa.seg[sa.nseg++] = SgdSeg{u.m, u.g, u.w, u.n};
    }
    TRY(launch_sgd(sa, cfg->dtype, x.s));
    TRY(x.mark(MOE_NUM_STAGES));
    return MOE_OK;
}

int moe_train_step(const moe_config* cfg, const void* X, const void* Y_target, moe_params* p,
                   float lr, float aux_coef, void* Y, moe_routing* r, moe_grads* g,
                   float* loss_out, void* workspace, size_t workspace_bytes, void* stream) {
    return train_step_impl(cfg, X, Y_target, p, lr, aux_coef, Y, r, g, loss_out, workspace,
                           workspace_bytes, stream, nullptr);
}

int moe_train_step_profiled(const moe_config* cfg, const void* X, const void* Y_target,
                            moe_params* p, float lr, float aux_coef, void* Y, moe_routing* r,
                            moe_grads* g, float* loss_out, void* workspace, size_t workspace_bytes,
                            void* stream, void* const* events) {
    if (!events) return MOE_ERR_NULL_PTR;
    return train_step_impl(cfg, X, Y_target, p, lr, aux_coef, Y, r, g, loss_out, workspace,
                           workspace_bytes, stream, events);
}

}  // extern "C"
