// Router scoring, group-limited top-k, gate renormalisation, dispatch tables,
// aux loss and the router backward, for gfx950.
//
// Sources: "Trainable MoE in CUDA" outline Part 2 (top-k and gate
// normalisation with its backward), Part 3 (router), Part 4 (counts, offsets,
// slots), Part 6 (aux loss); "AI Infra Kernel Lab" README, "Project status"
// (group-limited selection, ties to the smaller group/expert id).
//
// Layout: one 64-lane wavefront owns one token at a time; lane j holds the
// logits of experts j, j+64, j+128, j+192.  A workgroup of sixteen
// wavefronts (four tokens each) owns a chunk of 64 consecutive tokens, which
// is the unit of the histogram and of the stable slot ranking.  No floating-point atomics anywhere; the
// integer LDS histogram is order-independent and every float sum runs in a
// fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int CHUNK = 64;       // tokens per histogram chunk
constexpr int RT_WAVES = 16;    // wavefronts per routing workgroup (4 tokens each)
constexpr int EPL = MOE_MAX_EXPERTS / 64;  // expert values held per lane

// a beats b in the selection order (-value, id): larger value, then smaller id.
__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
    return (va > vb) || (va == vb && ia < ib);
}

// Wave reductions on DPP row moves: the quad swaps (lane ^ 1, lane ^ 2), then the
// half-row and row mirrors, leave every lane of each 16-lane row holding the row's
// result (each step combines two disjoint halves, and the two lanes of a pair get
// the same value since max and + are commutative).  The four row results are then
// read as scalars and combined in a fixed order, so every lane gets the same,
// deterministic value.  No LDS round trips, unlike a butterfly of ds_bpermute.
constexpr int DPP_QXOR1 = 0xB1, DPP_QXOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
template <int C> __device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, C, 0xF, 0xF, false);
}
template <int C> __device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<C>(__float_as_int(v)));
}
__device__ __forceinline__ float lane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wv_sum(float v) {
    v += dpp_f<DPP_QXOR1>(v);
    v += dpp_f<DPP_QXOR2>(v);
    v += dpp_f<DPP_HALF_MIRROR>(v);
    v += dpp_f<DPP_MIRROR>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wv_max(float v) {
    v = fmaxf(v, dpp_f<DPP_QXOR1>(v));
    v = fmaxf(v, dpp_f<DPP_QXOR2>(v));
    v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
    v = fmaxf(v, dpp_f<DPP_MIRROR>(v));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
template <int C> __device__ __forceinline__ void argmax_step(float& v, int& i) {
    const float vo = dpp_f<C>(v);
    const int io = dpp_i<C>(i);
    if (beats(vo, io, v, i)) { v = vo; i = io; }
}
// Wave-wide arg-max under (-value, id); every lane gets the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_step<DPP_QXOR1>(v, i);
    argmax_step<DPP_QXOR2>(v, i);
    argmax_step<DPP_HALF_MIRROR>(v, i);
    argmax_step<DPP_MIRROR>(v, i);
    float bv = lane_f(v, 0);
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float rv = lane_f(v, 16 * r);
        const int ri = __builtin_amdgcn_readlane(i, 16 * r);
        if (beats(rv, ri, bv, bi)) { bv = rv; bi = ri; }
    }
    v = bv; i = bi;
}

struct TokenScores {
    float l[EPL];     // logits
    float s[EPL];     // softmax p, or sigmoid s
    float q[EPL];     // aux probabilities
    float mx, z;      // softmax max and denominator; sigmoid: z = sum of s
};

__device__ __forceinline__ void load_logits(const float* __restrict__ lrow, int E, float (&l)[EPL]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
        int e = lane + 64 * m;
        l[m] = (e < E) ? lrow[e] : -INFINITY;
    }
}

__device__ __forceinline__ void score_token(const float (&l)[EPL], int E, int score, TokenScores& ts) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int m = 0; m < EPL; ++m) ts.l[m] = l[m];
    if (score == MOE_SCORE_SOFTMAX) {
        float mx = -INFINITY;
#pragma unroll
        for (int m = 0; m < EPL; ++m) mx = fmaxf(mx, ts.l[m]);
        mx = wv_max(mx);
        float z = 0.f;
#pragma unroll
        for (int m = 0; m < EPL; ++m) {
            int e = lane + 64 * m;
            ts.s[m] = (e < E) ? expf(ts.l[m] - mx) : 0.f;
            z += ts.s[m];
        }
        z = wv_sum(z);
        float inv = 1.0f / z;
#pragma unroll
        for (int m = 0; m < EPL; ++m) { ts.s[m] *= inv; ts.q[m] = ts.s[m]; }
        ts.mx = mx; ts.z = z;
    } else {
        float z = 0.f;
#pragma unroll
        for (int m = 0; m < EPL; ++m) {
            int e = lane + 64 * m;
            ts.s[m] = (e < E) ? 1.0f / (1.0f + expf(-ts.l[m])) : 0.f;
            z += ts.s[m];
        }
        z = wv_sum(z);
        float inv = 1.0f / z;
#pragma unroll
        for (int m = 0; m < EPL; ++m) ts.q[m] = ts.s[m] * inv;
        ts.mx = 0.f; ts.z = z;
    }
}

// Wave-wide float64 sum: the same DPP row moves on the two 32-bit halves, then the four row
// results in a fixed order.
template <int C> __device__ __forceinline__ double dpp_d(double v) {
    const long long b = __builtin_bit_cast(long long, v);
    const int lo = dpp_i<C>((int)(b & 0xffffffffll)), hi = dpp_i<C>((int)(b >> 32));
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ double lane_d(double v, int l) {
    const long long b = __builtin_bit_cast(long long, v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), l);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ double wv_sum_d(double v) {
    v += dpp_d<DPP_QXOR1>(v);
    v += dpp_d<DPP_QXOR2>(v);
    v += dpp_d<DPP_HALF_MIRROR>(v);
    v += dpp_d<DPP_MIRROR>(v);
    return (lane_d(v, 0) + lane_d(v, 16)) + (lane_d(v, 32) + lane_d(v, 48));
}

// Selection scores of the router variants: each score evaluated in float64 and rounded
// once to fp32, so that it is the fp32 rounding of the score up to the last bit of the
// float64 exponential (the "Numerical contracts" gate ranks scores plus the bias).  The
// fp32 max of the logits is exact, and so is the float64 difference l - max.
__device__ __forceinline__ void selection_scores(const float (&l)[EPL], int E, int score, float mx,
                                                 float (&v)[EPL]) {
    const int lane = threadIdx.x & 63;
    if (score == MOE_SCORE_SOFTMAX) {
        double z[EPL], zs = 0.0;
#pragma unroll
        for (int m = 0; m < EPL; ++m) {
            const int e = lane + 64 * m;
            z[m] = (e < E) ? exp((double)l[m] - (double)mx) : 0.0;
            zs += z[m];
        }
        zs = wv_sum_d(zs);
#pragma unroll
        for (int m = 0; m < EPL; ++m) v[m] = (float)(z[m] / zs);
    } else {
#pragma unroll
        for (int m = 0; m < EPL; ++m) v[m] = (float)(1.0 / (1.0 + exp(-(double)l[m])));
    }
}

// Score of expert e (owned by some lane) without a shuffle: recompute from its logit.
__device__ __forceinline__ float selected_score(float l, const TokenScores& ts, int score) {
    if (score == MOE_SCORE_SOFTMAX) return expf(l - ts.mx) / ts.z;
    return 1.0f / (1.0f + expf(-l));
}

// Selection ranks the logits (exact) for the plain gate, or the fp32 scores plus
// the correction bias when a bias or the top-2-sum group score is in use.
__global__ void __launch_bounds__(64 * RT_WAVES)
route_topk_kernel(RouteArgs a) {
    __shared__ int s_hist[MOE_MAX_EXPERTS];
    __shared__ float s_q[RT_WAVES][MOE_MAX_EXPERTS];
    __shared__ float s_l[RT_WAVES][MOE_MAX_EXPERTS];   // logits (for the unbiased gates)
    __shared__ float s_v[RT_WAVES][MOE_MAX_EXPERTS];   // selection values
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, k = a.k, G = a.n_groups;
    const int chunk = blockIdx.x;
    for (int e = tid; e < E; e += blockDim.x) s_hist[e] = 0;
    __syncthreads();

    float qacc[EPL];
#pragma unroll
    for (int m = 0; m < EPL; ++m) qacc[m] = 0.f;

    const int gsize = E / G;
    constexpr int TPW = CHUNK / RT_WAVES;           // tokens per wavefront
    const int t0 = chunk * CHUNK + wave * TPW;
    float lnext[EPL];                               // the next token's logits, in flight
    if (t0 < a.T) load_logits(a.logits + (size_t)t0 * E, E, lnext);
    for (int it = 0; it < TPW; ++it) {
        const int t = t0 + it;
        if (t >= a.T) break;                        // wave-uniform
        float lcur[EPL];
#pragma unroll
        for (int m = 0; m < EPL; ++m) lcur[m] = lnext[m];
        if (it + 1 < TPW && t + 1 < a.T) load_logits(a.logits + (size_t)(t + 1) * E, E, lnext);
        TokenScores ts;
        score_token(lcur, E, a.score, ts);
#pragma unroll
        for (int m = 0; m < EPL; ++m) qacc[m] += ts.q[m];

        // selection values
        const bool on_scores = a.bias != nullptr || a.group_score == MOE_GROUP_TOP2_SUM;
        float v[EPL];
        if (on_scores) selection_scores(ts.l, E, a.score, ts.mx, v);   // wave-uniform
#pragma unroll
        for (int m = 0; m < EPL; ++m) {
            int e = lane + 64 * m;
            if (!on_scores) v[m] = ts.l[m];
            else v[m] = (e < E) ? v[m] + (a.bias ? a.bias[e] : 0.f) : -INFINITY;
            if (e < E) { s_l[wave][e] = ts.l[m]; s_v[wave][e] = v[m]; }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // group limit: keep topk_groups groups by (-group score, group id); the
        // group score is the largest member value, or the sum of the two largest
        uint64_t kept_lo = ~0ull, kept_hi = ~0ull;   // bit per group (G <= 128 supported)
        if (G > 1) {
            const bool top2 = a.group_score == MOE_GROUP_TOP2_SUM;
            float gv[2] = {-INFINITY, -INFINITY};    // lanes own groups lane, lane+64
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int g = lane + 64 * h;
                if (g < G) {
                    float b1 = -INFINITY, b2 = -INFINITY;
                    const float* gvals = &s_v[wave][g * gsize];
                    int j = 0;
                    for (; j + 8 <= gsize; j += 8) {        // eight LDS reads in flight
                        float x[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) x[u] = gvals[j + u];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            if (x[u] > b1) { b2 = b1; b1 = x[u]; } else if (x[u] > b2) b2 = x[u];
                        }
                    }
                    for (; j < gsize; ++j) {
                        const float x = gvals[j];
                        if (x > b1) { b2 = b1; b1 = x; } else if (x > b2) b2 = x;
                    }
                    gv[h] = top2 ? b1 + b2 : b1;
                }
            }
            const float gv0 = gv[0], gv1 = gv[1];
            kept_lo = kept_hi = 0;
            bool t0 = lane >= G, t1 = lane + 64 >= G;  // taken / absent
            for (int r = 0; r < a.topk_groups; ++r) {
                float bv = -INFINITY; int bi = 0x7fffffff;
                if (!t0 && beats(gv0, lane, bv, bi)) { bv = gv0; bi = lane; }
                if (!t1 && beats(gv1, lane + 64, bv, bi)) { bv = gv1; bi = lane + 64; }
                wave_argmax(bv, bi);
                if (bi < 64) kept_lo |= 1ull << bi; else kept_hi |= 1ull << (bi - 64);
                if (bi == lane) t0 = true;
                if (bi == lane + 64) t1 = true;
            }
        }

        // top-k over eligible experts by (-value, id)
        bool taken[EPL];
#pragma unroll
        for (int m = 0; m < EPL; ++m) {
            int e = lane + 64 * m;
            bool elig = e < E;
            if (G > 1 && elig) {
                int g = e / gsize;
                elig = (g < 64) ? ((kept_lo >> g) & 1) : ((kept_hi >> (g - 64)) & 1);
            }
            taken[m] = !elig;
        }
        int sel_e = -1;      // lane i < k keeps the i-th pick
        for (int i = 0; i < k; ++i) {
            float bv = -INFINITY; int bi = 0x7fffffff;
#pragma unroll
            for (int m = 0; m < EPL; ++m) {
                int e = lane + 64 * m;
                if (!taken[m] && beats(v[m], e, bv, bi)) { bv = v[m]; bi = e; }
            }
            wave_argmax(bv, bi);
#pragma unroll
            for (int m = 0; m < EPL; ++m)
                if (bi == lane + 64 * m) taken[m] = true;
            if (lane == i) sel_e = bi;
        }
        // finite logits always leave k eligible experts; keep indices in range even
        // for malformed (NaN) input so that no later kernel indexes out of bounds
        if (lane < k && (sel_e < 0 || sel_e >= E)) sel_e = 0;
        // gates from the unbiased score of each pick
        float w = (lane < k) ? selected_score(s_l[wave][sel_e], ts, a.score) : 0.f;
        float S = wv_sum(w);
        if (lane < k) {
            a.topk_idx[(size_t)t * k + lane] = sel_e;
            a.gates[(size_t)t * k + lane] = (w / S) * a.route_scale;
            atomicAdd(&s_hist[sel_e], 1);
        }
        // s_l / s_v are rewritten for the next token only after every lane has read them
        __builtin_amdgcn_wave_barrier();
    }

    // aux partial sums: waves' running sums (token order) added in wave order
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
        int e = lane + 64 * m;
        if (e < E) s_q[wave][e] = qacc[m];
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
        float v = 0.f;
        for (int w = 0; w < RT_WAVES; ++w) v += s_q[w][e];
        a.qpart[(size_t)chunk * E + e] = v;
        a.hist[(size_t)e * a.nchunk + chunk] = s_hist[e];
    }
}

// One workgroup per expert: exclusive scan of its per-chunk counts.
__global__ void __launch_bounds__(256)
expert_scan_kernel(ScanArgs a) {
    __shared__ int s_wave[4];
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int* h = a.hist + (size_t)e * a.nchunk;
    int* cb = a.cbase + (size_t)e * a.nchunk;
    int running = 0;
    for (int base = 0; base < a.nchunk; base += 256) {
        int c = base + tid;
        int v = (c < a.nchunk) ? h[c] : 0;
        int inc = wave_incl_scan(v);
        if (lane == 63) s_wave[wave] = inc;
        __syncthreads();
        int before = running;
        for (int w = 0; w < wave; ++w) before += s_wave[w];
        if (c < a.nchunk) cb[c] = before + inc - v;
        int tot = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
        __syncthreads();
        running += tot;
    }
    if (tid == 0) a.counts[e] = running;
}

// One wavefront per chunk of 64 tokens: stable slots in ascending token order.
// The rank of a pick within the chunk is the number of earlier tokens (lanes) of
// the chunk that picked the same expert: a 64-bit mask of picking lanes is built
// per expert with integer LDS ORs (order-independent), and the rank is the
// popcount of that mask below the lane.  A token never picks an expert twice.
__global__ void __launch_bounds__(64)
slot_assign_kernel(SlotArgs a) {
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ unsigned long long s_mask[MOE_MAX_EXPERTS];
    const int lane = threadIdx.x, chunk = blockIdx.x, E = a.E, k = a.k;
    const int t = chunk * CHUNK + lane;
    const bool valid = t < a.T;
    int ex[MOE_MAX_K];
#pragma unroll
    for (int i = 0; i < MOE_MAX_K; ++i) ex[i] = (valid && i < k) ? a.topk_idx[(size_t)t * k + i] : -1;
    // offsets = exclusive scan of counts (lane owns experts 4*lane .. 4*lane+3)
    int c4[4], loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int e = lane * 4 + j;
        c4[j] = (e < E) ? a.counts[e] : 0;
        loc += c4[j];
    }
    int incl = wave_incl_scan(loc);
    int run = incl - loc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int e = lane * 4 + j;
        if (e < E) s_off[e] = run;
        run += c4[j];
    }
    if (lane == 63) s_off[E] = incl;
#pragma unroll
    for (int i = 0; i < MOE_MAX_K; ++i)
        if (ex[i] >= 0) s_mask[ex[i]] = 0ull;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MOE_MAX_K; ++i)
        if (ex[i] >= 0) atomicOr(&s_mask[ex[i]], 1ull << lane);
    if (chunk == 0) {
        for (int e = lane; e <= E; e += 64) a.offsets[e] = s_off[e];
        // m-tile prefix of every supported tile height (64, 128, 256 rows)
        for (int b = 0; b < 3; ++b) {
            const int bm = 64 << b;
            int tl = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) tl += (c4[j] + bm - 1) / bm;
            int ti = wave_incl_scan(tl);
            int tr = ti - tl;
            int* tp = a.tile_prefix + b * (MOE_MAX_EXPERTS + 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int e = lane * 4 + j;
                if (e < E) tp[e] = tr;
                tr += (c4[j] + bm - 1) / bm;
            }
            if (lane == 63) tp[E] = ti;
        }
        // the experts by rows, most first (ties: smaller id first): the order in which the
        // persistent weight-gradient contractions hand out their tiles
        __shared__ int s_cnt[MOE_MAX_EXPERTS];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (lane * 4 + j < E) s_cnt[lane * 4 + j] = c4[j];
        __syncthreads();
        int rank[4] = {0, 0, 0, 0};
        for (int f = 0; f < E; ++f) {
            const int cf = s_cnt[f];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane * 4 + j;
                rank[j] += (cf > c4[j] || (cf == c4[j] && f < e)) ? 1 : 0;
            }
        }
        int* order = a.tile_prefix + 3 * (MOE_MAX_EXPERTS + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (lane * 4 + j < E) order[rank[j]] = lane * 4 + j;
    }
    __syncthreads();
    if (!valid) return;
    const unsigned long long below = (1ull << lane) - 1ull;
    int base[MOE_MAX_K];
    float gt[MOE_MAX_K];
#pragma unroll
    for (int i = 0; i < MOE_MAX_K; ++i) {
        base[i] = (i < k) ? a.cbase[(size_t)ex[i] * a.nchunk + chunk] : 0;
        gt[i] = (i < k) ? a.gates[(size_t)t * k + i] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < MOE_MAX_K; ++i) {
        if (i < k) {
            const int e = ex[i];
            const int slot = s_off[e] + base[i] + __popcll(s_mask[e] & below);
            a.slot_of[(size_t)t * k + i] = slot;
            a.token_of[slot] = t;
            if (a.gate_of) a.gate_of[slot] = gt[i];
            if (a.src_k) a.src_k[slot] = i;
        }
    }
}

// Single workgroup: P_e, f_e, aux and (optionally) the MSE from partial sums.  The
// 1024 threads split the chunk partials of each expert into nslice = 1024 / E
// interleaved slices (several loads in flight per thread); slices, then experts,
// then the MSE partials are added in a fixed order, so the result is deterministic.
constexpr int FIN_THREADS = 1024;
__global__ void __launch_bounds__(FIN_THREADS)
finalize_kernel(FinalizeArgs a) {
    __shared__ float s_red[FIN_THREADS];
    const int tid = threadIdx.x;
    const int E = a.E;
    const int nslice = FIN_THREADS / E;                // E <= MOE_MAX_EXPERTS <= 1024
    float q = 0.f;
    if (a.T > 0 && tid < E * nslice) {
        const int e = tid % E, sl = tid / E;
        int c = sl;
        for (; c + 3 * nslice < a.nchunk; c += 4 * nslice) {
            const float v0 = a.qpart[(size_t)c * E + e], v1 = a.qpart[(size_t)(c + nslice) * E + e];
            const float v2 = a.qpart[(size_t)(c + 2 * nslice) * E + e], v3 = a.qpart[(size_t)(c + 3 * nslice) * E + e];
            q += v0; q += v1; q += v2; q += v3;
        }
        for (; c < a.nchunk; c += nslice) q += a.qpart[(size_t)c * E + e];
    }
    s_red[tid] = q;
    __syncthreads();
    float part = 0.f;                                  // f_e P_e of expert tid
    if (a.T > 0 && tid < E) {
        float P = 0.f;
        for (int sl = 0; sl < nslice; ++sl) P += s_red[sl * E + tid];
        P /= (float)a.T;
        const float f = (float)a.counts[tid] / ((float)a.T * (float)a.k);
        part = f * P;
    }
    __syncthreads();
    s_red[tid] = part;
    __syncthreads();
    for (int st = FIN_THREADS / 2; st >= 1; st >>= 1) {
        if (tid < st) s_red[tid] += s_red[tid + st];
        __syncthreads();
    }
    const float aux = (float)E * s_red[0];
    __syncthreads();
    float mse = 0.f;
    if (a.lpart != nullptr) {
        float v = 0.f;
        for (int b = tid; b < a.nlpart; b += FIN_THREADS) v += a.lpart[b];
        s_red[tid] = v;
        __syncthreads();
        for (int st = FIN_THREADS / 2; st >= 1; st >>= 1) {
            if (tid < st) s_red[tid] += s_red[tid + st];
            __syncthreads();
        }
        const double n = (double)a.T * (double)a.d;
        mse = (n > 0) ? (float)((double)s_red[0] / n) : 0.f;
    }
    if (tid == 0) {
        if (a.aux_out) a.aux_out[0] = aux;
        if (a.loss_out) {
            a.loss_out[0] = mse;
            a.loss_out[1] = aux;
            a.loss_out[2] = mse + a.aux_coef * aux;
        }
    }
}

// Router backward: renormalisation, aux gradient and score Jacobian -> dlogits.
template <class TD>
__global__ void __launch_bounds__(256)
router_bwd_kernel(RouterBwdArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= a.T) return;
    const int E = a.E, k = a.k;
    TokenScores ts;
    {
        float l[EPL];
        load_logits(a.logits + (size_t)t * E, E, l);
        score_token(l, E, a.score, ts);
    }
    int e_i = -1;
    float g_i = 0.f, dg_i = 0.f, w_i = 0.f;
    if (lane < k) {
        e_i = a.topk_idx[(size_t)t * k + lane];
        g_i = a.gates[(size_t)t * k + lane];
        if (a.dgate) {
            dg_i = a.dgate[(size_t)t * k + lane];
        } else {            // the row's partial sums over the down-projection column tiles, in order
            const long p = a.slot_of[(size_t)t * k + lane];
            for (int j = 0; j < a.nparts; ++j) dg_i += a.dgate_part[(long)j * a.part_ld + p];
        }
        w_i = selected_score(a.logits[(size_t)t * E + e_i], ts, a.score);
    }
    const float S = wv_sum(w_i);
    const float gdg = wv_sum(g_i * dg_i);
    // g = c w / S: dL/dw_i = (c dg_i - sum_j g_j dg_j) / S
    const float dw_i = (lane < k) ? (a.route_scale * dg_i - gdg) / S : 0.f;
    // aux gradient: dq_te = aux_coef * E * f_e / T, f_e = counts_e / (T k)
    const float c0 = a.aux_coef * (float)E / ((float)a.T * (float)a.T * (float)k);
    float sel[EPL], dq[EPL];
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
        int e = lane + 64 * m;
        sel[m] = 0.f;
        dq[m] = (e < E) ? c0 * (float)a.counts[e] : 0.f;
    }
    for (int i = 0; i < k; ++i) {
        int ei = __builtin_amdgcn_readlane(e_i, i);
        float dwi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dw_i), i));
#pragma unroll
        for (int m = 0; m < EPL; ++m)
            if (ei == lane + 64 * m) sel[m] += dwi;
    }
    float out[EPL];
    if (a.score == MOE_SCORE_SOFTMAX) {
        float dot = 0.f;
#pragma unroll
        for (int m = 0; m < EPL; ++m) dot += (dq[m] + sel[m]) * ts.s[m];
        dot = wv_sum(dot);
#pragma unroll
        for (int m = 0; m < EPL; ++m) out[m] = ts.s[m] * (dq[m] + sel[m] - dot);
    } else {
        float dot = 0.f;
#pragma unroll
        for (int m = 0; m < EPL; ++m) dot += dq[m] * ts.q[m];
        dot = wv_sum(dot);
        const float invZ = 1.0f / ts.z;
#pragma unroll
        for (int m = 0; m < EPL; ++m) {
            float ds = sel[m] + (dq[m] - dot) * invZ;
            out[m] = ds * ts.s[m] * (1.0f - ts.s[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
        int e = lane + 64 * m;
        if (e < E) reinterpret_cast<TD*>(a.dlogits)[(size_t)t * E + e] = from_f<TD>(out[m]);
    }
}

// ---- host launchers ------------------------------------------------------------
hipError_t launch_route_topk(const RouteArgs& a, hipStream_t s) {
    if (a.nchunk == 0) return hipSuccess;
    hipLaunchKernelGGL(route_topk_kernel, dim3(a.nchunk), dim3(64 * RT_WAVES), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_expert_scan(const ScanArgs& a, int E, hipStream_t s) {
    hipLaunchKernelGGL(expert_scan_kernel, dim3(E), dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_slot_assign(const SlotArgs& a, hipStream_t s) {
    // one workgroup at least, so that offsets and tile prefixes are written for T == 0
    int grid = a.nchunk > 0 ? a.nchunk : 1;
    hipLaunchKernelGGL(slot_assign_kernel, dim3(grid), dim3(64), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(FIN_THREADS), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_router_bwd(const RouterBwdArgs& a, int dtype, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    dim3 grid((a.T + 3) / 4);
    if (dtype == MOE_DTYPE_F32)
        hipLaunchKernelGGL(router_bwd_kernel<float>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(router_bwd_kernel<bf16>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
