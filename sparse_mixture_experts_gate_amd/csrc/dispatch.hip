// Token-major data movement of the sparse MoE layer for gfx950: gather into
// expert-major rows, gate-weighted combine (with the MSE fused in), combine
// backward, scatter of row gradients back to tokens, per-expert bias
// reductions and the SGD update.
//
// Sources: "Trainable MoE in CUDA" outline Part 4 (gather, scatter, weighted
// combine and its backward), Part 5 (bias gradients), Part 7 (MSE, SGD).
//
// Every kernel is HBM-bound.  One 64-lane wavefront owns one token and walks
// its row in 16-byte vectors, so each row is read once and written with
// coalesced 16-byte stores; the k expert-major rows of a token are visited
// in the token's top-k order.  Sums run in a fixed order and there are no
// atomics, so results are bitwise reproducible.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int TOK_WAVES = 4;    // tokens per 256-thread workgroup

// 16-byte loads of rows that a kernel reads once (the expert rows of a token, its
// targets, the router-path gradient) carry the nontemporal hint: a plain read stream
// measured 5.8 TB/s without it and 6.3 TB/s with it on one MI355X.
typedef unsigned int vu4 __attribute__((ext_vector_type(4)));
typedef float vf4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_once(const uint4* p) {
    const vu4 v = __builtin_nontemporal_load(reinterpret_cast<const vu4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ld_once(const float4* p) {
    const vf4 v = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void load_slots(const int32_t* slot_of, int t, int k, int* sl) {
#pragma unroll
    for (int i = 0; i < MOE_MAX_K; ++i) sl[i] = (i < k) ? slot_of[(size_t)t * k + i] : 0;
}

// KT > 0: k known at compile time, so the loops over the k expert rows unroll and
// all k loads of a vector are in flight together; KT == 0: any k.
template <class T, int KT>
__global__ void __launch_bounds__(256) gather_kernel(GatherArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * TOK_WAVES + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const int k = KT > 0 ? KT : a.k;
        int sl[MOE_MAX_K];
    load_slots(a.slot_of, t, k, sl);
    const uint4* src = reinterpret_cast<const uint4*>(a.X) + (size_t)t * a.vec;
    uint4* dst = reinterpret_cast<uint4*>(a.Xp);
    for (int v = lane; v < a.vec; v += 64) {
        uint4 x = ld_once(src + v);
#pragma unroll
        for (int i = 0; i < MOE_MAX_K; ++i) {
            if (i >= k) break;
            dst[(size_t)sl[i] * a.vec + v] = x;
        }
    }
}

template <class T, bool LOSS, int KT>
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
    __shared__ float s_part[TOK_WAVES];
    constexpr int N = Vec16<T>::N;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * TOK_WAVES + wave;
    float sq = 0.f;
    if (t < a.T) {
        const int k = KT > 0 ? KT : a.k;
        int sl[MOE_MAX_K];
        float g[MOE_MAX_K];
        load_slots(a.slot_of, t, k, sl);
#pragma unroll
        for (int i = 0; i < MOE_MAX_K; ++i)     // gates NULL: EO rows come gate-weighted already
            g[i] = (i < k) ? (a.gates ? a.gates[(size_t)t * k + i] : 1.f) : 0.f;
        const uint4* eo = reinterpret_cast<const uint4*>(a.EO);
        for (int v = lane; v < a.vec; v += 64) {
            float acc[N];
#pragma unroll
            for (int j = 0; j < N; ++j) acc[j] = 0.f;
#pragma unroll
            for (int i = 0; i < MOE_MAX_K; ++i) {
                if (i >= k) break;
                float x[N];
                Vec16<T>::unpack(ld_once(eo + (size_t)sl[i] * a.vec + v), x);
#pragma unroll
                for (int j = 0; j < N; ++j) acc[j] = fmaf(g[i], x[j], acc[j]);
            }
            const size_t o = (size_t)t * a.vec + v;
            if (a.Ys) {                    // shared branch: added with no gate
                float ys[N];
                Vec16<T>::unpack(ld_once(reinterpret_cast<const uint4*>(a.Ys) + o), ys);
#pragma unroll
                for (int j = 0; j < N; ++j) acc[j] += ys[j];
            }
            reinterpret_cast<uint4*>(a.Y)[o] = Vec16<T>::pack(acc);
            if (LOSS) {
                float yt[N], dy[N];
                Vec16<T>::unpack(ld_once(reinterpret_cast<const uint4*>(a.Yt) + o), yt);
#pragma unroll
                for (int j = 0; j < N; ++j) {
                    float r = acc[j] - yt[j];
                    sq = fmaf(r, r, sq);
                    dy[j] = r * a.inv_n2;
                }
                reinterpret_cast<uint4*>(a.dY)[o] = Vec16<T>::pack(dy);
            }
        }
    }
    if (LOSS) {
        sq = wave_sum(sq);
        if (lane == 0) s_part[wave] = sq;
        __syncthreads();
        if (threadIdx.x == 0) {
            float s = 0.f;
            for (int w = 0; w < TOK_WAVES; ++w) s += s_part[w];
            a.lpart[blockIdx.x] = s;
        }
    }
}

template <class T, int KT>
__global__ void __launch_bounds__(256) combine_bwd_kernel(CombineBwdArgs a) {
    constexpr int N = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * TOK_WAVES + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const int k = KT > 0 ? KT : a.k;
        int sl[MOE_MAX_K];
    float g[MOE_MAX_K], dg[MOE_MAX_K];
    load_slots(a.slot_of, t, k, sl);
#pragma unroll
    for (int i = 0; i < MOE_MAX_K; ++i) {
        g[i] = (i < k) ? a.gates[(size_t)t * k + i] : 0.f;
        dg[i] = 0.f;
    }
    const uint4* dy4 = reinterpret_cast<const uint4*>(a.dY) + (size_t)t * a.vec;
    const uint4* eo = reinterpret_cast<const uint4*>(a.EO);
    uint4* deo = reinterpret_cast<uint4*>(a.dEO);
    for (int v = lane; v < a.vec; v += 64) {
        float dy[N];
        Vec16<T>::unpack(ld_once(dy4 + v), dy);
#pragma unroll
        for (int i = 0; i < MOE_MAX_K; ++i) {
            if (i >= k) break;
            float x[N], o[N];
            const size_t r = (size_t)sl[i] * a.vec + v;
            Vec16<T>::unpack(ld_once(eo + r), x);
#pragma unroll
            for (int j = 0; j < N; ++j) {
                dg[i] = fmaf(dy[j], x[j], dg[i]);
                o[j] = g[i] * dy[j];
            }
            deo[r] = Vec16<T>::pack(o);
        }
    }
#pragma unroll
    for (int i = 0; i < MOE_MAX_K; ++i) {
        if (i >= k) break;
        float s = wave_sum(dg[i]);
        if (lane == 0) a.dgate[(size_t)t * k + i] = s;
    }
}

template <class T, int KT>
__global__ void __launch_bounds__(256) scatter_kernel(ScatterArgs a) {
    constexpr int N = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * TOK_WAVES + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const int k = KT > 0 ? KT : a.k;
        int sl[MOE_MAX_K];
    load_slots(a.slot_of, t, k, sl);
    const uint4* dxp = reinterpret_cast<const uint4*>(a.dXp);
    // router-path gradient is fp32 [T, d]: N floats per vector of T
    const float* dxr = a.dXr + (size_t)t * a.vec * N;
    // two vectors of the row per pass, all their loads issued before the sums (a lane
    // past the row's end reloads its first vector and does not store the second)
    for (int v0 = lane; v0 < a.vec; v0 += 128) {
        const bool two = v0 + 64 < a.vec;
        const int v1 = two ? v0 + 64 : v0;
        uint4 r[2][MOE_MAX_K];
#pragma unroll
        for (int i = 0; i < MOE_MAX_K; ++i) {
            if (i >= k) break;
            r[0][i] = ld_once(dxp + (size_t)sl[i] * a.vec + v0);
            r[1][i] = ld_once(dxp + (size_t)sl[i] * a.vec + v1);
        }
        float4 q[2][N / 4];
#pragma unroll
        for (int h = 0; h < N / 4; ++h) {
            q[0][h] = ld_once(reinterpret_cast<const float4*>(dxr + v0 * N) + h);
            q[1][h] = ld_once(reinterpret_cast<const float4*>(dxr + v1 * N) + h);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int v = u ? v1 : v0;
            float acc[N];
#pragma unroll
            for (int j = 0; j < N; ++j) acc[j] = 0.f;
#pragma unroll
            for (int i = 0; i < MOE_MAX_K; ++i) {
                if (i >= k) break;
                float x[N];
                Vec16<T>::unpack(r[u][i], x);
#pragma unroll
                for (int j = 0; j < N; ++j) acc[j] += x[j];
            }
#pragma unroll
            for (int h = 0; h < N / 4; ++h) {
                acc[4 * h] += q[u][h].x; acc[4 * h + 1] += q[u][h].y;
                acc[4 * h + 2] += q[u][h].z; acc[4 * h + 3] += q[u][h].w;
            }
            if (a.dXs) {                       // shared branch
                float xs[N];
                Vec16<T>::unpack(ld_once(reinterpret_cast<const uint4*>(a.dXs) + (size_t)t * a.vec + v), xs);
#pragma unroll
                for (int j = 0; j < N; ++j) acc[j] += xs[j];
            }
            if (u == 0 || two) reinterpret_cast<uint4*>(a.dX)[(size_t)t * a.vec + v] = Vec16<T>::pack(acc);
        }
    }
}

// Column sums of each expert's row segment (bias gradients).  A workgroup owns
// 32 16-byte column vectors of one expert; its 16 row groups of 32 lanes each sum
// the rows r = lo + g, lo + g + 16, ... (four loads in flight per lane), and the
// 16 partial sums are then added in row-group order: a fixed order, so the
// result is deterministic.
constexpr int COLSUM_RG = 16;
template <class T>
__global__ void __launch_bounds__(COLSUM_RG * 32) colsum_kernel(ColSumArgs a) {
    constexpr int N = Vec16<T>::N;
    __shared__ float part[COLSUM_RG][32 * N];
    const int e = blockIdx.y;
    const int vl = threadIdx.x & 31, rg = threadIdx.x >> 5;
    const int c = (blockIdx.x * 32 + vl) * N;              // first column of this lane
    const bool ok = c < a.ncols;
    const int lo = a.offsets[e], hi = a.offsets[e + 1];
    const T* src = reinterpret_cast<const T*>(a.src);
    float acc[N];
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = 0.f;
    if (ok) {
        int r = lo + rg;
        for (; r + 3 * COLSUM_RG < hi; r += 4 * COLSUM_RG) {
            float x[4][N];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                Vec16<T>::unpack(*reinterpret_cast<const uint4*>(src + (size_t)(r + u * COLSUM_RG) * a.ld + c), x[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < N; ++j) acc[j] += x[u][j];
        }
        for (; r < hi; r += COLSUM_RG) {
            float x[N];
            Vec16<T>::unpack(*reinterpret_cast<const uint4*>(src + (size_t)r * a.ld + c), x);
#pragma unroll
            for (int j = 0; j < N; ++j) acc[j] += x[j];
        }
    }
#pragma unroll
    for (int j = 0; j < N; ++j) part[rg][vl * N + j] = acc[j];
    __syncthreads();
    if (rg == 0 && ok) {
        float out[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            float t = part[0][vl * N + j];
            for (int g = 1; g < COLSUM_RG; ++g) t += part[g][vl * N + j];
            out[j] = t;
        }
#pragma unroll
        for (int j = 0; j < N; ++j) a.dst[(size_t)e * a.ncols + c + j] = out[j];
    }
}

// theta <- theta - lr * grad on the float32 master; working copy = RNE(master).
// Streaming kernel: each thread moves 8 parameters per step with 16-byte
// accesses only (two float4 of master, two of gradient, one 16-byte vector of
// bf16 working copy), two steps in flight; gradients are read once and the
// outputs are not re-read, so those accesses carry the nontemporal hint.
typedef float nf4 __attribute__((ext_vector_type(4)));
typedef unsigned int nu4 __attribute__((ext_vector_type(4)));

template <class TW>
__device__ __forceinline__ void sgd8(float* master, const float* grad, void* work, long i, float lr) {
    nf4* m4 = reinterpret_cast<nf4*>(master) + 2 * i;
    const nf4* g4 = reinterpret_cast<const nf4*>(grad) + 2 * i;
    nf4 m0 = m4[0], m1 = m4[1];
    const nf4 g0 = __builtin_nontemporal_load(g4), g1 = __builtin_nontemporal_load(g4 + 1);
    // one rounding per element, as in the SGD epilogue of the weight-gradient GEMMs
    m0.x = __builtin_fmaf(-lr, g0.x, m0.x); m0.y = __builtin_fmaf(-lr, g0.y, m0.y);
    m0.z = __builtin_fmaf(-lr, g0.z, m0.z); m0.w = __builtin_fmaf(-lr, g0.w, m0.w);
    m1.x = __builtin_fmaf(-lr, g1.x, m1.x); m1.y = __builtin_fmaf(-lr, g1.y, m1.y);
    m1.z = __builtin_fmaf(-lr, g1.z, m1.z); m1.w = __builtin_fmaf(-lr, g1.w, m1.w);
    m4[0] = m0;
    m4[1] = m1;
    if constexpr (sizeof(TW) == 2) {
        const float f[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        const uint4 u = Vec16<bf16>::pack(f);
        const nu4 v = {u.x, u.y, u.z, u.w};
        __builtin_nontemporal_store(v, reinterpret_cast<nu4*>(work) + i);
    } else if (work != master) {
        nf4* w4 = reinterpret_cast<nf4*>(work) + 2 * i;
        __builtin_nontemporal_store(m0, w4);
        __builtin_nontemporal_store(m1, w4 + 1);
    }
}

template <class TW>
__global__ void __launch_bounds__(256) sgd_kernel(SgdArgs a) {
    int sg = 0;
    while (sg + 1 < a.nseg && (int)blockIdx.x >= a.blk0[sg + 1]) ++sg;
    float* master = a.seg[sg].master;
    const float* grad = a.seg[sg].grad;
    void* work = a.seg[sg].work;
    const long n = a.seg[sg].n;
    const long n8 = n / 8;
    const long stride = (long)(a.blk0[sg + 1] - a.blk0[sg]) * blockDim.x;
    long i = (long)(blockIdx.x - a.blk0[sg]) * blockDim.x + threadIdx.x;
    const long i0 = i;
    for (; i + stride < n8; i += 2 * stride) {
        sgd8<TW>(master, grad, work, i, a.lr);
        sgd8<TW>(master, grad, work, i + stride, a.lr);
    }
    if (i < n8) sgd8<TW>(master, grad, work, i, a.lr);
    // tail (n not a multiple of 8)
    for (long t = 8 * n8 + i0; t < n; t += stride) {
        float m = __builtin_fmaf(-a.lr, grad[t], master[t]);
        master[t] = m;
        reinterpret_cast<TW*>(work)[t] = from_f<TW>(m);
    }
}

__global__ void shared_table_kernel(int32_t* tab, int T) {
    if (threadIdx.x != 0) return;
    tab[0] = 0;
    tab[1] = T;
    for (int b = 0; b < 3; ++b) {
        int32_t* tp = tab + 2 + b * (MOE_MAX_EXPERTS + 1);
        const int bm = 64 << b;
        tp[0] = 0;
        tp[1] = (T + bm - 1) / bm;
    }
    tab[2 + 3 * (MOE_MAX_EXPERTS + 1)] = 0;     // segment order: the one segment
}

// ---- host launchers ------------------------------------------------------------
static inline dim3 tok_grid(int T) { return dim3((T + TOK_WAVES - 1) / TOK_WAVES); }
int combine_loss_blocks(int T) { return (T + TOK_WAVES - 1) / TOK_WAVES; }

// Launch KERNEL<..., KT> with KT = k for the common k, else KT = 0 (any k).
#define MOE_LAUNCH_K(KERNEL, k, grid, s, a, ...)                                                  \
    do {                                                                                          \
        switch (k) {                                                                              \
            case 2: hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 2>), grid, dim3(256), 0, s, a); break; \
            case 4: hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 4>), grid, dim3(256), 0, s, a); break; \
            case 6: hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 6>), grid, dim3(256), 0, s, a); break; \
            case 8: hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 8>), grid, dim3(256), 0, s, a); break; \
            default: hipLaunchKernelGGL((KERNEL<__VA_ARGS__, 0>), grid, dim3(256), 0, s, a);        \
        }                                                                                         \
    } while (0)

hipError_t launch_gather(const GatherArgs& a, int dtype, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    if (dtype == MOE_DTYPE_F32) MOE_LAUNCH_K(gather_kernel, a.k, tok_grid(a.T), s, a, float);
    else MOE_LAUNCH_K(gather_kernel, a.k, tok_grid(a.T), s, a, bf16);
    return hipGetLastError();
}
hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    const bool loss = a.Yt != nullptr;
    if (dtype == MOE_DTYPE_F32) {
        if (loss) MOE_LAUNCH_K(combine_kernel, a.k, tok_grid(a.T), s, a, float, true);
        else MOE_LAUNCH_K(combine_kernel, a.k, tok_grid(a.T), s, a, float, false);
    } else {
        if (loss) MOE_LAUNCH_K(combine_kernel, a.k, tok_grid(a.T), s, a, bf16, true);
        else MOE_LAUNCH_K(combine_kernel, a.k, tok_grid(a.T), s, a, bf16, false);
    }
    return hipGetLastError();
}
hipError_t launch_combine_bwd(const CombineBwdArgs& a, int dtype, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    if (dtype == MOE_DTYPE_F32) MOE_LAUNCH_K(combine_bwd_kernel, a.k, tok_grid(a.T), s, a, float);
    else MOE_LAUNCH_K(combine_bwd_kernel, a.k, tok_grid(a.T), s, a, bf16);
    return hipGetLastError();
}
hipError_t launch_scatter(const ScatterArgs& a, int dtype, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    if (dtype == MOE_DTYPE_F32) MOE_LAUNCH_K(scatter_kernel, a.k, tok_grid(a.T), s, a, float);
    else MOE_LAUNCH_K(scatter_kernel, a.k, tok_grid(a.T), s, a, bf16);
    return hipGetLastError();
}
hipError_t launch_colsum(const ColSumArgs& a, int dtype, hipStream_t s) {
    // columns in 16-byte vectors: ncols, ld and the row base are multiples of 16 bytes
    const int per_wg = 32 * (dtype == MOE_DTYPE_F32 ? 4 : 8);
    dim3 grid((a.ncols + per_wg - 1) / per_wg, a.E);
    if (dtype == MOE_DTYPE_F32) hipLaunchKernelGGL(colsum_kernel<float>, grid, dim3(COLSUM_RG * 32), 0, s, a);
    else hipLaunchKernelGGL(colsum_kernel<bf16>, grid, dim3(COLSUM_RG * 32), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_sgd(SgdArgs& a, int dtype, hipStream_t s) {
    // workgroups per segment in proportion to its size, about 16384 in all
    long total = 0;
    for (int i = 0; i < a.nseg; ++i) total += a.seg[i].n;
    if (total == 0) return hipSuccess;
    int b = 0;
    for (int i = 0; i < a.nseg; ++i) {
        a.blk0[i] = b;
        long want = (a.seg[i].n / 8 + 255) / 256;
        long share = (long)((16384.0 * (double)a.seg[i].n) / (double)total) + 1;
        long nb = want < share ? want : share;
        if (nb < 1) nb = 1;
        b += (int)nb;
    }
    a.blk0[a.nseg] = b;
    if (dtype == MOE_DTYPE_F32) hipLaunchKernelGGL(sgd_kernel<float>, dim3(b), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(sgd_kernel<bf16>, dim3(b), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_shared_table(int32_t* tab, int T, hipStream_t s) {
    hipLaunchKernelGGL(shared_table_kernel, dim3(1), dim3(64), 0, s, tab, T);
    return hipGetLastError();
}

}  // namespace moe
