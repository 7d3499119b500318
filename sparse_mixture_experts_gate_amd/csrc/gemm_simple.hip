// Expert and router contractions for the float32 layer (one thread per output
// element, fp32 accumulation in ascending k).  The float32 layer is the small
// training-step shape whose tolerance is relative 1e-5, so these kernels aim
// at exactness, not speed; the bfloat16 layer runs on the MFMA kernels.
//
// Sources: "Trainable MoE in CUDA" outline Part 1 (matmul variants: X W^T,
// dY W, dY^T X; bias add and reduction), Part 3 (gate matmul and its
// gradient), Part 5 (expert up/down projections, activation, backward).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Expert of expert-major row r: the e with offsets[e] <= r < offsets[e+1].
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
    int lo = 0, hi = E;           // invariant: offsets[lo] <= r < offsets[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (offsets[mid] <= r) lo = mid; else hi = mid;
    }
    return lo;
}

// grid (ceil(ffn/256), rows): H / H1|H3 and A of one expert-major row.
template <class T, int EPI>
__global__ void __launch_bounds__(256) s_up_fwd(ExpertGemmArgs a) {
    const int r = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
    if (j >= a.ffn) return;
    const int e = expert_of_row(a.offsets, a.E, r);
    const T* x = reinterpret_cast<const T*>(a.Xp) + (size_t)r * a.d;
    const T* w1 = reinterpret_cast<const T*>(a.W1) + ((size_t)e * a.ffn + j) * a.d;
    float h1 = 0.f;
    for (int c = 0; c < a.d; ++c) h1 = fmaf(to_f<T>(x[c]), to_f<T>(w1[c]), h1);
    T* H = reinterpret_cast<T*>(a.H);
    T* A = reinterpret_cast<T*>(a.A);
    if (EPI == EPI_UP_SWIGLU) {
        const T* w3 = reinterpret_cast<const T*>(a.W3) + ((size_t)e * a.ffn + j) * a.d;
        float h3 = 0.f;
        for (int c = 0; c < a.d; ++c) h3 = fmaf(to_f<T>(x[c]), to_f<T>(w3[c]), h3);
        H[(size_t)r * 2 * a.ffn + j] = from_f<T>(h1);
        H[(size_t)r * 2 * a.ffn + a.ffn + j] = from_f<T>(h3);
        A[(size_t)r * a.ffn + j] = from_f<T>(siluf_(h1) * h3);
    } else {
        h1 += to_f<T>(reinterpret_cast<const T*>(a.b1)[(size_t)e * a.ffn + j]);
        H[(size_t)r * a.ffn + j] = from_f<T>(h1);
        A[(size_t)r * a.ffn + j] = from_f<T>(EPI == EPI_UP_RELU ? fmaxf(h1, 0.f) : geluf_(h1));
    }
}

// grid (ceil(d/256), rows): EO = A W2^T (+ b2).
template <class T>
__global__ void __launch_bounds__(256) s_down_fwd(ExpertGemmArgs a) {
    const int r = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
    if (c >= a.d) return;
    const int e = expert_of_row(a.offsets, a.E, r);
    const T* x = reinterpret_cast<const T*>(a.A) + (size_t)r * a.ffn;
    const T* w = reinterpret_cast<const T*>(a.W2) + ((size_t)e * a.d + c) * a.ffn;
    float acc = 0.f;
    for (int j = 0; j < a.ffn; ++j) acc = fmaf(to_f<T>(x[j]), to_f<T>(w[j]), acc);
    if (a.b2) acc += to_f<T>(reinterpret_cast<const T*>(a.b2)[(size_t)e * a.d + c]);
    reinterpret_cast<T*>(a.EO)[(size_t)r * a.d + c] = from_f<T>(acc);
}

// grid (ceil(ffn/256), rows): dA = dEO W2, then the activation backward.
template <class T, int EPI>
__global__ void __launch_bounds__(256) s_down_dgrad(ExpertGemmArgs a) {
    const int r = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
    if (j >= a.ffn) return;
    const int e = expert_of_row(a.offsets, a.E, r);
    const T* g = reinterpret_cast<const T*>(a.dEO) + (size_t)r * a.d;
    const T* w = reinterpret_cast<const T*>(a.W2) + (size_t)e * a.d * a.ffn + j;
    float dA = 0.f;
    for (int c = 0; c < a.d; ++c) dA = fmaf(to_f<T>(g[c]), to_f<T>(w[(size_t)c * a.ffn]), dA);
    const T* H = reinterpret_cast<const T*>(a.H);
    T* dH = reinterpret_cast<T*>(a.dH);
    if (EPI == EPI_DN_SWIGLU) {
        float h1 = to_f<T>(H[(size_t)r * 2 * a.ffn + j]);
        float h3 = to_f<T>(H[(size_t)r * 2 * a.ffn + a.ffn + j]);
        dH[(size_t)r * 2 * a.ffn + j] = from_f<T>(dA * h3 * silu_gradf_(h1));
        dH[(size_t)r * 2 * a.ffn + a.ffn + j] = from_f<T>(dA * siluf_(h1));
    } else {
        float h = to_f<T>(H[(size_t)r * a.ffn + j]);
        float gr = (EPI == EPI_DN_RELU) ? (h > 0.f ? 1.f : 0.f) : gelu_gradf_(h);
        dH[(size_t)r * a.ffn + j] = from_f<T>(dA * gr);
    }
}

// grid (ceil(d/256), rows): dXp = dH W1 (+ dH3 W3).
template <class T>
__global__ void __launch_bounds__(256) s_up_dgrad(ExpertGemmArgs a) {
    const int r = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
    if (c >= a.d) return;
    const int e = expert_of_row(a.offsets, a.E, r);
    const bool glu = a.expert == MOE_EXPERT_SWIGLU;
    const int hcols = glu ? 2 * a.ffn : a.ffn;
    const T* g = reinterpret_cast<const T*>(a.dH) + (size_t)r * hcols;
    const T* w1 = reinterpret_cast<const T*>(a.W1) + (size_t)e * a.ffn * a.d + c;
    float acc = 0.f;
    for (int j = 0; j < a.ffn; ++j) acc = fmaf(to_f<T>(g[j]), to_f<T>(w1[(size_t)j * a.d]), acc);
    if (glu) {
        const T* w3 = reinterpret_cast<const T*>(a.W3) + (size_t)e * a.ffn * a.d + c;
        for (int j = 0; j < a.ffn; ++j)
            acc = fmaf(to_f<T>(g[a.ffn + j]), to_f<T>(w3[(size_t)j * a.d]), acc);
    }
    reinterpret_cast<T*>(a.dXp)[(size_t)r * a.d + c] = from_f<T>(acc);
}

// out[e][m][n] = sum over rows r of expert e of P[r][pcol0 + m] * Q[r][n].
template <class T>
__global__ void __launch_bounds__(256)
s_wgrad(const int32_t* offsets, const T* P, int ldp, int pcol0, const T* Q, int ldq,
        float* out, int M, int N, float* master, T* work, float lr) {
    const int e = blockIdx.z, m = blockIdx.y, n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const int lo = offsets[e], hi = offsets[e + 1];
    float acc = 0.f;
    for (int r = lo; r < hi; ++r)
        acc = fmaf(to_f<T>(P[(size_t)r * ldp + pcol0 + m]), to_f<T>(Q[(size_t)r * ldq + n]), acc);
    const size_t o = ((size_t)e * M + m) * N + n;
    if (master) {           // SGD step in place of storing the gradient
        const float w = fmaf(-lr, acc, master[o]);
        master[o] = w;
        work[o] = from_f<T>(w);
    } else {
        out[o] = acc;
    }
}

// Router: logits = X Wg^T (fp32 out).
template <class T>
__global__ void __launch_bounds__(256) s_router_logits(RouterGemmArgs a) {
    const int t = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
    if (e >= a.E) return;
    const T* x = reinterpret_cast<const T*>(a.X) + (size_t)t * a.d;
    const T* w = reinterpret_cast<const T*>(a.Wg) + (size_t)e * a.d;
    float acc = 0.f;
    for (int c = 0; c < a.d; ++c) acc = fmaf(to_f<T>(x[c]), to_f<T>(w[c]), acc);
    a.logits[(size_t)t * a.E + e] = acc;
}
// dXr = dl Wg (fp32 out).
template <class T>
__global__ void __launch_bounds__(256) s_router_dx(RouterGemmArgs a) {
    const int t = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
    if (c >= a.d) return;
    const T* dl = reinterpret_cast<const T*>(a.dl) + (size_t)t * a.E;
    const T* w = reinterpret_cast<const T*>(a.Wg) + c;
    float acc = 0.f;
    for (int e = 0; e < a.E; ++e) acc = fmaf(to_f<T>(dl[e]), to_f<T>(w[(size_t)e * a.d]), acc);
    a.dXr[(size_t)t * a.d + c] = acc;
}
// dWg = dl^T X (fp32 out).
template <class T>
__global__ void __launch_bounds__(256) s_router_dwg(RouterGemmArgs a) {
    const int e = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
    if (c >= a.d) return;
    const T* dl = reinterpret_cast<const T*>(a.dl);
    const T* x = reinterpret_cast<const T*>(a.X);
    float acc = 0.f;
    for (int t = 0; t < a.T; ++t)
        acc = fmaf(to_f<T>(dl[(size_t)t * a.E + e]), to_f<T>(x[(size_t)t * a.d + c]), acc);
    a.dWg[(size_t)e * a.d + c] = acc;
}

// ---- launchers (float32 layer) -----------------------------------------------------
static inline dim3 g2(int cols, int rows) { return dim3((cols + 255) / 256, rows); }

hipError_t simple_up_fwd(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    dim3 g = g2(a.ffn, a.rows);
    if (a.expert == MOE_EXPERT_SWIGLU) hipLaunchKernelGGL((s_up_fwd<float, EPI_UP_SWIGLU>), g, dim3(256), 0, s, a);
    else if (a.expert == MOE_EXPERT_RELU) hipLaunchKernelGGL((s_up_fwd<float, EPI_UP_RELU>), g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((s_up_fwd<float, EPI_UP_GELU>), g, dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t simple_down_fwd(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    hipLaunchKernelGGL(s_down_fwd<float>, g2(a.d, a.rows), dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t simple_down_dgrad(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    dim3 g = g2(a.ffn, a.rows);
    if (a.expert == MOE_EXPERT_SWIGLU) hipLaunchKernelGGL((s_down_dgrad<float, EPI_DN_SWIGLU>), g, dim3(256), 0, s, a);
    else if (a.expert == MOE_EXPERT_RELU) hipLaunchKernelGGL((s_down_dgrad<float, EPI_DN_RELU>), g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((s_down_dgrad<float, EPI_DN_GELU>), g, dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t simple_up_dgrad(const ExpertGemmArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    hipLaunchKernelGGL(s_up_dgrad<float>, g2(a.d, a.rows), dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t simple_down_wgrad(const ExpertGemmArgs& a, hipStream_t s) {
    // dW2[e][c][j] = sum_r dEO[r][c] * A[r][j]
    hipLaunchKernelGGL(s_wgrad<float>, dim3((a.ffn + 255) / 256, a.d, a.E), dim3(256), 0, s,
                       a.offsets, (const float*)a.dEO, a.d, 0, (const float*)a.A, a.ffn, a.dW2, a.d, a.ffn,
                       a.W2m, (float*)a.W2w, a.lr);
    return hipGetLastError();
}
hipError_t simple_up_wgrad(const ExpertGemmArgs& a, hipStream_t s) {
    const bool glu = a.expert == MOE_EXPERT_SWIGLU;
    const int hcols = glu ? 2 * a.ffn : a.ffn;
    dim3 g((a.d + 255) / 256, a.ffn, a.E);
    hipLaunchKernelGGL(s_wgrad<float>, g, dim3(256), 0, s, a.offsets, (const float*)a.dH, hcols, 0,
                       (const float*)a.Xp, a.d, a.dW1, a.ffn, a.d, a.W1m, (float*)a.W1w, a.lr);
    if (glu)
        hipLaunchKernelGGL(s_wgrad<float>, g, dim3(256), 0, s, a.offsets, (const float*)a.dH, hcols, a.ffn,
                           (const float*)a.Xp, a.d, a.dW3, a.ffn, a.d, a.W3m, (float*)a.W3w, a.lr);
    return hipGetLastError();
}
hipError_t simple_router_logits(const RouterGemmArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    hipLaunchKernelGGL(s_router_logits<float>, g2(a.E, a.T), dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t simple_router_dx(const RouterGemmArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    hipLaunchKernelGGL(s_router_dx<float>, g2(a.d, a.T), dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t simple_router_dwg(const RouterGemmArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(s_router_dwg<float>, g2(a.d, a.E), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
