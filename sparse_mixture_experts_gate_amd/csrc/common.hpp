// Shared device helpers for the gfx950 kernels of the sparse MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

namespace moe {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// ---- conversions -----------------------------------------------------------
// float <-> bfloat16 with round-to-nearest-even (finite inputs).
__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }
__device__ __forceinline__ bf16 f2bf(float v) { return (bf16)v; }

template <class T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16>(bf16 v) { return (float)v; }
template <class T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }

// Eight values of a 16-byte vector of T (T = bf16: 8 lanes; T = float: 4 lanes).
template <class T> struct Vec16;
template <> struct Vec16<bf16> {
    static constexpr int N = 8;
    __device__ static void unpack(const uint4& u, float* f) {
        const bf16* p = reinterpret_cast<const bf16*>(&u);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (float)p[i];
    }
    __device__ static uint4 pack(const float* f) {
        uint4 u;
        bf16* p = reinterpret_cast<bf16*>(&u);
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = (bf16)f[i];
        return u;
    }
};
template <> struct Vec16<float> {
    static constexpr int N = 4;
    __device__ static void unpack(const uint4& u, float* f) {
        f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
    }
    __device__ static uint4 pack(const float* f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                          __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
};

// ---- wavefront reductions (fixed butterfly order: deterministic) ------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(v, o, MOE_WAVE);
        if (lane >= o) v += u;
    }
    return v;
}

// ---- activations --------------------------------------------------------------
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x * sigmoidf_(x); }
__device__ __forceinline__ float silu_gradf_(float x) {
    float s = sigmoidf_(x);
    return s * (1.0f + x * (1.0f - s));
}
__device__ __forceinline__ float geluf_(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_gradf_(float x) {
    float cdf = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
    float pdf = 0.39894228040143268f * __expf(-0.5f * x * x);
    return cdf + x * pdf;
}

// Faster forms for the bfloat16 GEMM epilogues, whose outputs are rounded to bf16
// (relative step 2^-8) right after:
//  * the logistic function with the hardware reciprocal (v_rcp_f32, 1 ulp);
//  * erf by the rational approximation 7.1.26 of Abramowitz and Stegun's Handbook
//    of Mathematical Functions: for z >= 0, with t = 1 / (1 + p z),
//    erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2), absolute error
//    at most 1.5e-7, and erf(-z) = -erf(z).  GELU' shares exp(-x^2 / 2) between the
//    normal CDF and density.
// The float32 layer and the routing keep the forms above.
__device__ __forceinline__ float sigmoid_fast_(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
__device__ __forceinline__ float silu_fast_(float x) { return x * sigmoid_fast_(x); }
__device__ __forceinline__ float silu_grad_fast_(float x) {
    const float s = sigmoid_fast_(x);
    return s * (1.0f + x * (1.0f - s));
}
// Phi(x) = (1 + erf(x / sqrt 2)) / 2 with e = exp(-x^2 / 2) given
__device__ __forceinline__ float normal_cdf_as_(float x, float e) {
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
    float poly = fmaf(1.061405429f, t, -1.453152027f);
    poly = fmaf(poly, t, 1.421413741f);
    poly = fmaf(poly, t, -0.284496736f);
    poly = fmaf(poly, t, 0.254829592f);
    const float erf_z = 1.0f - poly * t * e;          // erf(|x| / sqrt 2)
    return 0.5f + 0.5f * copysignf(erf_z, x);
}
__device__ __forceinline__ float gelu_fast_(float x) {
    return x * normal_cdf_as_(x, __expf(-0.5f * x * x));
}
__device__ __forceinline__ float gelu_grad_fast_(float x) {
    const float e = __expf(-0.5f * x * x);
    return normal_cdf_as_(x, e) + x * (0.39894228040143268f * e);
}

}  // namespace moe
