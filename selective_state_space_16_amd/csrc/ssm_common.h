// Device helpers shared by the gfx950 scan and decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;

// Activation storage: float, or bfloat16 held as raw 16-bit patterns.
template <int DT> struct Act;
template <> struct Act<0> { using T = float; };
template <> struct Act<1> { using T = uint16_t; };

__device__ __forceinline__ float ld_act(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_act(const uint16_t *p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);  // exact widening
}
__device__ __forceinline__ void st_act(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_act(uint16_t *p, int64_t i, float v) {
    // gfx950 converts with v_cvt_pk_bf16_f32 (round to nearest even)
    p[i] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Loads of data every lane of a wave shares, through the scalar cache.
typedef const __attribute__((address_space(4))) float *cf32_ptr;
typedef const __attribute__((address_space(4))) uint32_t *cu32_ptr;

// Row of N values starting at element `off`, identical for all lanes.
template <int N>
__device__ __forceinline__ void ld_row_uniform(const float *base, int64_t off, float (&r)[N]) {
    cf32_ptr p = (cf32_ptr)(base + off);
#pragma unroll
    for (int n = 0; n < N; ++n) r[n] = p[n];
}
template <int N>
__device__ __forceinline__ void ld_row_uniform(const uint16_t *base, int64_t off, float (&r)[N]) {
    if constexpr (N == 1) {
        r[0] = ld_act(base, off);  // a single 16-bit value: plain load
    } else {
        cu32_ptr p = (cu32_ptr)(base + off);  // off is even when N is even
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            uint32_t w = p[k];
            r[2 * k] = __uint_as_float(w << 16);
            r[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
        }
    }
}

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

constexpr float kLn2 = 0.6931471805599453f;

// softplus(u) = log(1 + exp(u)) = max(u, 0) + log1p(exp(-|u|)). With
// e = exp(-|u|) in (0, 1] and w = 1 + e rounded to float, w - 1 is exact
// (Sterbenz) and so is r = e - (w - 1), the rounding error of the sum. Then
// log1p(e) = log(w) + log(1 + r / w), and since |r| <= 2^-24 the second term
// differs from r by at most |r| (w - 1) / w + r^2, which is under one ulp of
// log1p(e) (as log1p(e) >= e / (1 + e)). This is the compensated-sum form of
// log1p (the rounding error of 1 + e fed back to first order): it needs no
// division, and gives e when w == 1.
__device__ __forceinline__ float softplus(float u) {
    const float e = fast_exp2(-__builtin_fabsf(u) * kLog2e);
    const float w = 1.0f + e;
    const float r = e - (w - 1.0f);
    return __builtin_fmaf(__builtin_amdgcn_logf(w), kLn2, __builtin_fmaxf(u, 0.0f) + r);
}

// A value as the activation dtype holds it: unchanged for float, rounded to
// the nearest bfloat16 (ties to even) for bfloat16.
template <int DT>
__device__ __forceinline__ float act_round(float v) {
    if constexpr (DT == 0) return v;
    else return (float)(__bf16)v;
}

// silu(z) = z * sigmoid(z) = z / (1 + exp(-z))
__device__ __forceinline__ float silu(float zv) {
    return zv * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-zv * kLog2e));
}

// The x branch ahead of the scan for one (token, channel): SiLU of the causal
// width-4 convolution, bias + w0 x_{t-3} + w1 x_{t-2} + w2 x_{t-1} + w3 x_t,
// summed in that order ("Notas sobre Mamba", section "O bloco Mamba": a short
// depthwise convolution, then SiLU, ahead of S6).
__device__ __forceinline__ float conv_silu(float w0, float w1, float w2, float w3, float bias, float xm3, float xm2,
                                           float xm1, float x0) {
    float u = __builtin_fmaf(w0, xm3, bias);
    u = __builtin_fmaf(w1, xm2, u);
    u = __builtin_fmaf(w2, xm1, u);
    u = __builtin_fmaf(w3, x0, u);
    return silu(u);
}

}  // namespace ssm
