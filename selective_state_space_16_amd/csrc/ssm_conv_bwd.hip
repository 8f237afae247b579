// The gradient through the x branch ahead of the scan (the Mamba block's
// short causal convolution of width 4, then SiLU: "Notas sobre Mamba", section
// "O bloco Mamba") for gfx950. The scan's own gradient runs unchanged on the
// branch's output; these kernels surround it:
//   conv_fwd_kernel    x = SiLU(b + w0 x_{t-3} + .. + w3 x_t), in the
//                      activation dtype, as the forward scan computes it;
//   conv_bwd_kernel    from the gradient of x: du = dx SiLU'(u), the raw x's
//                      gradient sum_j w_j du_{t+3-j}, that of the three raw
//                      tokens before token 0, and per-(b, chunk) partial sums
//                      of du x_{t-3+j} (taps) and du (bias);
//   conv_reduce_kernel the partial sums, in a fixed order.
// Every kernel maps one lane to a channel, so the loads and stores of a wave
// cover 64 consecutive channels of one token.
#include "ssm_common.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kConvThreads = 256;
constexpr int kConvSub = 16;  // tokens per register block of conv_bwd_kernel

template <int DT>
__device__ __forceinline__ float raw_at(const ConvBwdArgs &a, int64_t b, int64_t t, int64_t d) {
    using T = typename Act<DT>::T;
    if (t >= 0) return t < a.L ? ld_act((const T *)a.x_raw, (b * a.L + t) * a.D + d) : 0.0f;
    return a.conv_state ? ld_act((const T *)a.conv_state, (b * a.D + d) * 3 + (t + 3)) : 0.0f;
}

// grid: x = 256-channel block, y = token chunk (strided), z = batch row (strided)
template <int DT>
__global__ __launch_bounds__(kConvThreads) void conv_fwd_kernel(ConvBwdArgs a) {
    using T = typename Act<DT>::T;
    const int64_t d = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    if (d >= a.D) return;
    float w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = a.conv_w[d * 4 + j];
    const float bias = a.conv_b ? a.conv_b[d] : 0.0f;
    for (int64_t b = blockIdx.z; b < a.batch; b += gridDim.z)
        for (int64_t c = blockIdx.y; c < a.nchunk; c += gridDim.y) {
            const int64_t t0 = c * a.chunk, t1 = t0 + a.chunk < a.L ? t0 + a.chunk : a.L;
            float xm[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) xm[j] = raw_at<DT>(a, b, t0 - 3 + j, d);
            for (int64_t t = t0; t < t1; ++t) {
                const float raw = ld_act((const T *)a.x_raw, (b * a.L + t) * a.D + d);
                st_act((T *)a.xc, (b * a.L + t) * a.D + d,
                       conv_silu(w[0], w[1], w[2], w[3], bias, xm[0], xm[1], xm[2], raw));
                xm[0] = xm[1];
                xm[1] = xm[2];
                xm[2] = raw;
            }
        }
}

// grid as conv_fwd_kernel; one partial per (b, chunk) and channel
template <int DT>
__global__ __launch_bounds__(kConvThreads) void conv_bwd_kernel(ConvBwdArgs a) {
    using T = typename Act<DT>::T;
    const int64_t D = a.D, L = a.L;
    const int64_t d = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    if (d >= D) return;
    float w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = a.conv_w[d * 4 + j];
    const float bias = a.conv_b ? a.conv_b[d] : 0.0f;
    for (int64_t b = blockIdx.z; b < a.batch; b += gridDim.z)
        for (int64_t c = blockIdx.y; c < a.nchunk; c += gridDim.y) {
            const int64_t t0 = c * a.chunk, t1 = t0 + a.chunk < L ? t0 + a.chunk : L;
            float acc[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};  // taps 0..3, bias
            for (int64_t s0 = t0; s0 < t1; s0 += kConvSub) {
                // raw x of tokens s0-3 .. s0+18 and the gradient of x (zero past
                // L) of tokens s0 .. s0+18: the block's tokens and the three
                // after them, whose du the block's raw x also feed
                float xr[kConvSub + 6], g[kConvSub + 3], du[kConvSub + 3];
#pragma unroll
                for (int k = 0; k < kConvSub + 6; ++k) xr[k] = raw_at<DT>(a, b, s0 - 3 + k, d);
#pragma unroll
                for (int k = 0; k < kConvSub + 3; ++k) {
                    const int64_t t = s0 + k;
                    g[k] = t < L ? ld_act((const T *)a.gx, (b * L + t) * D + d) : 0.0f;
                }
#pragma unroll
                for (int k = 0; k < kConvSub + 3; ++k) {
                    float u = __builtin_fmaf(w[0], xr[k], bias);
                    u = __builtin_fmaf(w[1], xr[k + 1], u);
                    u = __builtin_fmaf(w[2], xr[k + 2], u);
                    u = __builtin_fmaf(w[3], xr[k + 3], u);
                    const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-u * kLog2e));
                    du[k] = g[k] * sg * __builtin_fmaf(u, 1.0f - sg, 1.0f);
                }
#pragma unroll
                for (int k = 0; k < kConvSub; ++k) {
                    const int64_t t = s0 + k;
                    if (t < t1) {
                        float gr = w[3] * du[k];
                        gr = __builtin_fmaf(w[2], du[k + 1], gr);
                        gr = __builtin_fmaf(w[1], du[k + 2], gr);
                        gr = __builtin_fmaf(w[0], du[k + 3], gr);
                        st_act((T *)a.dx_raw, (b * L + t) * D + d, gr);
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[j] = __builtin_fmaf(du[k], xr[k + j], acc[j]);
                        acc[4] += du[k];
                    }
                }
                if (s0 == 0 && a.dconv_state) {
                    // the raw x of token kk - 3 fed tokens 0 .. kk through taps kk .. 0
#pragma unroll
                    for (int kk = 0; kk < 3; ++kk) {
                        float gr = 0.0f;
#pragma unroll
                        for (int j = 0; j <= kk; ++j) gr = __builtin_fmaf(w[j], du[kk - j], gr);
                        st_act((T *)a.dconv_state, (b * D + d) * 3 + kk, gr);
                    }
                }
            }
            float *p = a.part + ((b * a.nchunk + c) * D + d) * 5;
#pragma unroll
            for (int j = 0; j < 5; ++j) p[j] = acc[j];
        }
}

// out[i] = sum over the nparts partials of element i (i < D * 5), partial 0
// first; taps to dconv_w (D, 4), the bias to dconv_b (D; NULL: skipped)
__global__ __launch_bounds__(kConvThreads) void conv_reduce_kernel(ConvBwdArgs a, int64_t nparts) {
    const int64_t i = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    if (i >= a.D * 5) return;
    float s = 0.0f;
    for (int64_t p = 0; p < nparts; ++p) s += a.part[p * a.D * 5 + i];
    const int64_t d = i / 5, j = i % 5;
    if (j < 4) a.dconv_w[d * 4 + j] = s;
    else if (a.dconv_b) a.dconv_b[d] = s;
}

// zeros of the activation dtype
template <int DT>
__global__ __launch_bounds__(kConvThreads) void act_zero_kernel(void *p, int64_t n) {
    using T = typename Act<DT>::T;
    const int64_t i = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    if (i < n) ((T *)p)[i] = T(0);
}

dim3 conv_grid(const ConvBwdArgs &a) {
    const int64_t cb = (a.D + kConvThreads - 1) / kConvThreads;
    return dim3((unsigned)cb, (unsigned)(a.nchunk < 65535 ? a.nchunk : 65535),
                (unsigned)(a.batch < 65535 ? a.batch : 65535));
}

}  // namespace

void conv_bwd_plan(int64_t L, int64_t *chunk, int64_t *nchunk) {
    // at most 64 chunks per batch row, each a whole number of register blocks
    int64_t n = (L + kConvSub - 1) / kConvSub;
    n = n < 64 ? n : 64;
    n = n > 0 ? n : 1;
    int64_t c = (L + n - 1) / n;
    c = (c + kConvSub - 1) / kConvSub * kConvSub;
    *chunk = c > 0 ? c : kConvSub;
    *nchunk = (L + *chunk - 1) / *chunk;
    if (*nchunk < 1) *nchunk = 1;
}

hipError_t launch_conv_fwd(const ConvBwdArgs &a, int dtype, hipStream_t s) {
    if (a.D <= 0 || a.L <= 0 || a.batch <= 0) return hipSuccess;
    if ((a.D + kConvThreads - 1) / kConvThreads > INT32_MAX) return hipErrorInvalidValue;
    if (dtype == 0) hipLaunchKernelGGL(conv_fwd_kernel<0>, conv_grid(a), dim3(kConvThreads), 0, s, a);
    else hipLaunchKernelGGL(conv_fwd_kernel<1>, conv_grid(a), dim3(kConvThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_conv_bwd(const ConvBwdArgs &a, int dtype, hipStream_t s) {
    if (a.D <= 0) return hipSuccess;
    if ((a.D * 5 + kConvThreads - 1) / kConvThreads > INT32_MAX) return hipErrorInvalidValue;
    if (a.L <= 0 || a.batch <= 0) {
        // no token: zero gradients of the taps, bias and earlier raw tokens
        if (a.dconv_state && a.batch > 0) {
            const int64_t n = a.batch * a.D * 3;
            const dim3 g((unsigned)((n + kConvThreads - 1) / kConvThreads));
            if (dtype == 0) hipLaunchKernelGGL(act_zero_kernel<0>, g, dim3(kConvThreads), 0, s, a.dconv_state, n);
            else hipLaunchKernelGGL(act_zero_kernel<1>, g, dim3(kConvThreads), 0, s, a.dconv_state, n);
        }
        hipLaunchKernelGGL(conv_reduce_kernel, dim3((unsigned)((a.D * 5 + kConvThreads - 1) / kConvThreads)),
                           dim3(kConvThreads), 0, s, a, (int64_t)0);
        return hipGetLastError();
    }
    if (dtype == 0) hipLaunchKernelGGL(conv_bwd_kernel<0>, conv_grid(a), dim3(kConvThreads), 0, s, a);
    else hipLaunchKernelGGL(conv_bwd_kernel<1>, conv_grid(a), dim3(kConvThreads), 0, s, a);
    hipLaunchKernelGGL(conv_reduce_kernel, dim3((unsigned)((a.D * 5 + kConvThreads - 1) / kConvThreads)),
                       dim3(kConvThreads), 0, s, a, a.batch * a.nchunk);
    return hipGetLastError();
}

}  // namespace ssm
