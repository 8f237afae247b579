// The gradient through the x branch ahead of the scan (the Mamba block's
// short causal convolution of width 4, then SiLU: "Notas sobre Mamba", section
// "O bloco Mamba") for gfx950. The scan's own gradient runs unchanged on the
// branch's output; these kernels surround it:
//   conv_fwd_kernel    x = SiLU(b + w0 x_{t-3} + .. + w3 x_t), in the
//                      activation dtype, as the forward scan computes it;
//   conv_bwd_kernel    from the gradient of x: du = dx SiLU'(u), the raw x's
//                      gradient sum_j w_j du_{t+3-j}, that of the three raw
//                      tokens before token 0, and per-(b, chunk) partial
//                      sums of du x_{t-3+j} (taps) and du (bias);
//   conv_reduce_kernel the partial sums, in a fixed order.
// Every kernel maps one lane to a channel, so the loads and stores of a wave
// cover 64 consecutive channels of one token.
#include "ssm_common.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kConvThreads = 256;
constexpr int64_t kConvBlocks = 2048;  // workgroups the chunks of a call aim at
// Tokens whose loads conv_fwd_kernel's lanes issue together before any of
// their stores: the stores go to another array, but the compiler cannot prove
// that, so without the grouping every load would wait for the store before it
// (339 -> 316 us on the large layer; the same grouping made conv_bwd_kernel
// slower, 466 -> 707 us, so it walks token by token).
constexpr int kConvGroup = 8;

// The raw x of token t (zero past L; before token 0 from conv_state, zero
// further back than it reaches or without it).
template <int DT>
__device__ __forceinline__ float raw_at(const ConvBwdArgs &a, int64_t b, int64_t t, int64_t d) {
    using T = typename Act<DT>::T;
    if (t >= 0) return t < a.L ? ld_act((const T *)a.x_raw, (b * a.L + t) * a.D + d) : 0.0f;
    return a.conv_state && t >= -3 ? ld_act((const T *)a.conv_state, (b * a.D + d) * 3 + (t + 3)) : 0.0f;
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
            for (int64_t tg = t0; tg < t1; tg += kConvGroup) {
                float r[kConvGroup];
#pragma unroll
                for (int k = 0; k < kConvGroup; ++k)
                    r[k] = tg + k < t1 ? ld_act((const T *)a.x_raw, (b * a.L + tg + k) * a.D + d) : 0.0f;
#pragma unroll
                for (int k = 0; k < kConvGroup; ++k) {
                    if (tg + k < t1)
                        st_act((T *)a.xc, (b * a.L + tg + k) * a.D + d,
                               conv_silu(w[0], w[1], w[2], w[3], bias, xm[0], xm[1], xm[2], r[k]));
                    xm[0] = xm[1];
                    xm[1] = xm[2];
                    xm[2] = r[k];
                }
            }
        }
}

// grid as conv_fwd_kernel; one partial per (b, chunk) and channel. A lane
// walks its chunk backwards, from the third token after it (whose du the
// chunk's last raw tokens also feed) down to its first, keeping the raw x of
// the four tokens its convolution reads and the du of the three tokens after
// the current one in registers: two loads and one store per token.
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
    const T *gp = (const T *)a.gx;
    for (int64_t b = blockIdx.z; b < a.batch; b += gridDim.z)
        for (int64_t c = blockIdx.y; c < a.nchunk; c += gridDim.y) {
            const int64_t t0 = c * a.chunk, t1 = t0 + a.chunk < L ? t0 + a.chunk : L;
            const int64_t te = t1 + 3 < L ? t1 + 3 : L;  // tokens t0 .. te-1 get a du
            float acc[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};  // taps 0..3, bias
            float dn1 = 0.0f, dn2 = 0.0f, dn3 = 0.0f;       // du of tokens t+1, t+2, t+3
            // raw x of tokens t-3 .. t for t = te - 1
            float x3 = raw_at<DT>(a, b, te - 4, d), x2 = raw_at<DT>(a, b, te - 3, d);
            float x1 = raw_at<DT>(a, b, te - 2, d), x0 = raw_at<DT>(a, b, te - 1, d);
#pragma unroll 4
            for (int64_t t = te - 1; t >= t0; --t) {
                const float g = ld_act(gp, (b * L + t) * D + d);
                const float xn = raw_at<DT>(a, b, t - 4, d);  // the raw x the next (earlier) token adds
                float u = __builtin_fmaf(w[0], x3, bias);
                u = __builtin_fmaf(w[1], x2, u);
                u = __builtin_fmaf(w[2], x1, u);
                u = __builtin_fmaf(w[3], x0, u);
                const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-u * kLog2e));
                const float du = g * sg * __builtin_fmaf(u, 1.0f - sg, 1.0f);
                if (t < t1) {
                    float gr = w[3] * du;
                    gr = __builtin_fmaf(w[2], dn1, gr);
                    gr = __builtin_fmaf(w[1], dn2, gr);
                    gr = __builtin_fmaf(w[0], dn3, gr);
                    st_act((T *)a.dx_raw, (b * L + t) * D + d, gr);
                    acc[0] = __builtin_fmaf(du, x3, acc[0]);
                    acc[1] = __builtin_fmaf(du, x2, acc[1]);
                    acc[2] = __builtin_fmaf(du, x1, acc[2]);
                    acc[3] = __builtin_fmaf(du, x0, acc[3]);
                    acc[4] += du;
                }
                dn3 = dn2;
                dn2 = dn1;
                dn1 = du;
                x0 = x1;
                x1 = x2;
                x2 = x3;
                x3 = xn;
            }
            if (t0 == 0 && a.dconv_state) {
                // dn1, dn2, dn3 now hold du of tokens 0, 1, 2 (zero past L); the
                // raw x of token k - 3 fed tokens 0 .. k through taps k .. 0
                const float du0 = dn1, du1 = dn2, du2 = dn3;
                T *cs = (T *)a.dconv_state + (b * D + d) * 3;
                st_act(cs, 0, w[0] * du0);
                st_act(cs, 1, __builtin_fmaf(w[1], du0, w[0] * du1));
                st_act(cs, 2, __builtin_fmaf(w[2], du0, __builtin_fmaf(w[1], du1, w[0] * du2)));
            }
            float *p = a.part + ((b * a.nchunk + c) * D + d) * 5;
#pragma unroll
            for (int j = 0; j < 5; ++j) p[j] = acc[j];
        }
}

// out[i] = sum over the nparts partials of element i (i < D * 5), in a fixed
// order: row r of a block's 8 rows adds partials r, r + 8, r + 16, .. of its
// 32 elements, and the rows' sums are then added in row order. Taps go to
// dconv_w (D, 4), the bias to dconv_b (D; NULL: skipped).
constexpr int kReduceRows = 8, kReduceCols = kConvThreads / kReduceRows;
__global__ __launch_bounds__(kConvThreads) void conv_reduce_kernel(ConvBwdArgs a, int64_t nparts) {
    __shared__ float rows[kReduceRows][kReduceCols];
    const int r = threadIdx.x / kReduceCols, col = threadIdx.x % kReduceCols;
    const int64_t n = a.D * 5;
    const int64_t i = (int64_t)blockIdx.x * kReduceCols + col;
    float s = 0.0f;
    if (i < n)
        for (int64_t p = r; p < nparts; p += kReduceRows) s += a.part[p * n + i];
    rows[r][col] = s;
    __syncthreads();
    if (r == 0 && i < n) {
        float t = rows[0][col];
#pragma unroll
        for (int k = 1; k < kReduceRows; ++k) t += rows[k][col];
        const int64_t d = i / 5, j = i % 5;
        if (j < 4) a.dconv_w[d * 4 + j] = t;
        else if (a.dconv_b) a.dconv_b[d] = t;
    }
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

void conv_bwd_plan(int64_t batch, int64_t L, int64_t D, int64_t *chunk, int64_t *nchunk) {
    // enough chunks for about kConvBlocks workgroups (each lane walks its chunk
    // in order), in whole multiples of 16 tokens
    const int64_t cblocks = (D + kConvThreads - 1) / kConvThreads;
    const int64_t rows = batch * cblocks > 0 ? batch * cblocks : 1;
    int64_t want = (kConvBlocks + rows - 1) / rows;
    const int64_t most = L > 0 ? (L + 15) / 16 : 1;
    want = want < most ? want : most;
    want = want > 0 ? want : 1;
    int64_t c = L > 0 ? (L + want - 1) / want : 16;
    c = (c + 15) / 16 * 16;
    *chunk = c;
    *nchunk = L > 0 ? (L + c - 1) / c : 1;
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
    if ((a.D * 5 + kReduceCols - 1) / kReduceCols > INT32_MAX) return hipErrorInvalidValue;
    if (a.L <= 0 || a.batch <= 0) {
        // no token: zero gradients of the taps, bias and earlier raw tokens
        if (a.dconv_state && a.batch > 0) {
            const int64_t n = a.batch * a.D * 3;
            const dim3 g((unsigned)((n + kConvThreads - 1) / kConvThreads));
            if (dtype == 0) hipLaunchKernelGGL(act_zero_kernel<0>, g, dim3(kConvThreads), 0, s, a.dconv_state, n);
            else hipLaunchKernelGGL(act_zero_kernel<1>, g, dim3(kConvThreads), 0, s, a.dconv_state, n);
        }
        hipLaunchKernelGGL(conv_reduce_kernel, dim3((unsigned)((a.D * 5 + kReduceCols - 1) / kReduceCols)),
                           dim3(kConvThreads), 0, s, a, (int64_t)0);
        return hipGetLastError();
    }
    if (dtype == 0) hipLaunchKernelGGL(conv_bwd_kernel<0>, conv_grid(a), dim3(kConvThreads), 0, s, a);
    else hipLaunchKernelGGL(conv_bwd_kernel<1>, conv_grid(a), dim3(kConvThreads), 0, s, a);
    hipLaunchKernelGGL(conv_reduce_kernel, dim3((unsigned)((a.D * 5 + kReduceCols - 1) / kReduceCols)),
                       dim3(kConvThreads), 0, s, a, a.batch * a.nchunk);
    return hipGetLastError();
}

}  // namespace ssm
