// Mamba-2 SSD decode step for gfx950: one token per (batch row, head) on a
// stored (P, N) float32 state, updated in place ("Mamba-2 e State Space
// Duality (SSD)", section "Mamba-2 e SSD": the scalar-times-identity
// transition; the recurrent form of "A forma dual: atenção mascarada"):
//
//   a = exp(delta A[h]);  S[p][n] = a S[p][n] + delta x[p] Bt[g][n]
//   y[p] = sum_n Ct[g][n] S[p][n] + Dskip[h] x[p]
//
// The step reads and writes the whole state once and does a few flops per
// element: it is HBM-bound. One workgroup per (b, h). A state row is N
// consecutive floats read by N / 4 consecutive lanes, 16 bytes each, so that
// every load and store instruction of a wave covers whole rows: the workgroup
// takes 1024 / N rows per pass and P N / 1024 passes, with every pass's loads
// issued before the first update. A row's readout meets through lane
// exchanges.
#include "ssm_common.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kStepThreads = 256;

template <int P, int N, int DT, bool SKIP>
__global__ __launch_bounds__(kStepThreads) void ssd_step_kernel(SsdStepArgs a) {
    using T = typename Act<DT>::T;
    constexpr int TPR = N / 4;                  // lanes per state row, 4 elements each
    constexpr int RPP = kStepThreads / TPR;     // rows per pass
    constexpr int PASSES = P / RPP;
    static_assert(TPR <= 64 && (TPR & (TPR - 1)) == 0 && P % RPP == 0, "whole rows per pass");
    const int64_t H = a.H, G = a.G;
    const int64_t bh = blockIdx.x, b = bh / H, h = bh % H, g = h / (H / G);
    const int tid = threadIdx.x, r0 = tid / TPR, n0 = (tid % TPR) * 4;
    using F4 = float __attribute__((ext_vector_type(4)));
    F4 *S = (F4 *)(a.state + (bh * P + r0) * N + n0);  // pass q: row r0 + q RPP
    F4 s[PASSES];
#pragma unroll
    for (int q = 0; q < PASSES; ++q) s[q] = S[q * RPP * N / 4];
    const float dt = ld_act((const T *)a.delta, bh);
    const float av = fast_exp2(dt * a.A[h] * kLog2e);
    float Bv[4], Cv[4], xv[PASSES];
    const int64_t bc = (b * G + g) * N + n0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        Bv[k] = ld_act((const T *)a.Bt, bc + k);
        Cv[k] = ld_act((const T *)a.Ct, bc + k);
    }
#pragma unroll
    for (int q = 0; q < PASSES; ++q) xv[q] = ld_act((const T *)a.x, bh * P + r0 + q * RPP);
    const float dsk = SKIP ? a.Dskip[h] : 0.0f;
#pragma unroll
    for (int q = 0; q < PASSES; ++q) {
        const float dx = dt * xv[q];
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = __builtin_fmaf(av, s[q][e], dx * Bv[e]);
            s[q][e] = v;
            acc = __builtin_fmaf(Cv[e], v, acc);
        }
        S[q * RPP * N / 4] = s[q];
#pragma unroll
        for (int m = 1; m < TPR; m *= 2) acc += __shfl_xor(acc, m);
        if (tid % TPR == 0) {
            if (SKIP) acc = __builtin_fmaf(dsk, xv[q], acc);
            st_act((T *)a.y, bh * P + r0 + q * RPP, acc);
        }
    }
}

template <int N, int DT>
hipError_t launch_ssd_step_n(const SsdStepArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)(a.batch * a.H));
    if (a.Dskip)
        hipLaunchKernelGGL((ssd_step_kernel<64, N, DT, true>), grid, dim3(kStepThreads), 0, s, a);
    else
        hipLaunchKernelGGL((ssd_step_kernel<64, N, DT, false>), grid, dim3(kStepThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool ssd_step_supported(int64_t P, int64_t N) { return P == 64 && (N == 64 || N == 128); }

hipError_t launch_ssd_step(const SsdStepArgs &a, int N, int dtype, hipStream_t s) {
    if (N == 64) return dtype == 0 ? launch_ssd_step_n<64, 0>(a, s) : launch_ssd_step_n<64, 1>(a, s);
    if (N == 128) return dtype == 0 ? launch_ssd_step_n<128, 0>(a, s) : launch_ssd_step_n<128, 1>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace ssm
