// Single-token recurrent decode step (S6) for gfx950.
//
// The step reads and rewrites the whole (batch, D, N) float state, so it is
// bound by memory traffic ("Notas sobre Mamba", section "Formulação MIMO":
// decode cost is governed by the state read and written each token). Each
// lane owns NPL = min(N, 4) consecutive state values of one channel and
// moves them as one 16-byte access; LPC = N / NPL lanes share a channel, so a
// wave covers 64 / LPC channels of one batch row and its state accesses are
// one contiguous span. The partial readouts of a channel's lanes are summed
// with DPP quad permutes; the first lane of the group finishes the channel
// (D skip, silu gate) and stores y.
#include "ssm_common.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kStepBlock = 256;

template <int NPL> struct Vec;
template <> struct Vec<1> { using T = float; };
template <> struct Vec<2> { using T = float2; };
template <> struct Vec<4> { using T = float4; };

template <int NPL>
__device__ __forceinline__ void ld_vec(const float *p, float (&r)[NPL]) {
    const typename Vec<NPL>::T v = *(const typename Vec<NPL>::T *)p;
    __builtin_memcpy(r, &v, sizeof(v));
}
template <int NPL>
__device__ __forceinline__ void st_vec(float *p, const float (&r)[NPL]) {
    typename Vec<NPL>::T v;
    __builtin_memcpy(&v, r, sizeof(v));
    *(typename Vec<NPL>::T *)p = v;
}

// Sum over the LPC lanes of a group (LPC in {1, 2, 4}; groups are aligned quads
// or pairs inside a quad).
template <int LPC>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPC >= 2)  // quad_perm [1,0,3,2]
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    if constexpr (LPC >= 4)  // quad_perm [2,3,0,1]
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    return v;
}

template <int N, int DT, bool GATE, bool SKIP>
__global__ __launch_bounds__(kStepBlock) void step_kernel(StepArgs a) {
    using T = typename Act<DT>::T;
    constexpr int NPL = N < 4 ? N : 4;
    constexpr int LPC = N / NPL;
    constexpr int CPB = kStepBlock / LPC;  // channels per block
    const int64_t D = a.D;
    const int64_t nblk = (D + CPB - 1) / CPB;  // flat grid: block id = b * nblk + channel block
    const int64_t b = blockIdx.x / nblk;
    const int tid = threadIdx.x;
    const int64_t d = (int64_t)(blockIdx.x % nblk) * CPB + tid / LPC;
    const int sub = tid % LPC;
    const bool valid = d < D;
    const int64_t dc = valid ? d : D - 1;
    const int n0 = sub * NPL;

    const T *xp = (const T *)a.x;
    const T *dp = (const T *)a.delta;
    const T *Bp = (const T *)a.Bt;
    const T *Cp = (const T *)a.Ct;
    const int64_t row = b * D + dc;
    const float dt = ld_act(dp, row);
    const float xv = ld_act(xp, row);

    float h[NPL], A2[NPL], Bv[NPL], Cv[NPL];
    float *sp = a.state + row * N + n0;
    ld_vec<NPL>(sp, h);
    ld_vec<NPL>(a.A + dc * N + n0, A2);
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        Bv[j] = ld_act(Bp, b * N + n0 + j);
        Cv[j] = ld_act(Cp, b * N + n0 + j);
    }
    const float dx = dt * xv;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        h[j] = __builtin_fmaf(fast_exp2(dt * (A2[j] * kLog2e)), h[j], dx * Bv[j]);
        acc = __builtin_fmaf(Cv[j], h[j], acc);
    }
    if (valid) st_vec<NPL>(sp, h);
    acc = group_sum<LPC>(acc);
    if (!valid || sub != 0) return;
    if (SKIP) acc = __builtin_fmaf(a.Dskip[d], xv, acc);
    if (GATE) acc *= silu(ld_act((const T *)a.z, row));
    st_act((T *)a.y, row, acc);
}

template <int N, int DT, bool GATE, bool SKIP>
hipError_t launch_step_typed(const StepArgs &a, hipStream_t s) {
    constexpr int NPL = N < 4 ? N : 4;
    constexpr int CPB = kStepBlock / (N / NPL);
    const dim3 grid((unsigned)((a.D + CPB - 1) / CPB * a.batch));
    hipLaunchKernelGGL((step_kernel<N, DT, GATE, SKIP>), grid, dim3(kStepBlock), 0, s, a);
    return hipGetLastError();
}

template <int N, int DT>
hipError_t launch_step_flags(const StepArgs &a, hipStream_t s) {
    const bool gate = a.z != nullptr, skip = a.Dskip != nullptr;
    if (gate && skip) return launch_step_typed<N, DT, true, true>(a, s);
    if (gate) return launch_step_typed<N, DT, true, false>(a, s);
    if (skip) return launch_step_typed<N, DT, false, true>(a, s);
    return launch_step_typed<N, DT, false, false>(a, s);
}

template <int N>
hipError_t launch_step_dtype(const StepArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch_step_flags<N, 0>(a, s) : launch_step_flags<N, 1>(a, s);
}

}  // namespace

hipError_t launch_step(const StepArgs &a, int N, int dtype, hipStream_t s) {
    switch (N) {
        case 1: return launch_step_dtype<1>(a, dtype, s);
        case 2: return launch_step_dtype<2>(a, dtype, s);
        case 4: return launch_step_dtype<4>(a, dtype, s);
        case 8: return launch_step_dtype<8>(a, dtype, s);
        case 16: return launch_step_dtype<16>(a, dtype, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
