// Single-token recurrent decode step (S6) for gfx950.
//
// The step reads and rewrites the whole (batch, D, N) float state, so it is
// bound by memory traffic ("Notas sobre Mamba", section "Formulação MIMO":
// decode cost is governed by the state read and written each token).
//
// A wave serves 64 consecutive channels of kRows batch rows. Their state is
// one contiguous span of 64 * N floats per row, read and written as LPC = N /
// NPL wave-wide 16-byte accesses (NPL = min(N, 4) floats per lane): in access
// q, lane l holds states n0 = (l % LPC) * NPL .. + NPL of channel
// q * (64 / LPC) + l / LPC. The per-channel inputs (x, delta, z) and the output
// y move as one 64-lane access per row, lane l owning channel l; the lanes
// that work on a channel fetch its x and delta from lane l with ds_bpermute,
// and the channel's readout, summed over its LPC lanes with DPP quad
// permutes, comes back the same way. A is read once for the kRows rows, and
// every load of a row group is issued before the first use.
//
// MODE kConv adds the x branch ahead of the step ("Notas sobre Mamba",
// section "O bloco Mamba"): the lane that moves a channel's x reads the raw x
// of the three tokens before it from conv_state, uses SiLU of the causal
// width-4 convolution as x, and shifts this token's raw x into conv_state.
#include "ssm_common.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kStepBlock = 256;
constexpr int kWaveCh = 64;  // channels per wave
constexpr int kBlockCh = kWaveCh * (kStepBlock / 64);
constexpr int kRows = 2;  // batch rows per lane
constexpr unsigned kMaxGridY = 65535;

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

// NPL consecutive B or C values as one access. bfloat16 rows are kept as raw
// 16-bit patterns until use.
template <int NPL> struct Raw16;
template <> struct Raw16<1> { using T = uint16_t; };
template <> struct Raw16<2> { using T = uint32_t; };
template <> struct Raw16<4> { using T = uint2; };

template <int NPL, int DT> struct BcRaw {
    using T = typename Vec<NPL>::T;
    static __device__ __forceinline__ T load(const float *p) { return *(const T *)p; }
    static __device__ __forceinline__ void widen(const T &v, float (&r)[NPL]) { __builtin_memcpy(r, &v, sizeof(v)); }
};
template <int NPL> struct BcRaw<NPL, 1> {
    using T = typename Raw16<NPL>::T;
    static __device__ __forceinline__ T load(const uint16_t *p) { return *(const T *)p; }
    static __device__ __forceinline__ void widen(const T &v, float (&r)[NPL]) {
        uint16_t u[NPL];
        __builtin_memcpy(u, &v, sizeof(v));
#pragma unroll
        for (int j = 0; j < NPL; ++j) r[j] = __uint_as_float((uint32_t)u[j] << 16);
    }
};

// Sum over the LPC lanes of a group (LPC in {1, 2, 4}; groups are aligned quads
// or pairs inside a quad); every lane of the group gets the sum.
template <int LPC>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LPC >= 2)  // quad_perm [1,0,3,2]
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    if constexpr (LPC >= 4)  // quad_perm [2,3,0,1]
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    return v;
}

// Value of v in lane `src` of the wave.
__device__ __forceinline__ float from_lane(int src, float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src * 4, __builtin_bit_cast(int, v)));
}

// What the step computes besides the exponential-Euler update on an
// activated step size.
enum StepMode { kEuler = 0, kSoftplus = 1, kTrap = 2, kConv = 3 };

// Grid: x = block of kBlockCh channels, y = group of kRows batch rows
// (strided by gridDim.y when the groups outnumber kMaxGridY).
// MODE kSoftplus: delta holds the step size before its activation,
// softplus(delta + dt_bias). MODE kTrap: the exponential-trapezoidal rule
// ("Notas sobre Mamba", section "Recorrência trapezoidal"),
//   h = a h + (1 - lam) delta a v_prev + lam delta v,  a = exp(delta A),
// with v = B x of this token and v_prev = B_prev x_prev of the previous one
// (zero when x_prev and B_prev are not given), taken as
//   h = a (h + ((1 - lam) delta x_prev) B_prev) + (lam delta x) B.
// MODE kConv: as kSoftplus, with x before the block's convolution and SiLU.
template <int N, int DT, bool GATE, bool SKIP, int MODE>
__global__ __launch_bounds__(kStepBlock) void step_kernel(StepArgs a) {
    constexpr bool CONV = MODE == kConv, SP = MODE == kSoftplus || CONV, TRAP = MODE == kTrap;
    using T = typename Act<DT>::T;
    constexpr int NPL = N < 4 ? N : 4;
    constexpr int LPC = N / NPL;        // lanes per channel = accesses per row
    constexpr int CPA = kWaveCh / LPC;  // channels per access
    using BC = BcRaw<NPL, DT>;
    const int64_t D = a.D;
    const int l = threadIdx.x & 63;
    const int64_t cw = (int64_t)blockIdx.x * kBlockCh + (threadIdx.x >> 6) * kWaveCh;  // wave's first channel
    const int n0 = (l % LPC) * NPL;
    // Channel of this lane in access q, clamped into range for loads.
    int64_t chq[LPC];
    bool okq[LPC];
#pragma unroll
    for (int q = 0; q < LPC; ++q) {
        const int64_t c = cw + q * CPA + l / LPC;
        okq[q] = c < D;
        chq[q] = c < D ? c : D - 1;
    }
    const bool own_ok = cw + l < D;
    const int64_t own = own_ok ? cw + l : D - 1;  // channel whose x, delta, z and y this lane moves
    const T *xp = (const T *)a.x;
    const T *dp = (const T *)a.delta;
    const T *Bp = (const T *)a.Bt;
    const T *Cp = (const T *)a.Ct;
    const int64_t groups = (a.batch + kRows - 1) / kRows;

    float A2[LPC][NPL];
#pragma unroll
    for (int q = 0; q < LPC; ++q) ld_vec<NPL>(a.A + chq[q] * N + n0, A2[q]);
    const float ds = SKIP ? a.Dskip[own] : 0.0f;
    const float dtb = (SP && a.dt_bias) ? a.dt_bias[own] : 0.0f;  // bias of a raw step size
    // taps and bias of the convolution for the channel this lane moves
    float cwv[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cbias = 0.0f;
    if constexpr (CONV) {
        ld_vec<4>(a.conv_w + own * 4, cwv);
        cbias = a.conv_b ? a.conv_b[own] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < LPC; ++q)
#pragma unroll
        for (int j = 0; j < NPL; ++j) A2[q][j] *= kLog2e;

    for (int64_t g = blockIdx.y; g < groups; g += gridDim.y) {
        int64_t bc[kRows];
        bool bok[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int64_t b = g * kRows + r;
            bok[r] = b < a.batch;
            bc[r] = bok[r] ? b : a.batch - 1;
        }
        float h[kRows][LPC][NPL], xo[kRows], dto[kRows], zo[kRows], lo[kRows], xpo[kRows], cso[kRows][3];
        typename BC::T braw[kRows], craw[kRows], bpraw[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r)
#pragma unroll
            for (int q = 0; q < LPC; ++q) ld_vec<NPL>(a.state + (bc[r] * D + chq[q]) * N + n0, h[r][q]);
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int64_t row = bc[r] * D + own;
            xo[r] = ld_act(xp, row);
            dto[r] = ld_act(dp, row);
            if constexpr (SP) dto[r] = act_round<DT>(softplus(dto[r] + dtb));
            if (GATE) zo[r] = ld_act((const T *)a.z, row);
            braw[r] = BC::load(Bp + bc[r] * N + n0);
            craw[r] = BC::load(Cp + bc[r] * N + n0);
            if constexpr (CONV) {
#pragma unroll
                for (int j = 0; j < 3; ++j) cso[r][j] = ld_act((const T *)a.conv_state, row * 3 + j);
            }
            if constexpr (TRAP) {
                lo[r] = ld_act((const T *)a.lam, row);
                if (a.x_prev) {
                    xpo[r] = ld_act((const T *)a.x_prev, bc[r] * D + own);
                    bpraw[r] = BC::load((const T *)a.B_prev + bc[r] * N + n0);
                }
            }
        }

        if constexpr (CONV) {
            // x of this token from the branch's convolution; the raw x moves
            // into the window
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const float raw = xo[r];
                xo[r] = act_round<DT>(conv_silu(cwv[0], cwv[1], cwv[2], cwv[3], cbias, cso[r][0], cso[r][1],
                                                cso[r][2], raw));
                if (bok[r] && own_ok) {
                    T *cs = (T *)a.conv_state + (bc[r] * D + own) * 3;
                    st_act(cs, 0, cso[r][1]);
                    st_act(cs, 1, cso[r][2]);
                    st_act(cs, 2, raw);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            float Bv[NPL], Cv[NPL], Bpv[NPL], acc[LPC];
            BC::widen(braw[r], Bv);
            BC::widen(craw[r], Cv);
            if constexpr (TRAP) {
                if (a.x_prev) BC::widen(bpraw[r], Bpv);
            }
#pragma unroll
            for (int q = 0; q < LPC; ++q) {
                const int src = q * CPA + l / LPC;
                const float dt = LPC == 1 ? dto[r] : from_lane(src, dto[r]);
                const float xv = LPC == 1 ? xo[r] : from_lane(src, xo[r]);
                float s = 0.0f;
                if constexpr (TRAP) {
                    const float lm = LPC == 1 ? lo[r] : from_lane(src, lo[r]);
                    const float dx = lm * dt * xv;
                    if (a.x_prev) {
                        const float xp = LPC == 1 ? xpo[r] : from_lane(src, xpo[r]);
                        const float px = (dt - lm * dt) * xp;
#pragma unroll
                        for (int j = 0; j < NPL; ++j) h[r][q][j] = __builtin_fmaf(px, Bpv[j], h[r][q][j]);
                    }
#pragma unroll
                    for (int j = 0; j < NPL; ++j) {
                        h[r][q][j] = __builtin_fmaf(fast_exp2(dt * A2[q][j]), h[r][q][j], dx * Bv[j]);
                        s = __builtin_fmaf(Cv[j], h[r][q][j], s);
                    }
                } else {
                    const float dx = dt * xv;
#pragma unroll
                    for (int j = 0; j < NPL; ++j) {
                        h[r][q][j] = __builtin_fmaf(fast_exp2(dt * A2[q][j]), h[r][q][j], dx * Bv[j]);
                        s = __builtin_fmaf(Cv[j], h[r][q][j], s);
                    }
                }
                if (bok[r] && okq[q]) st_vec<NPL>(a.state + (bc[r] * D + chq[q]) * N + n0, h[r][q]);
                acc[q] = group_sum<LPC>(s);
            }
            // Channel l's sum sits in access l / CPA, lane (l % CPA) * LPC.
            float v = acc[0];
            if constexpr (LPC > 1) {
                const int src = (l % CPA) * LPC;
#pragma unroll
                for (int q = 0; q < LPC; ++q) {
                    const float t = from_lane(src, acc[q]);
                    v = l / CPA == q ? t : v;
                }
            }
            if (SKIP) v = __builtin_fmaf(ds, xo[r], v);
            if (GATE) v *= silu(zo[r]);
            if (bok[r] && own_ok) st_act((T *)a.y, bc[r] * D + own, v);
        }
    }
}

template <int N, int DT, bool GATE, bool SKIP, int MODE>
hipError_t launch_step_typed(const StepArgs &a, hipStream_t s) {
    const int64_t groups = (a.batch + kRows - 1) / kRows;
    if ((a.D + kBlockCh - 1) / kBlockCh > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((a.D + kBlockCh - 1) / kBlockCh), (unsigned)(groups < kMaxGridY ? groups : kMaxGridY));
    hipLaunchKernelGGL((step_kernel<N, DT, GATE, SKIP, MODE>), grid, dim3(kStepBlock), 0, s, a);
    return hipGetLastError();
}

template <int N, int DT, int MODE>
hipError_t launch_step_mode(const StepArgs &a, hipStream_t s) {
    const bool gate = a.z != nullptr, skip = a.Dskip != nullptr;
    if (gate && skip) return launch_step_typed<N, DT, true, true, MODE>(a, s);
    if (gate) return launch_step_typed<N, DT, true, false, MODE>(a, s);
    if (skip) return launch_step_typed<N, DT, false, true, MODE>(a, s);
    return launch_step_typed<N, DT, false, false, MODE>(a, s);
}

template <int N, int DT>
hipError_t launch_step_flags(const StepArgs &a, hipStream_t s) {
    if (a.lam) return launch_step_mode<N, DT, kTrap>(a, s);
    if (a.conv_w) return launch_step_mode<N, DT, kConv>(a, s);
    if (a.delta_softplus) return launch_step_mode<N, DT, kSoftplus>(a, s);
    return launch_step_mode<N, DT, kEuler>(a, s);
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
