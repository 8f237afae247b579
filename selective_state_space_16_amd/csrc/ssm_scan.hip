// Selective scan (S6) forward kernels for gfx950.
//
// Mapping: one lane owns one (batch row, channel) pair and keeps all N state
// values of that channel in registers; a wave covers 64 consecutive channels
// of one batch row, so the per-token vectors Bt[t,:] and Ct[t,:] are the same
// for every lane and are read once per wave through the scalar cache, while
// x, delta, z and y are read and written as contiguous 64-channel rows.
// The (batch, L, D, N) expanded state never leaves the registers ("Notas sobre
// Mamba", section "A varredura paralela ciente do hardware").
//
// Long sequences are cut into K chunks so that enough waves run at once. The
// recurrence h <- a*h + b composes associatively: applying the pairs of a
// chunk in order equals one pair (P, S) with P = prod a_t = exp(A * sum delta)
// and S = the chunk's end state from a zero start. Three launches:
//   1. summary: every chunk but the last computes S and sum(delta);
//   2. carry:   per (b, d, n), fold the chunk pairs in order to get each
//               chunk's carried-in state;
//   3. final:   every chunk rescans from its carried-in state, writes y, and
//               the last chunk writes state_out.
// With K = 1 only the final launch runs, from state_in.
//
// TRAP: the exponential-trapezoidal rule ("Notas sobre Mamba", section
// "Recorrência trapezoidal"): h = a h + (1 - lam) delta a v_prev + lam delta v
// with v = B x of this token and v_prev that of the previous one, taken as
// h = a (h + ((1 - lam) delta x_prev) B_prev) + (lam delta x) B. The pair
// composition is unchanged (a = exp(delta A)); a chunk's summary includes its
// first token's term in the input of the token before it, read from memory
// (or x_prev, B_prev for token 0).
//
// With conv_w, x is the raw input of the x branch ahead of the scan ("Notas
// sobre Mamba", section "O bloco Mamba"): each lane keeps the raw x of the
// three tokens before the current one and uses SiLU of the causal width-4
// convolution, rounded to the activation dtype, as x.
#include "ssm_common.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kWave = 64;
enum { kFinal = 0, kSummary = 1 };

template <int N, int DT, int MODE, bool GATE, bool SKIP, bool TRAP>
__global__ __launch_bounds__(kWave) void scan_chunk_kernel(ScanArgs a) {
    using T = typename Act<DT>::T;
    const int lane = threadIdx.x;
    const int64_t D = a.D, L = a.L;
    // flat grid: block id = (b * chunks + k) * channel_blocks + channel_block
    const int64_t nb = (D + kWave - 1) / kWave;
    const int64_t chunks = (MODE == kSummary) ? a.K - 1 : a.K;
    const int64_t bid = blockIdx.x;
    const int64_t d = (bid % nb) * kWave + lane;
    const int64_t k = (bid / nb) % chunks;
    const int64_t b = bid / (nb * chunks);
    const bool valid = d < D;
    const int64_t dc = valid ? d : D - 1;  // clamp so that every load stays in bounds
    const int64_t t0 = k * a.Lc;
    const int64_t t1 = (t0 + a.Lc < L) ? t0 + a.Lc : L;

    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = a.A[dc * N + n] * kLog2e;

    if (MODE == kSummary) {
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = 0.0f;
    } else if (a.K > 1) {
        const float *src = a.ws_state + ((b * a.K + k) * D + dc) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = src[n];
    } else if (a.state_in) {
        const float *src = a.state_in + (b * D + dc) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = src[n];
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = 0.0f;
    }

    const T *xp = (const T *)a.x;
    const T *dp = (const T *)a.delta;
    const T *zp = (const T *)a.z;
    const T *Bp = (const T *)a.Bt;
    const T *Cp = (const T *)a.Ct;
    T *yp = (T *)a.y;
    const float dskip = (SKIP && MODE == kFinal) ? a.Dskip[dc] : 0.0f;
    const float dtb = a.dt_bias ? a.dt_bias[dc] : 0.0f;  // bias of a raw step size

    // TRAP: x and Bt of the token before this one
    float xprev = 0.0f, Bprev[N];
#pragma unroll
    for (int n = 0; n < N; ++n) Bprev[n] = 0.0f;
    if constexpr (TRAP) {
        if (t0 > 0) {
            xprev = ld_act(xp, (b * L + t0 - 1) * D + dc);
            ld_row_uniform<N>(Bp, (b * L + t0 - 1) * N, Bprev);
        } else if (a.x_prev) {
            xprev = ld_act((const T *)a.x_prev, b * D + dc);
            ld_row_uniform<N>((const T *)a.B_prev, b * N, Bprev);
        }
    }

    // the x branch: taps, bias and the raw x of the three tokens before t0
    // (before token 0: conv_state, or zeros)
    const bool conv = a.conv_w != nullptr;
    float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cbias = 0.0f, xm[3] = {0.0f, 0.0f, 0.0f};
    if (conv) {
#pragma unroll
        for (int j = 0; j < 4; ++j) cw[j] = a.conv_w[dc * 4 + j];
        cbias = a.conv_b ? a.conv_b[dc] : 0.0f;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int64_t s = t0 - 3 + j;
            if (s >= 0) xm[j] = ld_act(xp, (b * L + s) * D + dc);
            else if (a.conv_state) xm[j] = ld_act((const T *)a.conv_state, (b * D + dc) * 3 + (s + 3));
        }
    }
    float dsum = 0.0f;
#pragma unroll 4
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t row = (b * L + t) * D + dc;
        float dt = ld_act(dp, row);
        if (a.delta_softplus) dt = act_round<DT>(softplus(dt + dtb));
        float xv = ld_act(xp, row);
        if (conv) {
            const float raw = xv;
            xv = act_round<DT>(conv_silu(cw[0], cw[1], cw[2], cw[3], cbias, xm[0], xm[1], xm[2], raw));
            xm[0] = xm[1];
            xm[1] = xm[2];
            xm[2] = raw;
        }
        float Bv[N];
        ld_row_uniform<N>(Bp, (b * L + t) * N, Bv);
        float dx = dt * xv;
        if constexpr (TRAP) {
            const float lm = ld_act((const T *)a.lam, row);
            const float px = (dt - lm * dt) * xprev;
            dx = lm * dt * xv;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                h[n] = __builtin_fmaf(px, Bprev[n], h[n]);
                Bprev[n] = Bv[n];
            }
            xprev = xv;
        }
        if (MODE == kSummary) {
            dsum += dt;
#pragma unroll
            for (int n = 0; n < N; ++n) h[n] = __builtin_fmaf(fast_exp2(dt * A2[n]), h[n], dx * Bv[n]);
        } else {
            float Cv[N];
            ld_row_uniform<N>(Cp, (b * L + t) * N, Cv);
            float acc = 0.0f;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                h[n] = __builtin_fmaf(fast_exp2(dt * A2[n]), h[n], dx * Bv[n]);
                acc = __builtin_fmaf(Cv[n], h[n], acc);
            }
            if (SKIP) acc = __builtin_fmaf(dskip, xv, acc);
            if (GATE) acc *= silu(ld_act(zp, row));
            if (valid) st_act(yp, row, acc);
        }
    }

    if (!valid) return;
    if (MODE == kSummary) {
        float *dst = a.ws_state + ((b * a.K + k) * D + d) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) dst[n] = h[n];
        a.ws_dsum[(b * a.K + k) * D + d] = dsum;
    } else if (k == a.K - 1 && a.state_out) {
        float *dst = a.state_out + (b * D + d) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) dst[n] = h[n];
    }
}

// Per (b, d, n): replace each chunk's summary S_k by the state carried into
// chunk k, folding h <- exp(A * sum delta_k) * h + S_k in chunk order.
template <int N>
__global__ __launch_bounds__(256) void scan_carry_kernel(ScanArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t D = a.D, K = a.K;
    if (i >= a.batch * D * N) return;
    const int64_t n = i % N;
    const int64_t d = (i / N) % D;
    const int64_t b = i / ((int64_t)N * D);
    const float A2 = a.A[d * N + n] * kLog2e;
    float carry = a.state_in ? a.state_in[i] : 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float *slot = a.ws_state + ((b * K + k) * D + d) * N + n;
        const float s = *slot;
        *slot = carry;
        if (k + 1 < K) carry = __builtin_fmaf(fast_exp2(A2 * a.ws_dsum[(b * K + k) * D + d]), carry, s);
    }
}

__global__ __launch_bounds__(256) void state_copy_kernel(const float *src, float *dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

template <int N, int DT, bool GATE, bool SKIP, bool TRAP>
hipError_t launch_typed(const ScanArgs &a, hipStream_t s) {
    const dim3 blk(kWave);
    const int64_t nb = (a.D + kWave - 1) / kWave;
    if (a.K > 1) {
        hipLaunchKernelGGL((scan_chunk_kernel<N, DT, kSummary, GATE, SKIP, TRAP>),
                           dim3((unsigned)(nb * (a.K - 1) * a.batch)), blk, 0, s, a);
        const int64_t total = a.batch * a.D * N;
        hipLaunchKernelGGL((scan_carry_kernel<N>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    }
    hipLaunchKernelGGL((scan_chunk_kernel<N, DT, kFinal, GATE, SKIP, TRAP>),
                       dim3((unsigned)(nb * a.K * a.batch)), blk, 0, s, a);
    return hipGetLastError();
}

template <int N, int DT, bool TRAP>
hipError_t launch_rule(const ScanArgs &a, hipStream_t s) {
    const bool gate = a.z != nullptr, skip = a.Dskip != nullptr;
    if (gate && skip) return launch_typed<N, DT, true, true, TRAP>(a, s);
    if (gate) return launch_typed<N, DT, true, false, TRAP>(a, s);
    if (skip) return launch_typed<N, DT, false, true, TRAP>(a, s);
    return launch_typed<N, DT, false, false, TRAP>(a, s);
}

template <int N, int DT>
hipError_t launch_flags(const ScanArgs &a, hipStream_t s) {
    return a.lam ? launch_rule<N, DT, true>(a, s) : launch_rule<N, DT, false>(a, s);
}

template <int N>
hipError_t launch_dtype(const ScanArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch_flags<N, 0>(a, s) : launch_flags<N, 1>(a, s);
}

}  // namespace

void scan_plan(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t *K, int64_t *Lc) {
    (void)N;
    // Aim for about 4096 waves in flight; never cut below 64 tokens per chunk.
    const int64_t waves = batch * ((D + kWave - 1) / kWave);
    int64_t k = waves > 0 ? (4096 + waves - 1) / waves : 1;
    const int64_t kmax = (L + 63) / 64;
    if (k > kmax) k = kmax;
    if (k < 1) k = 1;
    int64_t lc = (L + k - 1) / k;
    lc = (lc + 7) / 8 * 8;
    if (lc < 1) lc = 1;
    *Lc = lc;
    *K = (L + lc - 1) / lc;
    if (*K < 1) *K = 1;
}

hipError_t launch_scan(const ScanArgs &a, int N, int dtype, hipStream_t s) {
    switch (N) {
        case 1: return launch_dtype<1>(a, dtype, s);
        case 2: return launch_dtype<2>(a, dtype, s);
        case 4: return launch_dtype<4>(a, dtype, s);
        case 8: return launch_dtype<8>(a, dtype, s);
        case 16: return launch_dtype<16>(a, dtype, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_state_copy(const float *src, float *dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace ssm
