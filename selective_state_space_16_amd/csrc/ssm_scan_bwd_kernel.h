#pragma once
// Gradient of the selective scan (S6) for gfx950: the kernels.
//
// The loss is sum(dy * y) + sum(dstate * state_out). Per (batch row b,
// channel d), with a_t = exp(delta_t A), h_t = a_t h_{t-1} + delta_t B_t x_t and
// the gradient G_t = dLoss/dh_t, the chain rule gives
//
//   G_t = C_t ds_t + a_{t+1} G_{t+1},        ds_t = dy_t silu(z_t),
//
// a linear recurrence run backwards in t. The states are recomputed rather
// than stored ("Notas sobre Mamba", section "A varredura paralela ciente do
// hardware": the backward recomputes the intermediate states), so nothing of
// size (batch, L, D, N) is written. The sequence is cut into chunks of 32
// tokens:
//   1. forward summaries: each chunk's end state from a zero start, and the
//      same at its inner 8-token block entries;
//   2. reverse summaries: the gradient each chunk sends into the state before
//      it from a zero gradient at its end (both summaries in one pass, with
//      each chunk's summed delta);
//   3. carries per (b, d, n) over the chunks: from state_in, the state
//      entering every chunk; from dstate, the gradient entering every chunk
//      from the tokens after it;
//   4. per chunk, from its entering state and gradient: the state entering
//      each block of 8 tokens (affine in the chunk's entering state), the
//      block's states again, then token by token backwards, every gradient.
//      Bt and Ct of the chunk, and with bfloat16 activations its x, delta, z
//      and dy of the block's channels, are staged in LDS first, so the token
//      loops never wait for a global load.
//      dB and dC sum over the channels: exchanges within each wave, then LDS
//      across the block's waves, one partial per block of channels; dA and dD
//      sum over (b, t): one partial per (b, chunk);
//   5. the partials are summed, in a fixed order.
//
// TRAP: the exponential-trapezoidal rule ("Notas sobre Mamba", section
// "Recorrência trapezoidal"), h_t = a_t (h_{t-1} + (1 - lam_t) delta_t v_{t-1})
// + lam_t delta_t v_t with v_t = B_t x_t. The state's gradient runs as above;
// v_t feeds h_t and h_{t+1}, so its gradient takes lam_t delta_t G_t plus
// (1 - lam_{t+1}) delta_{t+1} a_{t+1} G_{t+1}, carried from token to token.
#include "ssm_common.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kBwdThreads = 256;
constexpr int kSub = kBwdSub;  // tokens per recomputed block

// The recurrence the gradient goes through: the exponential-Euler rule with
// the step size given, or given before its activation, or the
// exponential-trapezoidal rule.
enum BwdMode { kBwdEuler = 0, kBwdSoftplus = 1, kBwdTrap = 2 };

// The step size of a token: given, or softplus(raw + bias) rounded to the
// activation dtype, as the forward scan computes it.
template <int DT, typename T>
__device__ __forceinline__ float delta_at(const T *dp, int64_t row, bool sp, float dtb) {
    const float v = ld_act(dp, row);
    return sp ? act_round<DT>(softplus(v + dtb)) : v;
}

// silu(z) and its derivative sigmoid(z) (1 + z (1 - sigmoid(z))).
__device__ __forceinline__ void silu_and_grad(float z, float &g, float &dg) {
    const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp2(-z * kLog2e));
    g = z * sg;
    dg = sg * (1.0f + z * (1.0f - sg));
}

// v from lane (lane ^ BIT): DPP lane moves inside rows of 16 lanes for BIT 1,
// 2 (quad permutes) and 8 (a rotation by 8), swizzles inside 32 lanes for 4
// and 16, a permute for 32. Every lane has a source, so the DPP moves need no
// initial value.
template <int BIT>
__device__ __forceinline__ float xor_lane(float v) {
    const int x = __float_as_int(v);
    if constexpr (BIT == 1) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    } else if constexpr (BIT == 2) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    } else if constexpr (BIT == 4) {
        return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x101F));  // and 31, xor 4
    } else if constexpr (BIT == 8) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));  // row_ror:8
    } else if constexpr (BIT == 16) {
        return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x401F));  // and 31, xor 16
    } else {
        return __shfl_xor(v, BIT);
    }
}

// u[i] += fp * v[i + 4] of lane ^ 1 (i < 4): one DPP multiply-add each. The
// s_nop covers the wait a DPP source written by the previous VALU instruction
// needs (the compiler does not fold the move into a multiply-add itself).
__device__ __forceinline__ void fmac_quad_neighbour(float (&u)[4], const float (&v)[8], float fp) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "+v"(u[0]), "+v"(u[1]), "+v"(u[2]), "+v"(u[3])
        : "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(fp));
}

// One halving exchange of wave_sum_vec and the ones after it: lanes with bit
// BIT set keep the upper HALF elements of the current vector, the others the
// lower HALF, each adding its partner's (lane ^ BIT) copy of the kept half.
// Recursion on constants keeps every array index a compile-time constant.
template <int HALF, int BIT, int N>
__device__ __forceinline__ void halve(float (&v)[N], int lane) {
    if constexpr (HALF >= 1) {
        const bool upper = (lane & BIT) != 0;
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            const float send = upper ? v[i] : v[i + HALF];
            const float keep = upper ? v[i + HALF] : v[i];
            v[i] = keep + xor_lane<BIT>(send);
        }
        halve<HALF / 2, BIT * 2>(v, lane);
    }
}

template <int BIT, int SPAN>
__device__ __forceinline__ float fold(float s) {
    if constexpr (BIT < SPAN) {
        return fold<BIT * 2, SPAN>(s + xor_lane<BIT>(s));
    } else {
        return s;
    }
}

// Sum of v[0..N) over the lanes of a wave that share bit SPAN and above
// (SPAN = 64: the whole wave). The halving exchanges leave lane l with the
// sum, over N lanes, of one element, named by the bits of l below log2(N);
// the remaining exchanges add the lanes that hold the same element. Returns
// that sum.
template <int N, int SPAN>
__device__ __forceinline__ float wave_sum_vec(float (&v)[N], int lane) {
    halve<N / 2, 1>(v, lane);
    return fold<N, SPAN>(v[0]);
}

// The element of v that wave_sum_vec<N, SPAN> leaves in lane `lane`.
template <int N>
__device__ __forceinline__ int wave_sum_index(int lane) {
    int idx = 0;
#pragma unroll
    for (int s = 0; (N >> (s + 1)) >= 1; ++s)
        if (lane & (1 << s)) idx += N >> (s + 1);
    return idx;
}

// 1+2. the summaries of every chunk k, in one forward pass over its tokens:
// its end state from a zero start (S_k, for k < K - 1), the gradient it sends
// into the state before it from a zero gradient at its end (R_k, for k >= 1),
// and its summed delta. In token order, R_k is the sum of C_t ds_t times the
// product of a_s over the chunk's tokens up to and including t, so the decay
// a_t of each token serves both summaries.
template <int N, int DT, bool GATE, int MODE>
__global__ __launch_bounds__(kBwdThreads) void bwd_summary_kernel(BwdArgs a) {
    using T = typename Act<DT>::T;
    const int64_t D = a.D, L = a.L, K = a.K;
    // flat grid: block id = (b * K + k) * channel_blocks + channel_block
    const int64_t nb = (D + kBwdThreads - 1) / kBwdThreads, bid = blockIdx.x;
    const int64_t d = (bid % nb) * kBwdThreads + threadIdx.x;
    const int64_t k = (bid / nb) % K, b = bid / (nb * K);
    const bool valid = d < D;
    const int64_t dc = valid ? d : D - 1;
    const int64_t t0 = k * kBwdChunk, t1 = t0 + kBwdChunk < L ? t0 + kBwdChunk : L;
    float A2[N], h[N], P[N], R[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[dc * N + n] * kLog2e;
        h[n] = 0.0f;
        P[n] = 1.0f;
        R[n] = 0.0f;
    }
    const T *xp = (const T *)a.x, *dp = (const T *)a.delta, *zp = (const T *)a.z, *gp = (const T *)a.dy;
    const T *Bp = (const T *)a.Bt, *Cp = (const T *)a.Ct;
    constexpr bool sp = MODE == kBwdSoftplus, TRAP = MODE == kBwdTrap;
    const float dtb = (sp && a.dt_bias) ? a.dt_bias[dc] : 0.0f;
    // TRAP: x and Bt of the token before the chunk (before token 0: x_prev, B_prev)
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
    float dsum = 0.0f;
    // Tokens go in groups of GS (a divisor of the block size). The per-lane
    // loads of a group (x, delta, dy, z, lam) are issued one group ahead, so
    // that the loop waits for memory once per group rather than once per
    // token; tokens past the chunk's end read its last token and are not used.
    // Four tokens measured best on the large layer (groups of eight raised the
    // registers to 158 and cost occupancy); the trapezoidal rule, which keeps
    // one more vector per state, takes two.
    constexpr int GS = TRAP ? 2 : 4;
    static_assert(kSub % GS == 0, "block entries fall on group starts");
    float gx[GS], gd[GS], gg[GS], gz[GS], gl[GS];
    auto load_group = [&](int64_t tg, float (&ox)[GS], float (&od)[GS], float (&og)[GS], float (&oz)[GS],
                          float (&ol)[GS]) {
#pragma unroll
        for (int u = 0; u < GS; ++u) {
            const int64_t t = tg + u < t1 ? tg + u : t1 - 1;
            const int64_t row = (b * L + t) * D + dc;
            ox[u] = ld_act(xp, row);
            od[u] = ld_act(dp, row);
            og[u] = ld_act(gp, row);
            oz[u] = GATE ? ld_act(zp, row) : 0.0f;
            ol[u] = TRAP ? ld_act((const T *)a.lam, row) : 0.0f;
        }
    };
    load_group(t0, gx, gd, gg, gz, gl);
    for (int64_t tg = t0; tg < t1; tg += GS) {
        if (tg > t0 && (tg - t0) % kSub == 0 && valid) {
            // a block entry inside the chunk: the state so far from a zero
            // chunk start, and the delta summed so far
            const int64_t j = (tg - t0) / kSub - 1;
            float *dst = a.ckp + (((b * K + k) * kBwdCk + j) * D + d) * N;
#pragma unroll
            for (int n = 0; n < N; ++n) dst[n] = h[n];
            a.ckd[((b * K + k) * kBwdCk + j) * D + d] = dsum;
        }
        float cx[GS], cd[GS], cg[GS], cz[GS], cl[GS];
#pragma unroll
        for (int u = 0; u < GS; ++u) {
            cx[u] = gx[u];
            cd[u] = gd[u];
            cg[u] = gg[u];
            cz[u] = gz[u];
            cl[u] = gl[u];
        }
        if (tg + GS < t1) load_group(tg + GS, gx, gd, gg, gz, gl);
#pragma unroll
        for (int u = 0; u < GS; ++u) {
            const int64_t t = tg + u;
            if (t >= t1) break;
            const float dt = sp ? act_round<DT>(softplus(cd[u] + dtb)) : cd[u], xv = cx[u];
            float dtx = dt * xv, mux = 0.0f;
            if constexpr (TRAP) {  // h = a (h + (1 - lam) delta v_{t-1}) + lam delta v_t
                const float lm = cl[u];
                mux = (dt - lm * dt) * xprev;
                dtx = lm * dt * xv;
                xprev = xv;
            }
            float ds = cg[u];
            if (GATE) {
                float g, dg;
                silu_and_grad(cz[u], g, dg);
                ds *= g;
            }
            float Bv[N], Cv[N];
            ld_row_uniform<N>(Bp, (b * L + t) * N, Bv);
            ld_row_uniform<N>(Cp, (b * L + t) * N, Cv);
            dsum += dt;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const float av = fast_exp2(dt * A2[n]);
                if constexpr (TRAP) {
                    h[n] = __builtin_fmaf(av, __builtin_fmaf(mux, Bprev[n], h[n]), dtx * Bv[n]);
                    Bprev[n] = Bv[n];
                } else {
                    h[n] = __builtin_fmaf(av, h[n], dtx * Bv[n]);
                }
                P[n] *= av;
                R[n] = __builtin_fmaf(P[n] * Cv[n], ds, R[n]);
            }
        }
    }
    if (!valid) return;
    const int64_t o = ((b * K + k) * D + d) * N;
    if (k + 1 < K) {
#pragma unroll
        for (int n = 0; n < N; ++n) a.hst[o + n] = h[n];
    }
    if (k > 0) {
#pragma unroll
        for (int n = 0; n < N; ++n) a.gq[o + n] = R[n];
    }
    a.dsum[(b * K + k) * D + d] = dsum;
}

// 3. the carries, per (b, d, n): in chunk order, the state entering each chunk
// (from state_in: h <- exp(A sum delta_k) h + S_k); in reverse chunk order,
// the gradient entering each chunk from its end (from dstate: q <- R_k +
// exp(A sum delta_k) q). Each summary slot is replaced by its carry.
template <int N>
__global__ __launch_bounds__(256) void bwd_carry_kernel(BwdArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t D = a.D, K = a.K;
    if (i >= a.batch * D * N) return;
    const int64_t n = i % N, d = (i / N) % D, b = i / ((int64_t)N * D);
    const float A2 = a.A[d * N + n] * kLog2e;
    const int64_t base = (b * K * D + d) * N + n, kstride = D * N;
    const float *ds = a.dsum + b * K * D + d;
    // four chunks per step: their loads first, then the dependent chain
    float h = a.state_in ? a.state_in[i] : 0.0f;
    for (int64_t k0 = 0; k0 < K; k0 += 4) {
        float sv[4], dv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t k = k0 + u;
            sv[u] = k + 1 < K ? a.hst[base + k * kstride] : 0.0f;
            dv[u] = k + 1 < K ? ds[k * D] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t k = k0 + u;
            if (k < K) {
                a.hst[base + k * kstride] = h;
                h = __builtin_fmaf(fast_exp2(A2 * dv[u]), h, sv[u]);
            }
        }
    }
    float q = a.dstate ? a.dstate[i] : 0.0f;
    for (int64_t k0 = K - 1; k0 >= 0; k0 -= 4) {
        float rv[4], dv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t k = k0 - u;
            rv[u] = k > 0 ? a.gq[base + k * kstride] : 0.0f;
            dv[u] = k > 0 ? ds[k * D] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t k = k0 - u;
            if (k >= 0) {
                a.gq[base + k * kstride] = q;
                q = __builtin_fmaf(fast_exp2(A2 * dv[u]), q, rv[u]);
            }
        }
    }
}

// 4. the gradients of one chunk, for one batch row and a block of channels.
// A lane owns NP = bwd_np(N) state elements of a channel: all of them when
// N <= 8 (4 for the trapezoidal rule); otherwise N / NP lanes, SPAN lanes
// apart in the wave, share a channel, so that the recomputed states of 8
// tokens fit in registers, and their per-channel sums meet through lane
// exchanges. Bt and Ct of the chunk are staged in LDS.
template <int N, int DT, bool GATE, bool SKIP, int MODE>
__global__ __launch_bounds__(kBwdThreads) void bwd_chunk_kernel(BwdArgs a) {
    using T = typename Act<DT>::T;
    constexpr int NP = bwd_np(N, MODE == kBwdTrap);  // state elements per lane
    constexpr int R = N / NP;                // lanes per channel
    constexpr int SPAN = 64 / R;             // channels per wave
    constexpr int CPB = kBwdThreads / R;     // channels per block
    constexpr int NCK = kBwdChunk / kSub;    // checkpoints per chunk
    constexpr int NW = kBwdThreads / 64;     // waves per block
    // row j + 1: token t0 + j; row 0: the token before the chunk (TRAP)
    __shared__ float sBC[2][kBwdChunk + 1][N];  // Bt rows, then Ct rows
    float(&sB)[kBwdChunk + 1][N] = sBC[0];
    float(&sC)[kBwdChunk + 1][N] = sBC[1];
    constexpr int kCt = (kBwdChunk + 1) * N;  // from a Bt element to the Ct element of its row
    __shared__ float ck[NCK][NP][kBwdThreads];   // state entering each block of kSub tokens
    __shared__ float red[2][NW][kSub][N];        // per-wave sums of dCt, dBt
    // bfloat16: the chunk's x, delta, z, dy (and lam) of the block's channels,
    // staged once with coalesced loads, so that the token loops read LDS rather
    // than wait for a global load per token
    constexpr bool STG = DT == 1;
    constexpr int NA = MODE == kBwdTrap ? 5 : 4;
    __shared__ T sA[STG ? NA : 1][STG ? kBwdChunk : 1][STG ? CPB : 1];
    const int64_t D = a.D, L = a.L, K = a.K;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = R == 1 ? 0 : lane / SPAN, cl = lane % SPAN;
    // flat grid: block id = (b * K + k) * channel_blocks + channel_block
    const int64_t nb = (D + CPB - 1) / CPB, bid = blockIdx.x;
    const int64_t cb = bid % nb, k = (bid / nb) % K, b = bid / (nb * K);
    const int64_t d = cb * CPB + w * SPAN + cl;
    const bool valid = d < D;
    const int64_t dc = valid ? d : D - 1;
    const int64_t t0 = k * kBwdChunk, t1 = t0 + kBwdChunk < L ? t0 + kBwdChunk : L;
    const int cnt_chunk = (int)(t1 - t0);
    const T *xp = (const T *)a.x, *dp = (const T *)a.delta, *zp = (const T *)a.z, *gp = (const T *)a.dy;
    constexpr bool sp = MODE == kBwdSoftplus, TRAP = MODE == kBwdTrap;
    const float dtb = (sp && a.dt_bias) ? a.dt_bias[dc] : 0.0f;
    const T *lp = (const T *)a.lam;
    for (int i = tid; i < (kBwdChunk + 1) * N; i += kBwdThreads) {
        const int jj = i / N, n = i % N;
        float bv = 0.0f, cv = 0.0f;
        if (jj >= 1 && jj - 1 < cnt_chunk) {
            const int64_t o = (b * L + t0 + jj - 1) * N + n;
            bv = ld_act((const T *)a.Bt, o);
            cv = ld_act((const T *)a.Ct, o);
        } else if (TRAP && jj == 0) {
            if (t0 > 0) bv = ld_act((const T *)a.Bt, (b * L + t0 - 1) * N + n);
            else if (a.B_prev) bv = ld_act((const T *)a.B_prev, b * N + n);
        }
        sB[jj][n] = bv;
        sC[jj][n] = cv;
    }
    const int64_t ch0 = cb * CPB;  // first channel of the block
    const int nch = (int)(D - ch0 < CPB ? D - ch0 : CPB);  // channels of the block that exist
    if constexpr (STG) {
        // thread (c, j0): channel c of the block (the last existing one past D),
        // tokens j0, j0 + 256 / CPB, ...; a wave reads consecutive channels
        const int c = tid % CPB, cc = c < nch ? c : nch - 1;
        const int64_t col = ch0 + cc;
        for (int j = tid / CPB; j < cnt_chunk; j += kBwdThreads / CPB) {
            const int64_t row = (b * L + t0 + j) * D + col;
            sA[0][j][c] = xp[row];
            sA[1][j][c] = dp[row];
            if (GATE) sA[2][j][c] = zp[row];
            sA[3][j][c] = gp[row];
            if constexpr (MODE == kBwdTrap) sA[NA - 1][j][c] = lp[row];
        }
    }
    // this lane's channel in the staged rows (past D: the last existing one)
    const int cws = valid ? w * SPAN + cl : nch - 1;
    auto act = [&](int arr, int tl) -> float {
        return STG ? __uint_as_float((uint32_t)sA[arr][tl][cws] << 16) : 0.0f;
    };
    // TRAP: x of the token before token t (x_prev before token 0; none: 0)
    auto x_before = [&](int64_t t) -> float {
        if (t > 0) return ld_act(xp, (b * L + t - 1) * D + dc);
        return a.x_prev ? ld_act((const T *)a.x_prev, b * D + dc) : 0.0f;
    };
    const int n0 = r * NP;  // first state element of this lane
    // With NP = 8, odd lanes hold their upper four elements first: position i
    // of every per-lane state vector is element sx[i] = n0 + (i ^ own). Lanes
    // l and l ^ 1 then hold the same element at positions i and i + 4, so the
    // first halving of the channel sums adds the partner's upper half with no
    // select.
    constexpr bool SWQ = NP == 8;
    const int own = SWQ ? (lane & 1) * 4 : 0;
    int sx[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) sx[i] = n0 + (i ^ own);
    float A2[NP], h[NP], G[NP], Gb[NP];
    // TRAP: Gb = (1 - lam) delta a G of the token after: the gradient of this
    // token's input through the next token's update; after the chunk, that of
    // its first token, whose a G is the gradient entering from the end
    float mu1 = 0.0f;
    if (TRAP && t1 < L) {
        const int64_t row1 = (b * L + t1) * D + dc;
        const float dt1 = ld_act(dp, row1);
        mu1 = dt1 - ld_act(lp, row1) * dt1;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        A2[i] = a.A[dc * N + sx[i]] * kLog2e;
        h[i] = a.hst[((b * K + k) * D + dc) * N + sx[i]];
        G[i] = a.gq[((b * K + k) * D + dc) * N + sx[i]];
        Gb[i] = mu1 * G[i];
    }
    __syncthreads();
    // forward through the chunk up to its last block, keeping the state
    // entering each block
    // the state entering each block: the chunk's entering state h carried
    // through exp(A sum delta) plus the block entry's state from a zero chunk
    // start (both from the summary pass: the recurrence is affine in h)
    const int nblk = (cnt_chunk + kSub - 1) / kSub;
#pragma unroll
    for (int i = 0; i < NP; ++i) ck[0][i][tid] = h[i];
    for (int j = 1; j < nblk; ++j) {
        const int64_t o = ((b * K + k) * kBwdCk + j - 1) * D + dc;
        const float cs = a.ckd[o];
#pragma unroll
        for (int i = 0; i < NP; ++i)
            ck[j][i][tid] = __builtin_fmaf(fast_exp2(cs * A2[i]), h[i], a.ckp[o * N + sx[i]]);
    }
    float dA[NP], dD = 0.0f, dT = 0.0f;
#pragma unroll
    for (int i = 0; i < NP; ++i) dA[i] = 0.0f;
    const float dsk = SKIP ? a.Dskip[dc] : 0.0f;
    // the element whose sum over the wave's channels chan_sum leaves in this lane
    const int elem = SWQ ? n0 + own + wave_sum_index<4>(cl >> 1) : n0 + wave_sum_index<NP>(cl);
    // sums over the wave's channels of f times a per-lane state vector v
    // (position order). With SWQ the first halving takes the neighbour's
    // upper half times its factor in one multiply-add each.
    auto chan_sum = [&](const float(&v)[NP], float f) -> float {
        if constexpr (SWQ) {
            float u[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = v[i] * f;
            fmac_quad_neighbour(u, v, xor_lane<1>(f));
            halve<2, 2>(u, lane);
            return fold<8, SPAN>(u[0]);
        } else {
            float t[NP];
#pragma unroll
            for (int i = 0; i < NP; ++i) t[i] = v[i] * f;
            return wave_sum_vec<NP, SPAN>(t, lane);
        }
    };
    for (int blk = nblk - 1; blk >= 0; --blk) {
        const int s0 = blk * kSub;
        const int cnt = cnt_chunk - s0 < kSub ? cnt_chunk - s0 : kSub;
        // states of the block: hb[j] = state entering token s0 + j; with
        // bfloat16 activations also ea[j][i], the decay of token s0 + j, kept
        // for the reverse walk (float32 recomputes it, and its lower register
        // count keeps three waves per SIMD)
        float hb[kSub + 1][NP], ea[STG ? kSub : 1][NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) hb[0][i] = ck[blk][i][tid];
        float xpr = TRAP ? (STG && s0 > 0 ? act(0, s0 - 1) : x_before(t0 + s0)) : 0.0f;
        // Bt of row s0 + u at position i of the lane: brow(i, u * N); Ct: brow(i, kCt + u * N)
        const float *bq[(NP + 3) / 4];
#pragma unroll
        for (int q = 0; q < (NP + 3) / 4; ++q) bq[q] = &sBC[0][0][0] + s0 * N + n0 + ((4 * q) ^ own);
        auto brow = [&](int i, int off) -> float { return bq[i / 4][off + (i % 4)]; };
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
            if (j < cnt) {
                const int64_t row = (b * L + t0 + s0 + j) * D + dc;
                float dt, xv;
                if constexpr (STG) {
                    const float rv = act(1, s0 + j);
                    dt = sp ? act_round<DT>(softplus(rv + dtb)) : rv;
                    xv = act(0, s0 + j);
                } else {
                    dt = delta_at<DT>(dp, row, sp, dtb);
                    xv = ld_act(xp, row);
                }
                if constexpr (TRAP) {
                    const float lm = STG ? act(NA - 1, s0 + j) : ld_act(lp, row);
                    const float mux = (dt - lm * dt) * xpr, dx = lm * dt * xv;
#pragma unroll
                    for (int i = 0; i < NP; ++i) {
                        const float e = fast_exp2(dt * A2[i]);
                        if constexpr (STG) ea[j][i] = e;
                        hb[j + 1][i] = __builtin_fmaf(e, __builtin_fmaf(mux, brow(i, j * N), hb[j][i]),
                                                      dx * brow(i, (j + 1) * N));
                    }
                    xpr = xv;
                } else {
                    const float dx = dt * xv;
#pragma unroll
                    for (int i = 0; i < NP; ++i) {
                        const float e = fast_exp2(dt * A2[i]);
                        if constexpr (STG) ea[j][i] = e;
                        hb[j + 1][i] = __builtin_fmaf(e, hb[j][i], dx * brow(i, (j + 1) * N));
                    }
                }
            }
        }
        (void)xpr;
#pragma unroll
        for (int j = kSub - 1; j >= 0; --j) {
            if (j >= cnt) continue;
            const int tl = s0 + j;
            const int64_t row = (b * L + t0 + tl) * D + dc;
            const float raw = STG ? act(1, tl) : ld_act(dp, row), xv = STG ? act(0, tl) : ld_act(xp, row);
            const float dyv = STG ? act(3, tl) : ld_act(gp, row);
            const float dt = sp ? act_round<DT>(softplus(raw + dtb)) : raw;
            float gate = 1.0f, dgate = 0.0f;
            if (GATE) silu_and_grad(STG ? act(2, tl) : ld_act(zp, row), gate, dgate);
            const float ds = valid ? dyv * gate : 0.0f;
            const float xvv = valid ? xv : 0.0f;
            // TRAP: the token before, its weight (1 - lam) delta, and this token's lam delta
            float lm = 0.0f, xpv = 0.0f, mu = 0.0f, gam = dt;
            if constexpr (TRAP) {
                lm = STG ? act(NA - 1, tl) : ld_act(lp, row);
                xpv = STG && tl > 0 ? act(0, tl - 1) : x_before(t0 + tl);
                mu = dt - lm * dt;
                gam = lm * dt;
            }
            const float mux = mu * xpv;
            // Ga = a G is the gradient of h_{t-1}; gah = Ga (h_{t-1} + (1 - lam) delta v_{t-1});
            // d(delta) takes sum(gah A), and x sum(G B) (Euler) or the trapezoid's terms
            // dCt takes ds times the state, dBt x times the input's gradient
            // (Euler: delta x times G), summed over channels below
            float pre = 0.0f, gaa = 0.0f, gb = 0.0f, gbb = 0.0f, gav = 0.0f, gin[NP];
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const float Cv = brow(i, kCt + (j + 1) * N), Bv = brow(i, (j + 1) * N);
                pre = __builtin_fmaf(Cv, hb[j + 1][i], pre);
                G[i] = __builtin_fmaf(Cv, ds, G[i]);
                gb = __builtin_fmaf(G[i], Bv, gb);
                if constexpr (TRAP) {
                    gin[i] = __builtin_fmaf(gam, G[i], Gb[i]);  // gradient of v_t = B_t x_t
                    gbb = __builtin_fmaf(Gb[i], Bv, gbb);
                } else {
                    gin[i] = G[i];
                }
                G[i] *= STG ? ea[STG ? j : 0][i] : fast_exp2(dt * A2[i]);  // the gradient of h_{t-1}
                float hp = hb[j][i];
                if constexpr (TRAP) {
                    const float Bp = brow(i, j * N);
                    hp = __builtin_fmaf(mux, Bp, hp);
                    gav = __builtin_fmaf(G[i], Bp, gav);
                    Gb[i] = mu * G[i];
                }
                const float gah = G[i] * hp;
                gaa = __builtin_fmaf(gah, A2[i], gaa);
                dA[i] = __builtin_fmaf(gah, dt, dA[i]);
            }
            if (R > 1) {  // the channel's other state elements, in the other lanes
                pre = fold<SPAN, 64>(pre);
                gaa = fold<SPAN, 64>(gaa);
                gb = fold<SPAN, 64>(gb);
                if constexpr (TRAP) {
                    gbb = fold<SPAN, 64>(gbb);
                    gav = fold<SPAN, 64>(gav);
                }
            }
            float gdt, gx;
            if constexpr (TRAP) {
                // d(delta) = sum Ga A p + (1 - lam) x_{t-1} sum Ga B_{t-1} + lam x sum G B
                gdt = __builtin_fmaf(gaa, kLn2, __builtin_fmaf((1.0f - lm) * xpv, gav, lm * xv * gb));
                gx = __builtin_fmaf(gam, gb, gbb);
            } else {
                gdt = __builtin_fmaf(gaa, kLn2, gb * xv);
                gx = gb * dt;
            }
            if (SKIP) {
                pre = __builtin_fmaf(dsk, xv, pre);
                gx = __builtin_fmaf(ds, dsk, gx);
            }
            dD = __builtin_fmaf(ds, xv, dD);
            if (valid && r == 0) {
                st_act((T *)a.dx, row, gx);
                // through the activation: d softplus(u) / du = sigmoid(u)
                const float g = sp ? gdt * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-(raw + dtb) * kLog2e)) : gdt;
                dT += g;
                st_act((T *)a.ddelta, row, g);
                if (GATE) st_act((T *)a.dz, row, dyv * pre * dgate);
                if (TRAP) st_act((T *)a.dlam, row, dt * (xv * gb - xpv * gav));
            }
            const float sc = chan_sum(hb[j + 1], ds);
            const float sb = chan_sum(gin, TRAP ? xvv : dt * xvv);
            if (cl < NP) {
                red[0][w][j][elem] = sc;
                red[1][w][j][elem] = sb;
            }
        }
        __syncthreads();
        // the block's sums over its channels, one partial per channel block
        for (int i = tid; i < 2 * kSub * N; i += kBwdThreads) {
            const int which = i / (kSub * N), j = (i / N) % kSub, n = i % N;
            if (j < cnt) {
                float sum = 0.0f;
#pragma unroll
                for (int v = 0; v < NW; ++v) sum += red[which][v][j][n];
                float *dst = which == 0 ? a.pdC : a.pdB;
                dst[((cb * a.batch + b) * L + t0 + s0 + j) * N + n] = sum;
            }
        }
        __syncthreads();
    }
    if constexpr (TRAP) {
        // the token before token 0: its input's gradient is Gb after token 0
        if (k == 0 && a.dx_prev) {
            const float xp0 = valid ? ld_act((const T *)a.x_prev, b * D + dc) : 0.0f;
            float gp = 0.0f;
#pragma unroll
            for (int i = 0; i < NP; ++i) gp = __builtin_fmaf(Gb[i], sB[0][sx[i]], gp);
            if (R > 1) gp = fold<SPAN, 64>(gp);
            if (valid && r == 0) st_act((T *)a.dx_prev, b * D + d, gp);
            const float sb = chan_sum(Gb, xp0);
            if (cl < NP) red[1][w][0][elem] = sb;
            __syncthreads();
            for (int n = tid; n < N; n += kBwdThreads) {
                float sum = 0.0f;
#pragma unroll
                for (int v = 0; v < NW; ++v) sum += red[1][v][0][n];
                a.pdBp[(cb * a.batch + b) * N + n] = sum;
            }
        }
    }
    if (!valid) return;
#pragma unroll
    for (int i = 0; i < NP; ++i) a.pdA[((b * K + k) * D + d) * N + sx[i]] = dA[i];
    if (r == 0) {
        a.pdD[(b * K + k) * D + d] = dD;
        a.pdT[(b * K + k) * D + d] = dT;
    }
    if (k == 0 && a.dstate_in) {
#pragma unroll
        for (int i = 0; i < NP; ++i) a.dstate_in[(b * D + d) * N + sx[i]] = G[i];
    }
}

// 5. the sums of the partials, in a fixed order (partial 0 first), eight
// loads in flight per step.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float *part, int64_t nparts, int64_t stride,
                                                         float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float s = 0.0f;
    int64_t p = 0;
    for (; p + 8 <= nparts; p += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[(p + u) * stride + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; p < nparts; ++p) s += part[p * stride + i];
    out[i] = s;
}

template <int N, int DT, bool GATE, bool SKIP, int MODE>
hipError_t launch_bwd_typed(const BwdArgs &a, hipStream_t s) {
    const int64_t D = a.D, K = a.K;
    const int64_t nb = (D + kBwdThreads - 1) / kBwdThreads;
    hipLaunchKernelGGL((bwd_summary_kernel<N, DT, GATE, MODE>), dim3((unsigned)(nb * K * a.batch)), dim3(kBwdThreads),
                       0, s, a);
    const int64_t total = a.batch * D * N;
    hipLaunchKernelGGL((bwd_carry_kernel<N>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
    const int64_t ncb = bwd_channel_blocks(D, N, MODE == kBwdTrap);
    hipLaunchKernelGGL((bwd_chunk_kernel<N, DT, GATE, SKIP, MODE>), dim3((unsigned)(ncb * K * a.batch)),
                       dim3(kBwdThreads), 0, s, a);
    const int64_t bln = a.batch * a.L * N;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((bln + 255) / 256)), dim3(256), 0, s, a.pdB, ncb, bln,
                       a.dBt, bln);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((bln + 255) / 256)), dim3(256), 0, s, a.pdC, ncb, bln,
                       a.dCt, bln);
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((D * N + 255) / 256)), dim3(256), 0, s, a.pdA,
                       a.batch * K, D * N, a.dA, D * N);
    if (a.dDskip)
        hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((D + 255) / 256)), dim3(256), 0, s, a.pdD, a.batch * K,
                           D, a.dDskip, D);
    if (a.ddt_bias)
        hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((D + 255) / 256)), dim3(256), 0, s, a.pdT, a.batch * K,
                           D, a.ddt_bias, D);
    if (MODE == kBwdTrap && a.dx_prev)
        hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((a.batch * N + 255) / 256)), dim3(256), 0, s, a.pdBp,
                           ncb, a.batch * N, a.dB_prev, a.batch * N);
    return hipGetLastError();
}

template <int N, int DT, int MODE>
hipError_t launch_bwd_flags(const BwdArgs &a, hipStream_t s) {
    const bool gate = a.z != nullptr, skip = a.Dskip != nullptr;
    if (gate && skip) return launch_bwd_typed<N, DT, true, true, MODE>(a, s);
    if (gate) return launch_bwd_typed<N, DT, true, false, MODE>(a, s);
    if (skip) return launch_bwd_typed<N, DT, false, true, MODE>(a, s);
    return launch_bwd_typed<N, DT, false, false, MODE>(a, s);
}

}  // namespace

}  // namespace ssm
