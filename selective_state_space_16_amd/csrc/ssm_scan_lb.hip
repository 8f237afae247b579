// Single-pass selective scan (S6) forward for gfx950: register-resident chunk
// scan with a decoupled look-back between workgroups.
//
// The recurrence h <- dA*h + dBx is an associative composition of affine maps
// ("Notas sobre Mamba", section "A varredura paralela ciente do hardware":
// the scan over (A-bar_t, B-bar_t x_t) pairs). Applying a run of tokens to a
// state equals one pair (P, S): P = prod dA = exp(A * sum delta) and S = the
// run's end state from a zero start. This kernel uses that at two levels:
//
//  - A workgroup owns one chunk of W*T tokens of one channel block. Each wave
//    owns T consecutive tokens of the chunk. In phase A it computes
//    dA = exp2(delta * A*log2(e)) and dBx = delta*x*B for its tokens once and
//    keeps them in registers, folding them into its segment's (P, S). The
//    segments are combined through LDS.
//  - Chunks of the same channel block pass states through global memory:
//    every chunk publishes its aggregate (sum delta, S) as soon as phase A is
//    done, then looks back over earlier chunks (aggregates, or an inclusive
//    end state) to obtain its carried-in state, and publishes its own
//    inclusive end state. Workgroups are numbered chunk-major and dispatched
//    in order, so a chunk only ever waits on chunks dispatched before it.
//  - Phase C rescans each wave's tokens from its carried-in state using the
//    registers from phase A (no second exponential), reads y = C.h + D.x,
//    applies the silu(z) gate and stores y.
//
// Lane layout: a wave is 4 rows of 16 lanes. A channel's N states are split
// over NGR = N/NL rows (NL = min(N, 4) states per lane); the 16 lanes of a row
// are 16 consecutive channels. Bt[t,:] and Ct[t,:] are the same for every
// channel, so a row keeps the values of its state group for 16/NL tokens in
// one register and broadcasts them to its lanes with DPP row_newbcast. The
// readout sum over a channel's rows uses permlane16/32 swaps, which also
// scatter the finished tokens over the rows so that every lane finishes
// (skip, gate, store) T/NGR of the T tokens.
//
// Cross-workgroup publication: data words are written with device-scope
// stores, the wave waits for them to complete (s_waitcnt), and only then a
// flag word carrying this call's epoch is written; readers poll the flag
// with device-scope loads and read the data after seeing it. Every wait is
// bounded: on timeout the kernel records an error word in the workspace
// header and continues with a zero state.
#include <type_traits>

#include "ssm_common.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kSegT = 16;         // tokens per wave segment
constexpr int kLbWaves = 4;       // waves (segments) per workgroup
constexpr int kChunk = kSegT * kLbWaves;
constexpr int kXcds = 8;          // XCDs of an MI355X
constexpr long kSpinLimit = 1L << 20;   // polls before a wait gives up (about a second)

template <int N>
struct Geo {
    static constexpr int NL = N < 4 ? N : 4;     // states per lane
    static constexpr int NGR = N / NL;           // rows per channel
    static constexpr int SETS = 4 / NGR;         // channel sets per wave
    static constexpr int CPW = SETS * 16;        // channels per wave
    static constexpr int TPV = 16 / NL;          // tokens per broadcast register
    static constexpr int BREGS = kSegT / TPV;    // broadcast registers per segment
    static constexpr int OWN = kSegT / NGR;      // tokens each lane finishes
};

// DPP row_newbcast: every lane of a row gets lane SRC of that row.
template <int SRC>
__device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + SRC, 0xF, 0xF, true));
}

// acc += (lane SRC of the row's `c`) * h, as one v_fmac_f32 with a DPP source.
// The leading s_nop covers the DPP read-after-VALU-write hazard, which the
// compiler does not see inside inline assembly.
#define SSM_FMAC_BCAST(SRC)                                                                       \
    template <>                                                                                   \
    __device__ __forceinline__ void fmac_bcast<SRC>(float &acc, float c, float h) {               \
        asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:" #SRC                    \
                     " row_mask:0xf bank_mask:0xf"                                                \
                     : "+v"(acc)                                                                  \
                     : "v"(c), "v"(h));                                                           \
    }
template <int SRC>
__device__ __forceinline__ void fmac_bcast(float &acc, float c, float h);
SSM_FMAC_BCAST(0) SSM_FMAC_BCAST(1) SSM_FMAC_BCAST(2) SSM_FMAC_BCAST(3)
SSM_FMAC_BCAST(4) SSM_FMAC_BCAST(5) SSM_FMAC_BCAST(6) SSM_FMAC_BCAST(7)
SSM_FMAC_BCAST(8) SSM_FMAC_BCAST(9) SSM_FMAC_BCAST(10) SSM_FMAC_BCAST(11)
SSM_FMAC_BCAST(12) SSM_FMAC_BCAST(13) SSM_FMAC_BCAST(14) SSM_FMAC_BCAST(15)
#undef SSM_FMAC_BCAST

template <int I, int END, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < END) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, END>(f);
    }
}

// v_permlane32_swap: lanes 32-63 of a trade places with lanes 0-31 of b, so
// a = [a.lo, b.lo] and b = [a.hi, b.hi]. v_permlane16_swap: the odd rows of a
// trade places with the even rows of b. Written as inline assembly (with the
// two wait states a VALU-written source needs) because the compiler builtin
// returns both results in one register when they feed the same add.
__device__ __forceinline__ void swap_halves(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_odd_even_rows(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ void st_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_flag(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Complete this wave's stores, then raise the flag.
__device__ __forceinline__ void publish_flag(uint32_t *flag, uint32_t epoch, int lane) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int N, int DT, bool GATE, bool SKIP>
__global__ __launch_bounds__(64 * kLbWaves) void scan_lb_kernel(LbArgs a) {
    using G = Geo<N>;
    using T = typename Act<DT>::T;
    constexpr int NL = G::NL, NGR = G::NGR, CPW = G::CPW, TPV = G::TPV, BREGS = G::BREGS;

    __shared__ float seg_s[kLbWaves][64][NL];
    __shared__ float seg_d[kLbWaves][64];
    __shared__ float carry_in[64][NL];

    const int w = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int row = l >> 4, k16 = l & 15;
    const int g = row % NGR;                 // state group of this lane
    const int64_t D = a.D, L = a.L;
    // Workgroups go to the 8 XCDs round-robin (block id mod 8). Each XCD gets
    // a contiguous range of columns so that neighbouring channel blocks, which
    // share cache lines of x, delta, z and y, meet in the same L2; within an
    // XCD the blocks run chunk-major, so a chunk's predecessor (same column)
    // has a smaller block id on the same XCD and is dispatched before it.
    const int64_t bid = blockIdx.x;
    const int64_t part = bid % kXcds, slot = bid / kXcds;
    const int64_t cpp = a.ncols_pad / kXcds;  // columns per XCD
    const int64_t k = slot / cpp;             // chunk
    const int64_t col = part * cpp + slot % cpp;  // (batch row, channel block)
    if (col >= a.ncols) return;               // padding column
    const int64_t b = col / a.nbd;
    const int64_t d = (col % a.nbd) * CPW + (row / NGR) * 16 + k16;
    const bool valid = d < D;
    const int64_t dc = valid ? d : D - 1;
    const int64_t t0 = k * kChunk + (int64_t)w * kSegT;
    const int nstate0 = g * NL;

    float A2[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) A2[j] = a.A[dc * N + nstate0 + j] * kLog2e;

    const T *xp = (const T *)a.x;
    const T *dp = (const T *)a.delta;
    const T *Bp = (const T *)a.Bt;
    const T *Cp = (const T *)a.Ct;

    // Inputs of this wave's segment. Tokens past the end act as the identity
    // map (delta = 0, x = 0) and are never stored.
    float xv[kSegT], dv[kSegT];
#pragma unroll
    for (int t = 0; t < kSegT; ++t) {
        const int64_t tt = t0 + t;
        if (tt < L) {
            const int64_t r = (b * L + tt) * D + dc;
            xv[t] = ld_act(xp, r);
            dv[t] = ld_act(dp, r);
        } else {
            xv[t] = 0.0f;
            dv[t] = 0.0f;
        }
    }
    float Bq[BREGS], Cq[BREGS];
#pragma unroll
    for (int q = 0; q < BREGS; ++q) {
        int64_t tt = t0 + q * TPV + k16 / NL;
        tt = tt < L ? tt : L - 1;
        const int64_t off = (b * L + tt) * N + nstate0 + (k16 % NL);
        Bq[q] = ld_act(Bp, off);
        Cq[q] = ld_act(Cp, off);
    }

    // Start reading the predecessor's flag now (after the input loads, so that
    // waiting for those does not wait for it); it is looked at after phase A.
    uint32_t early_flag = 0;
    if (w == 0 && k > 0) early_flag = ld_flag(a.incl_flag + (k - 1) * a.ncols + col);

    // Phase A: discretise once, keep dA and dBx, fold the segment.
    float dA[kSegT][NL], u[kSegT][NL], S[NL];
    float dsum = 0.0f;
#pragma unroll
    for (int j = 0; j < NL; ++j) S[j] = 0.0f;
    static_for<0, kSegT>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        const float dx = dv[t] * xv[t];
        dsum += dv[t];
        static_for<0, NL>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            dA[t][j] = fast_exp2(dv[t] * A2[j]);
            u[t][j] = row_bcast<(t % TPV) * NL + j>(Bq[t / TPV]) * dx;
            S[j] = __builtin_fmaf(dA[t][j], S[j], u[t][j]);
        });
    });
#pragma unroll
    for (int j = 0; j < NL; ++j) seg_s[w][l][j] = S[j];
    seg_d[w][l] = dsum;
    __syncthreads();

    if (w == 0) {
        // Chunk aggregate: fold the segments in order.
        float Sagg[NL], dagg = seg_d[0][l];
#pragma unroll
        for (int j = 0; j < NL; ++j) Sagg[j] = seg_s[0][l][j];
#pragma unroll
        for (int v = 1; v < kLbWaves; ++v) {
            const float dd = seg_d[v][l];
#pragma unroll
            for (int j = 0; j < NL; ++j) Sagg[j] = __builtin_fmaf(fast_exp2(A2[j] * dd), Sagg[j], seg_s[v][l][j]);
            dagg += dd;
        }
        const int64_t item = k * a.ncols + col;
        const bool publish = k + 1 < a.K;
        // Chunk 0 publishes only its inclusive state, right after reading
        // state_in: the look-back never reads state_in itself, so state_out
        // (written by the last chunk, which depends on chunk 0) may alias it.
        if (publish && k > 0) {
#pragma unroll
            for (int j = 0; j < NL; ++j) st_dev(a.agg_s + item * (64 * NL) + l * NL + j, Sagg[j]);
            st_dev(a.agg_d + item * 64 + l, dagg);
            publish_flag(a.agg_flag + item, a.epoch, l);
        }
        // Carried-in state of the chunk.
        float H[NL];
        if (k == 0) {
            const float *si = a.state_in ? a.state_in + (b * D + dc) * N + nstate0 : nullptr;
#pragma unroll
            for (int j = 0; j < NL; ++j) H[j] = si ? si[j] : 0.0f;
        } else {
            // Walk back to the nearest chunk whose inclusive state is out,
            // waiting at each chunk until at least its aggregate is.
            int64_t j0 = k - 1;
            long spin = 0;
            bool failed = false;
            bool ready = __builtin_amdgcn_readfirstlane(early_flag) == a.epoch;
            while (!ready) {
                const int64_t it = j0 * a.ncols + col;
                if (__builtin_amdgcn_readfirstlane(ld_flag(a.incl_flag + it)) == a.epoch) break;
                if (__builtin_amdgcn_readfirstlane(ld_flag(a.agg_flag + it)) == a.epoch) {
                    --j0;  // chunk 0 has no aggregate: the walk ends at an inclusive state
                    spin = 0;
                    continue;
                }
                // give up after kSpinLimit polls, or at once when another wait already failed
                if (++spin > kSpinLimit || (spin % 64 == 0 && __builtin_amdgcn_readfirstlane(ld_flag(a.error)) != 0)) {
                    if (l == 0) __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    failed = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (failed) {
#pragma unroll
                for (int j = 0; j < NL; ++j) H[j] = 0.0f;
            } else {
                // Replay the chain forward from that state, chunk by chunk, with
                // the same operations every chunk uses for its own inclusive
                // state, so the carry does not depend on where the walk stopped.
                const int64_t it0 = j0 * a.ncols + col;
#pragma unroll
                for (int j = 0; j < NL; ++j) H[j] = ld_dev(a.incl + it0 * (64 * NL) + l * NL + j);
                for (int64_t jj = j0 + 1; jj < k; ++jj) {
                    const int64_t it = jj * a.ncols + col;
                    const float dd = ld_dev(a.agg_d + it * 64 + l);
#pragma unroll
                    for (int j = 0; j < NL; ++j)
                        H[j] = __builtin_fmaf(fast_exp2(A2[j] * dd), H[j], ld_dev(a.agg_s + it * (64 * NL) + l * NL + j));
                }
            }
        }
        if (publish) {
#pragma unroll
            for (int j = 0; j < NL; ++j)
                st_dev(a.incl + item * (64 * NL) + l * NL + j, __builtin_fmaf(fast_exp2(A2[j] * dagg), H[j], Sagg[j]));
            publish_flag(a.incl_flag + item, a.epoch, l);
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) carry_in[l][j] = H[j];
    }
    __syncthreads();

    // This wave's carried-in state: the chunk's, pushed through earlier segments.
    float h[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) h[j] = carry_in[l][j];
    for (int v = 0; v < w; ++v) {
        const float dd = seg_d[v][l];
#pragma unroll
        for (int j = 0; j < NL; ++j) h[j] = __builtin_fmaf(fast_exp2(A2[j] * dd), h[j], seg_s[v][l][j]);
    }

    // Phase C: rescan from registers; partial readout over this lane's states.
    float yp[kSegT];
    static_for<0, kSegT>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        yp[t] = 0.0f;
        static_for<0, NL>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            h[j] = __builtin_fmaf(dA[t][j], h[j], u[t][j]);
            fmac_bcast<(t % TPV) * NL + j>(yp[t], Cq[t / TPV], h[j]);
        });
    });

    if (k == a.K - 1 && w == kLbWaves - 1 && a.state_out && valid) {
        float *so = a.state_out + (b * D + d) * N + nstate0;
#pragma unroll
        for (int j = 0; j < NL; ++j) so[j] = h[j];
    }

    // Sum the partial readouts over a channel's rows. Afterwards row r holds
    // the finished token t = NGR*q + (r % NGR) of group q.
    float yo[G::OWN];
    if constexpr (NGR == 4) {
#pragma unroll
        for (int q = 0; q < kSegT / 4; ++q) {
            float a0 = yp[4 * q + 0], a2 = yp[4 * q + 2], a1 = yp[4 * q + 1], a3 = yp[4 * q + 3];
            swap_halves(a0, a2);   // rows 0,1: token 0 | rows 2,3: token 2
            swap_halves(a1, a3);   // rows 0,1: token 1 | rows 2,3: token 3
            float s02 = a0 + a2, s13 = a1 + a3;
            swap_odd_even_rows(s02, s13);
            yo[q] = s02 + s13;
        }
    } else if constexpr (NGR == 2) {
#pragma unroll
        for (int q = 0; q < kSegT / 2; ++q) {
            float a0 = yp[2 * q + 0], a1 = yp[2 * q + 1];
            swap_odd_even_rows(a0, a1);
            yo[q] = a0 + a1;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kSegT; ++q) yo[q] = yp[q];
    }

    // Finish the owned tokens: D skip, silu gate, store.
    const float dskip = SKIP ? a.Dskip[dc] : 0.0f;
    T *yptr = (T *)a.y;
    const T *zp = (const T *)a.z;
#pragma unroll
    for (int q = 0; q < G::OWN; ++q) {
        const int t = NGR * q + g;
        const int64_t tt = t0 + t;
        // x of token t; t depends on the row, so select by value
        float xt = xv[NGR * q];
#pragma unroll
        for (int c = 1; c < NGR; ++c) xt = (g == c) ? xv[NGR * q + c] : xt;
        float yv = yo[q];
        if (SKIP) yv = __builtin_fmaf(dskip, xt, yv);
        if (tt < L && valid) {
            const int64_t r = (b * L + tt) * D + d;
            if (GATE) yv *= silu(ld_act(zp, r));
            st_act(yptr, r, yv);
        }
    }
}

template <int N, int DT, bool GATE, bool SKIP>
hipError_t launch_lb_typed(const LbArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((scan_lb_kernel<N, DT, GATE, SKIP>), dim3((unsigned)(a.ncols_pad * a.K)), dim3(64 * kLbWaves),
                       0, s, a);
    return hipGetLastError();
}

template <int N, int DT>
hipError_t launch_lb_flags(const LbArgs &a, hipStream_t s) {
    const bool gate = a.z != nullptr, skip = a.Dskip != nullptr;
    if (gate && skip) return launch_lb_typed<N, DT, true, true>(a, s);
    if (gate) return launch_lb_typed<N, DT, true, false>(a, s);
    if (skip) return launch_lb_typed<N, DT, false, true>(a, s);
    return launch_lb_typed<N, DT, false, false>(a, s);
}

template <int N>
hipError_t launch_lb_dtype(const LbArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch_lb_flags<N, 0>(a, s) : launch_lb_flags<N, 1>(a, s);
}

template <int N>
void lb_geometry(int64_t batch, int64_t L, int64_t D, LbPlan *p) {
    using G = Geo<N>;
    p->cpw = G::CPW;
    p->nl = G::NL;
    p->nbd = (D + G::CPW - 1) / G::CPW;
    p->ncols = batch * p->nbd;
    p->ncols_pad = (p->ncols + kXcds - 1) / kXcds * kXcds;
    p->K = (L + kChunk - 1) / kChunk;
}

}  // namespace

bool lb_plan(int64_t batch, int64_t L, int64_t D, int64_t N, LbPlan *p) {
    switch (N) {
        case 1: lb_geometry<1>(batch, L, D, p); break;
        case 2: lb_geometry<2>(batch, L, D, p); break;
        case 4: lb_geometry<4>(batch, L, D, p); break;
        case 8: lb_geometry<8>(batch, L, D, p); break;
        case 16: lb_geometry<16>(batch, L, D, p); break;
        default: return false;
    }
    p->chunk = kChunk;
    const int64_t items = p->ncols * p->K;
    // header | agg_s | agg_d | incl | agg_flag | incl_flag
    size_t off = 256;
    p->off_agg_s = off;
    off += (size_t)items * 64 * p->nl * sizeof(float);
    p->off_agg_d = off;
    off += (size_t)items * 64 * sizeof(float);
    p->off_incl = off;
    off += (size_t)items * 64 * p->nl * sizeof(float);
    p->off_agg_flag = off;
    off += (size_t)items * sizeof(uint32_t);
    p->off_incl_flag = off;
    off += (size_t)items * sizeof(uint32_t);
    p->bytes = (off + 255) / 256 * 256;
    return true;
}

hipError_t launch_scan_lb(const LbArgs &a, int N, int dtype, hipStream_t s) {
    switch (N) {
        case 1: return launch_lb_dtype<1>(a, dtype, s);
        case 2: return launch_lb_dtype<2>(a, dtype, s);
        case 4: return launch_lb_dtype<4>(a, dtype, s);
        case 8: return launch_lb_dtype<8>(a, dtype, s);
        case 16: return launch_lb_dtype<16>(a, dtype, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
