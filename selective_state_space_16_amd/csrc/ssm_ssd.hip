// Mamba-2 state space dual (SSD) layer for gfx950, by chunks on the matrix
// cores.
//
// With the transition restricted to a scalar per head, a_t = exp(delta_t A_h),
// the output of a head is y = M x with M_ji = (prod_{i<k<=j} a_k) C_j . B_i
// delta_i, a masked product like causal attention ("Notas sobre Mamba",
// section "A forma dual: atenção mascarada"). The sequence is cut into chunks
// of Q = 64 tokens; inside a chunk the dual (quadratic) form is a pair of
// small matrix products, and between chunks the (P, N) state carries the rest
// (the chunked algorithm of section "O algoritmo SSD" and of "Mamba-2 e State
// Space Duality (SSD)", where Q is typically 64). Per chunk, with cum_j the
// log2 decay from the chunk start through token j:
//
//   G      = C B^T                                  (Q x Q, K = N)
//   M_ji   = G_ji exp2(cum_j - cum_i) delta_i,  i <= j (0 above the diagonal)
//   y      = M x + diag(exp2(cum)) C H^T + D x      (K = Q, then K = N)
//   H      = exp2(cum_last) H + x^T (w o B),        w_i = delta_i exp2(cum_last - cum_i)
//
// One workgroup of four waves walks the chunks of one (batch row, head) in
// order. The state H (P x N float) stays in the matrix-core accumulators of
// the waves for the whole sequence; a bfloat16 copy in LDS feeds C H^T. All
// products are v_mfma_f32_16x16x32_bf16 with float accumulation.
#include "ssm_common.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;   // tokens per chunk
constexpr int kP = 64;   // head dimension
constexpr int kThreads = 256;

// LDS of one workgroup. Rows are padded by 16 bytes so that the 16 lanes that
// read one 16-byte piece each from 16 consecutive rows hit different banks.
template <int N>
struct SsdShared {
    static constexpr int RN = N + 8, RQ = kQ + 8;
    alignas(16) uint16_t Cs[kQ][RN];  // C rows of the chunk
    alignas(16) uint16_t Bs[kQ][RN];  // B rows; then M [kQ][RQ]; then y [kQ][RQ]
    alignas(16) uint16_t BT[N][RQ];   // w_i B[i][n], transposed
    alignas(16) uint16_t XT[kP][RQ];  // x, transposed
    alignas(16) uint16_t Hs[kP][RN];  // the state rounded to bfloat16
    float cum[kQ];                    // log2 decay from the chunk start through token j
    float dl[kQ];                     // delta
    float w[kQ];                      // delta_i exp2(cum_last - cum_i)
};

__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) { return *(const bf16x8 *)__builtin_assume_aligned(p, 16); }
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint16_t to_bf16(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
__device__ __forceinline__ float from_bf16(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// The ten 16 x 16 tiles of the chunk's lower triangle, as (row block, column
// block), dealt to the four waves round robin.
__constant__ const int kLowJ[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ const int kLowI[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

// Matrix-core tile layout (16 x 16 x 32, bfloat16): the A operand row r,
// k = 8 kk .. 8 kk + 7 sits in lane r + 16 kk; the B operand column c, the same
// k, in lane c + 16 kk; result element e of lane l is row 4 (l / 16) + e,
// column l % 16. So A is read from a [row][k] array and B from a [column][k]
// array, one 16-byte piece per lane.
template <int N, bool SKIP>
__global__ __launch_bounds__(kThreads, 2) void ssd_kernel(SsdArgs a) {
    constexpr int NB = N / 16, RQ = kQ + 8;
    __shared__ SsdShared<N> sh;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int lr = l & 15, lq = l >> 4;
    const int64_t H = a.H, L = a.L, G = a.G;
    const int64_t b = blockIdx.x / H, h = blockIdx.x % H, g = h / (H / G);
    const float A2 = a.A[h] * kLog2e;
    const float dsk = SKIP ? a.Dskip[h] : 0.0f;
    const uint16_t *xp = (const uint16_t *)a.x;
    const uint16_t *dp = (const uint16_t *)a.delta;
    const uint16_t *Bp = (const uint16_t *)a.Bt;
    const uint16_t *Cp = (const uint16_t *)a.Ct;
    uint16_t *yp = (uint16_t *)a.y;
    uint16_t (*Ms)[RQ] = reinterpret_cast<uint16_t (*)[RQ]>(&sh.Bs[0][0]);

    // The state: wave w holds rows p = 16 w + 4 lq + e, columns n = 16 nb + lr.
    f32x4 Hacc[NB];
    const float *si = a.state_in ? a.state_in + (b * H + h) * (int64_t)(kP * N) : nullptr;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            Hacc[nb][e] = si ? si[(16 * w + 4 * lq + e) * N + 16 * nb + lr] : 0.0f;
            sh.Hs[16 * w + 4 * lq + e][16 * nb + lr] = to_bf16(Hacc[nb][e]);
        }

    const int64_t nchunks = (L + kQ - 1) / kQ;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * kQ;
        // 1. the chunk's delta, x (transposed), B and C; tokens past L are zero
        if (w == 0) sh.dl[l] = t0 + l < L ? from_bf16(dp[(b * L + t0 + l) * H + h]) : 0.0f;
        for (int q = tid; q < kQ * kP / 8; q += kThreads) {
            const int t = q / (kP / 8), p0 = (q % (kP / 8)) * 8;
            uint4 v = {0, 0, 0, 0};
            if (t0 + t < L) v = *(const uint4 *)(xp + ((b * L + t0 + t) * H + h) * kP + p0);
            uint16_t e[8];
            __builtin_memcpy(e, &v, sizeof(v));
#pragma unroll
            for (int k = 0; k < 8; ++k) sh.XT[p0 + k][t] = e[k];
        }
        for (int q = tid; q < kQ * N / 8; q += kThreads) {
            const int t = q / (N / 8), n0 = (q % (N / 8)) * 8;
            uint4 vb = {0, 0, 0, 0}, vc = {0, 0, 0, 0};
            if (t0 + t < L) {
                const int64_t off = ((b * L + t0 + t) * G + g) * N + n0;
                vb = *(const uint4 *)(Bp + off);
                vc = *(const uint4 *)(Cp + off);
            }
            *(uint4 *)&sh.Bs[t][n0] = vb;
            *(uint4 *)&sh.Cs[t][n0] = vc;
        }
        __syncthreads();
        // 2. cumulative log2 decay (an inclusive scan over the 64 tokens) and
        //    the state-update weights
        if (w == 0) {
            float v = sh.dl[l] * A2;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float u = __shfl_up(v, d);
                if (l >= d) v += u;
            }
            sh.cum[l] = v;
            sh.w[l] = sh.dl[l] * fast_exp2(__shfl(v, 63) - v);
        }
        __syncthreads();
        // 3. G = C B^T on the lower-triangle tiles, and BT = (w o B)^T
        f32x4 Gt[3];
        int ntiles = 0;
        for (int k = w; k < 10; k += 4, ++ntiles) {
            const int jb = kLowJ[k], ib = kLowI[k];
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < N / 32; ++kb)
                acc = mfma(ld8(&sh.Cs[16 * jb + lr][32 * kb + 8 * lq]), ld8(&sh.Bs[16 * ib + lr][32 * kb + 8 * lq]), acc);
            Gt[ntiles] = acc;
        }
        for (int q = tid; q < kQ * N / 8; q += kThreads) {
            const int t = q / (N / 8), n0 = (q % (N / 8)) * 8;
            uint16_t e[8];
            __builtin_memcpy(e, &sh.Bs[t][n0], sizeof(e));
            const float wt = sh.w[t];
#pragma unroll
            for (int k = 0; k < 8; ++k) sh.BT[n0 + k][t] = to_bf16(from_bf16(e[k]) * wt);
        }
        __syncthreads();  // every read of Bs is done: its space now holds M
        // 4. M: decay, delta and the causal mask on the wave's tiles; zeros above
        for (int k = w, i = 0; k < 10; k += 4, ++i) {
            const int jb = kLowJ[k], ib = kLowI[k];
            const int ii = 16 * ib + lr;
            const float ci = sh.cum[ii], di = sh.dl[ii];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jj = 16 * jb + 4 * lq + e;
                const float v = ii <= jj ? Gt[i][e] * fast_exp2(sh.cum[jj] - ci) * di : 0.0f;
                Ms[jj][ii] = to_bf16(v);
            }
        }
        for (int q = tid; q < 6 * 256; q += kThreads) {  // the six tiles above the diagonal
            const int tile = q / 256, r = (q % 256) / 16, cc = q % 16;
            const int jb = tile < 3 ? 0 : tile < 5 ? 1 : 2;
            const int ib = tile < 3 ? tile + 1 : tile < 5 ? tile - 1 : 3;
            Ms[16 * jb + r][16 * ib + cc] = 0;
        }
        __syncthreads();
        // 5. y for the wave's 16 tokens: M x + diag(exp2(cum)) C H^T + D x
        float yv[4][4];
        {
            const int jb = w;
#pragma unroll
            for (int pb = 0; pb < 4; ++pb) {
                f32x4 yd = {0.0f, 0.0f, 0.0f, 0.0f}, yo = {0.0f, 0.0f, 0.0f, 0.0f};
                for (int kb = 0; kb <= jb / 2; ++kb)
                    yd = mfma(ld8(&Ms[16 * jb + lr][32 * kb + 8 * lq]), ld8(&sh.XT[16 * pb + lr][32 * kb + 8 * lq]), yd);
#pragma unroll
                for (int kb = 0; kb < N / 32; ++kb)
                    yo = mfma(ld8(&sh.Cs[16 * jb + lr][32 * kb + 8 * lq]), ld8(&sh.Hs[16 * pb + lr][32 * kb + 8 * lq]), yo);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int jj = 16 * jb + 4 * lq + e, pp = 16 * pb + lr;
                    float v = __builtin_fmaf(fast_exp2(sh.cum[jj]), yo[e], yd[e]);
                    if (SKIP) v = __builtin_fmaf(dsk, from_bf16(sh.XT[pp][jj]), v);
                    yv[pb][e] = v;
                }
            }
        }
        __syncthreads();  // M, C and the state copy are read: y goes where M was
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
            for (int e = 0; e < 4; ++e) Ms[16 * w + 4 * lq + e][16 * pb + lr] = to_bf16(yv[pb][e]);
        // 6. the state: H = exp2(cum_last) H + x^T (w o B), on the wave's 16 rows
        {
            const float dec = fast_exp2(sh.cum[kQ - 1]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                f32x4 acc = Hacc[nb] * dec;
#pragma unroll
                for (int kb = 0; kb < kQ / 32; ++kb)
                    acc = mfma(ld8(&sh.XT[16 * w + lr][32 * kb + 8 * lq]), ld8(&sh.BT[16 * nb + lr][32 * kb + 8 * lq]), acc);
                Hacc[nb] = acc;
#pragma unroll
                for (int e = 0; e < 4; ++e) sh.Hs[16 * w + 4 * lq + e][16 * nb + lr] = to_bf16(acc[e]);
            }
        }
        __syncthreads();
        // 7. y rows out, 16 bytes per thread and piece
        for (int q = tid; q < kQ * kP / 8; q += kThreads) {
            const int t = q / (kP / 8), p0 = (q % (kP / 8)) * 8;
            if (t0 + t < L) *(uint4 *)(yp + ((b * L + t0 + t) * H + h) * kP + p0) = *(const uint4 *)&Ms[t][p0];
        }
        __syncthreads();  // the next chunk's loads overwrite the LDS
    }
    if (a.state_out) {
        float *so = a.state_out + (b * H + h) * (int64_t)(kP * N);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) so[(16 * w + 4 * lq + e) * N + 16 * nb + lr] = Hacc[nb][e];
    }
}

template <int N>
hipError_t launch_ssd_n(const SsdArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)(a.batch * a.H));
    if (a.Dskip) hipLaunchKernelGGL((ssd_kernel<N, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((ssd_kernel<N, false>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool ssd_supported(int64_t P, int64_t N) { return P == kP && (N == 64 || N == 128); }

hipError_t launch_ssd(const SsdArgs &a, int N, hipStream_t s) {
    if (a.batch * a.H > INT32_MAX) return hipErrorInvalidValue;
    switch (N) {
        case 64: return launch_ssd_n<64>(a, s);
        case 128: return launch_ssd_n<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
