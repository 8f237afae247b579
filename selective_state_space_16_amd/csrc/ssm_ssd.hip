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
// log2 decay from the chunk start through token j, the kernel forms the
// transposed products
//
//   G^T      = B C^T                                      (K = N)
//   M^T_ij   = G^T_ij exp2(cum_j - cum_i) delta_i,  i <= j  (0 below)
//   y^T      = x^T M^T + (H C^T) diag(exp2(cum)) + D x^T  (K = Q, then K = N)
//   H        = exp2(cum_last) H + x^T (w o B),            w_i = delta_i exp2(cum_last - cum_i)
//
// One workgroup of four waves walks the chunks of one (batch row, head) in
// order; wave w owns the 16 tokens 16 w .. 16 w + 15 of every chunk for y and
// the 16 rows 16 w .. of the state. The state H (P x N float) stays in the
// matrix-core accumulators for the whole sequence; a bfloat16 copy in LDS
// feeds H C^T. A 16 x 16 tile of G^T comes out of the matrix core with each
// lane holding four consecutive rows of one column, which is the operand
// layout of the 16 x 16 x 16 product: M^T is masked and scaled in registers
// and goes straight back in, never through LDS. The next chunk's x, B, C and
// delta are loaded into registers while the current one is computed. Two
// workgroup barriers per chunk.
#include "ssm_common.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQ = 64;   // tokens per chunk
constexpr int kP = 64;   // head dimension
constexpr int kThreads = 256;

// LDS of one workgroup. Rows are padded by 16 bytes so that the 16 lanes that
// read one piece each from 16 consecutive rows hit different banks.
template <int N>
struct SsdShared {
    static constexpr int RN = N + 8, RQ = kQ + 8;
    alignas(16) uint16_t Cs[kQ][RN];  // C rows of the chunk
    alignas(16) uint16_t Bs[kQ][RN];  // B rows
    alignas(16) uint16_t BT[N][RQ];   // w_i B[i][n], transposed
    alignas(16) uint16_t XT[kP][RQ];  // x, transposed
    alignas(16) uint16_t Hs[kP][RN];  // the state rounded to bfloat16
    float cum[kQ];                    // log2 decay from the chunk start through token j
    float dl[kQ];                     // delta
};

__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) { return *(const bf16x8 *)__builtin_assume_aligned(p, 16); }
__device__ __forceinline__ s16x4 ld4(const uint16_t *p) { return *(const s16x4 *)__builtin_assume_aligned(p, 8); }
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint16_t to_bf16(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
__device__ __forceinline__ float from_bf16(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// The chunk's global data, held in registers between its load and its LDS
// store, as 16-byte pieces of 8 consecutive p (x) or n (Bt, Ct) of one token.
// x and Bt pieces are stored transposed, so lane l holds token l (wave w holds
// the pieces 8 (w + 4 k)): the 64 lanes of a transposed store then write one
// contiguous row. Ct pieces are stored as rows: 16-byte pieces in row order.
// The delta of token `lane` (every wave holds all 64). Tokens past L are read
// from token L - 1 and zeroed where they are stored, so that no instruction
// needs a loaded value before the chunk is consumed and the loads stay in
// flight.
template <int N>
struct ChunkRegs {
    static constexpr int XP = kP / 8 / 4, BP = N / 8 / 4;
    u32x4 x[XP], b[BP], c[BP];
    uint16_t dl;
};

// The chunk's loads: a wave-uniform base per tensor (the chunk's first token
// in this batch row and head or group) plus a 32-bit per-lane byte offset that
// is the same for every chunk. The last, partial chunk clamps its tokens to
// L - 1 instead.
template <int N>
__device__ __forceinline__ void load_chunk(ChunkRegs<N> &r, const SsdArgs &a, int64_t b, int64_t h, int64_t g,
                                           int64_t t0, int tid) {
    using R = ChunkRegs<N>;
    const int64_t L = a.L, H = a.H, G = a.G;
    const int l = tid & 63, w = tid >> 6;
    const char *xb = (const char *)a.x + ((b * L + t0) * H + h) * (kP * 2);
    const char *bb = (const char *)a.Bt + ((b * L + t0) * G + g) * (N * 2);
    const char *cb = (const char *)a.Ct + ((b * L + t0) * G + g) * (N * 2);
    const char *db = (const char *)a.delta + ((b * L + t0) * H + h) * 2;
    const uint32_t xs = (uint32_t)(H * kP * 2), bs = (uint32_t)(G * N * 2), ds = (uint32_t)(H * 2);
    const bool part = t0 + kQ > L;
    const uint32_t last = (uint32_t)(L - 1 - t0);  // used only when part
    // token of this lane (x, Bt, delta) and of this thread's Ct pieces
    uint32_t ul = (uint32_t)l;
    if (part) ul = ul < last ? ul : last;
    r.dl = *(const uint16_t *)(db + ul * ds);
#pragma unroll
    for (int k = 0; k < R::XP; ++k) r.x[k] = *(const u32x4 *)(xb + ul * xs + 16 * (w + 4 * k));
#pragma unroll
    for (int k = 0; k < R::BP; ++k) r.b[k] = *(const u32x4 *)(bb + ul * bs + 16 * (w + 4 * k));
    const uint32_t cn = (uint32_t)((tid % (N / 8)) * 16);
#pragma unroll
    for (int k = 0; k < R::BP; ++k) {
        uint32_t t = (uint32_t)((tid + k * kThreads) / (N / 8));
        if (part) t = t < last ? t : last;
        r.c[k] = *(const u32x4 *)(cb + t * bs + cn);
    }
}

// An empty statement that takes the chunk registers as inputs and outputs: the
// code that unpacks them cannot move above it, so the loads that fill them
// stay in flight until the chunk is consumed.
template <int N>
__device__ __forceinline__ void pin(ChunkRegs<N> &r) {
#pragma unroll
    for (int k = 0; k < ChunkRegs<N>::XP; ++k) asm volatile("" : "+v"(r.x[k]));
#pragma unroll
    for (int k = 0; k < ChunkRegs<N>::BP; ++k) asm volatile("" : "+v"(r.b[k]), "+v"(r.c[k]));
    uint32_t d = r.dl;
    asm volatile("" : "+v"(d));
    r.dl = (uint16_t)d;
}

// The products of wave W for its 16 tokens j = 16 W + lr of the chunk: the
// G^T tiles of i blocks 0 .. W, masked and scaled into M^T in registers, and
// y^T = x^T M^T + (H C^T) exp2(cum_j) + D x^T as four 16 x 16 tiles of p,
// packed to bfloat16 in `yout` (tile pb: rows p = 16 pb + 4 lq .. + 3).
// W is a compile-time constant so that the independent tiles interleave.
template <int N, bool SKIP, int W>
__device__ __forceinline__ void wave_products(SsdShared<N> &sh, int lr, int lq, float dsk, u32x2 (&yout)[4]) {
    constexpr int KB = N / 32, NT = W + 1;
    bf16x8 cf[KB];  // C rows of the wave's tokens: the B operand of G^T and of H C^T
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) cf[kb] = ld8(&sh.Cs[16 * W + lr][32 * kb + 8 * lq]);
    const int jj = 16 * W + lr;
    const float cum_j = sh.cum[jj];
    f32x4 gacc[NT];
#pragma unroll
    for (int ib = 0; ib < NT; ++ib) gacc[ib] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ib = 0; ib < NT; ++ib) gacc[ib] = mfma32(ld8(&sh.Bs[16 * ib + lr][32 * kb + 8 * lq]), cf[kb], gacc[ib]);
    s16x4 mt[NT];
#pragma unroll
    for (int ib = 0; ib < NT; ++ib)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ii = 16 * ib + 4 * lq + e;
            float v = gacc[ib][e] * fast_exp2(cum_j - sh.cum[ii]) * sh.dl[ii];
            if (ib == W) v = ii <= jj ? v : 0.0f;  // the diagonal tile: i <= j only
            mt[ib][e] = (short)to_bf16(v);
        }
    f32x4 yd[4], yo[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) yd[pb] = yo[pb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) yo[pb] = mfma32(ld8(&sh.Hs[16 * pb + lr][32 * kb + 8 * lq]), cf[kb], yo[pb]);
#pragma unroll
    for (int ib = 0; ib < NT; ++ib)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) yd[pb] = mfma16(ld4(&sh.XT[16 * pb + lr][16 * ib + 4 * lq]), mt[ib], yd[pb]);
    const float dec_j = fast_exp2(cum_j);
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
        uint16_t out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = __builtin_fmaf(dec_j, yo[pb][e], yd[pb][e]);
            if (SKIP) v = __builtin_fmaf(dsk, from_bf16(sh.XT[16 * pb + 4 * lq + e][jj]), v);
            out[e] = to_bf16(v);
        }
        __builtin_memcpy(&yout[pb], out, sizeof(out));
    }
}

// Matrix-core layouts. 16 x 16 x 32: the A operand row r, k = 8 kk .. + 7 sits
// in lane r + 16 kk; the B operand column c, the same k, in lane c + 16 kk.
// 16 x 16 x 16: the same with 4 k per lane (k = 4 kk .. + 3). Both: result
// element e of lane l is row 4 (l / 16) + e, column l % 16. So A is read from a
// [row][k] array and B from a [column][k] array.
template <int N, bool SKIP>
__global__ __launch_bounds__(kThreads, 2) void ssd_kernel(SsdArgs a) {
    constexpr int NB = N / 16, KB = N / 32;
    __shared__ SsdShared<N> sh;
    using R = ChunkRegs<N>;
    const int tid = threadIdx.x, l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
    const int lr = l & 15, lq = l >> 4;
    const int64_t H = a.H, L = a.L, G = a.G;
    // Workgroups are dealt to the 8 XCDs in turn (block id mod 8). When the
    // count divides evenly, XCD x takes the x-th eighth of the (b, h) pairs in
    // order, so the heads of a batch row, which read the same Bt and Ct,
    // share one XCD's L2.
    const int64_t nwg = (int64_t)gridDim.x;
    const int64_t pair = nwg % 8 == 0 ? (int64_t)(blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;
    const int64_t b = pair / H, h = pair % H, g = h / (H / G);
    const float A2 = a.A[h] * kLog2e;
    const float dsk = SKIP ? a.Dskip[h] : 0.0f;
    uint16_t *yp = (uint16_t *)a.y;

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

    // y of the previous chunk, stored once that chunk's successor has landed
    // (so that waiting for the loads never waits for these stores)
    u32x2 yout[4];
    int64_t yt0 = -1;
    const int64_t yrow = (b * L + 16 * w + lr) * H + h;  // this lane's token of chunk 0
    auto store_y = [&]() {
        if (yt0 >= 0 && yt0 + 16 * w + lr < L) {
#pragma unroll
            for (int pb = 0; pb < 4; ++pb)
                *(u32x2 *)(yp + (yrow + yt0 * H) * kP + 16 * pb + 4 * lq) = yout[pb];
        }
    };
    R r;
    load_chunk<N>(r, a, b, h, g, 0, tid);
    const int64_t nchunks = (L + kQ - 1) / kQ;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * kQ;
        pin<N>(r);
        store_y();
        // 1. decay: an inclusive scan of delta A over the 64 tokens, in every
        //    wave (lane = token), and the state-update weights
        const float dl = t0 + l < L ? from_bf16(r.dl) : 0.0f;
        float cum = dl * A2;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float u = __shfl_up(cum, d);
            if (l >= d) cum += u;
        }
        const float cum_last = __shfl(cum, 63);
        const float wl = dl * fast_exp2(cum_last - cum);
        if (w == 0) {
            sh.cum[l] = cum;
            sh.dl[l] = dl;
        }
        // 2. the chunk into LDS: x and w o B transposed (lane = token), B and C
        //    as rows
        const bool lin = t0 + l < L;
#pragma unroll
        for (int k = 0; k < R::XP; ++k) {
            const int p0 = 8 * (w + 4 * k);
            uint16_t e[8];
            __builtin_memcpy(e, &r.x[k], sizeof(e));
#pragma unroll
            for (int j = 0; j < 8; ++j) sh.XT[p0 + j][l] = lin ? e[j] : 0;
        }
#pragma unroll
        for (int k = 0; k < R::BP; ++k) {
            const int n0 = 8 * (w + 4 * k);
            *(u32x4 *)&sh.Bs[l][n0] = lin ? r.b[k] : u32x4{0, 0, 0, 0};
            uint16_t e[8];
            __builtin_memcpy(e, &r.b[k], sizeof(e));
#pragma unroll
            for (int j = 0; j < 8; ++j) sh.BT[n0 + j][l] = to_bf16(from_bf16(e[j]) * wl);  // wl = 0 past L
        }
#pragma unroll
        for (int k = 0; k < R::BP; ++k) {
            const int q = tid + k * kThreads, t = q / (N / 8), n0 = (q % (N / 8)) * 8;
            *(u32x4 *)&sh.Cs[t][n0] = t0 + t < L ? r.c[k] : u32x4{0, 0, 0, 0};
        }
        __syncthreads();
        // 3. the next chunk's loads, in flight during this chunk's products
        if (c + 1 < nchunks) load_chunk<N>(r, a, b, h, g, t0 + kQ, tid);
        asm volatile("" ::: "memory");  // keeps the loads here: they are consumed next chunk
        // 4-5. the wave's tokens: G^T, M^T, and y^T (stored at the next chunk)
        switch (w) {
            case 0: wave_products<N, SKIP, 0>(sh, lr, lq, dsk, yout); break;
            case 1: wave_products<N, SKIP, 1>(sh, lr, lq, dsk, yout); break;
            case 2: wave_products<N, SKIP, 2>(sh, lr, lq, dsk, yout); break;
            default: wave_products<N, SKIP, 3>(sh, lr, lq, dsk, yout); break;
        }
        yt0 = t0;
        // 6. the state: H = exp2(cum_last) H + x^T (w o B), on the wave's 16 rows
        {
            const float dec = fast_exp2(cum_last);
            bf16x8 xf[kQ / 32];
#pragma unroll
            for (int kb = 0; kb < kQ / 32; ++kb) xf[kb] = ld8(&sh.XT[16 * w + lr][32 * kb + 8 * lq]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                f32x4 acc = Hacc[nb] * dec;
#pragma unroll
                for (int kb = 0; kb < kQ / 32; ++kb) acc = mfma32(xf[kb], ld8(&sh.BT[16 * nb + lr][32 * kb + 8 * lq]), acc);
                Hacc[nb] = acc;
            }
        }
        __syncthreads();  // every read of this chunk's LDS is done
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) sh.Hs[16 * w + 4 * lq + e][16 * nb + lr] = to_bf16(Hacc[nb][e]);
    }
    store_y();
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
