// Mamba-2 state space dual (SSD) layer for gfx950, by chunks on the matrix
// cores.
//
// With the transition restricted to a scalar per head, a_t = exp(delta_t A_h),
// the output of a head is y = M x with M_ts = (prod_{s<k<=t} a_k) C_t . B_s
// delta_s, a masked product like causal attention ("Notas sobre Mamba",
// section "A forma dual: atenção mascarada"). The sequence is cut into chunks
// of Q = 64 tokens; inside a chunk the dual (quadratic) form is a pair of
// small matrix products, and between chunks the (P, N) state carries the rest
// (the chunked algorithm of section "O algoritmo SSD" and of "Mamba-2 e State
// Space Duality (SSD)", where Q is typically 64). Per chunk, with cum_t the
// log2 decay from the chunk start through token t and w_t = delta_t
// exp2(cum_last - cum_t), the kernel forms, for the state H^T (N x P) that
// enters the chunk,
//
//   G^T      = B C^T                                        (K = N)
//   M^T_st   = G^T_st exp2(cum_t - cum_s) delta_s, s <= t    (0 above), + D on
//              the diagonal
//   y^T      = (H C^T) diag(exp2(cum)) + x^T M^T             (K = N, then K = Q)
//   H^T      = exp2(cum_last) H^T + B^T (w o x)              (K = Q)
//
// One workgroup of four waves walks the chunks of one (batch row, head) in
// order, with two roles:
//
// * Waves 0 and 1 own the head-dimension halves p = 32 w .. 32 w + 31: their
//   state columns stay in the matrix-core accumulators for the whole sequence
//   as H^T tiles, and they form y^T and the state update. An accumulator tile
//   holds four consecutive n of one p per lane, which is the A-operand layout
//   of the products over n, so H C^T takes the state straight from registers.
// * Waves 2 and 3 move the data and form the masked matrix. While waves 0
//   and 1 finish a chunk, they hold the next chunk's x, B, C (and delta) in
//   registers, loaded as whole rows so that the loads coalesce; after the
//   barrier that frees the LDS they store the rows there, and after a second
//   barrier they form the ten G^T tiles on or below the diagonal (five each)
//   from LDS, mask and weight them, and store M^T as the register images the
//   consumers read back lane by lane.
//
// Three workgroup barriers per chunk: S (the chunk's rows are in LDS: the
// consumers start on H C^T while the masked matrix is formed), A (M^T is in
// LDS: x^T M^T and the state update), B (the consumers are done with the
// chunk). The products over 32 k use the 16 x 16 x 32 bfloat16 instruction;
// where the k of an operand come from two 16-row tiles (the state over n, the
// tokens of x and B) the k order inside the instruction is permuted the same
// way on both operands, which leaves the sum unchanged. Operands that need the
// other orientation (x^T and B^T, k = tokens) are read with the LDS transpose
// read ds_read_b64_tr_b16. About 53 KB of LDS, so that three workgroups share
// a CU.
#include "ssm_common.h"
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kQ = 64;  // tokens per chunk
constexpr int kP = 64;  // head dimension
constexpr int kThreads = 256;

// LDS of one workgroup: one chunk. Row strides are chosen for the reads the
// consumers make: x and B are read four rows at a time, 32 bytes per row (the
// transpose read), so their rows are 32 bytes longer than a multiple of 128
// bytes; C is read 16 rows at a time, 8 bytes per row, so its rows are 8
// bytes longer than one.
template <int N>
struct SsdShared {
    static constexpr int RX = kP + 16, RB = N + 16, RC = N + 4;
    alignas(16) uint16_t Xs[kQ][RX];   // x[t][p]
    alignas(16) uint16_t Bs[kQ][RB];   // B[t][n]
    alignas(16) uint16_t Cs[kQ][RC];   // C[t][n]
    alignas(16) uint16_t Mt[6][64][8]; // M^T tile pairs, as the consumers' B operands (lane-major)
    alignas(16) float ecum[kQ];        // exp2(cum_t)
    alignas(16) float wt[kQ];          // w_t
    alignas(16) float pcum[kQ];        // cum_t
    alignas(16) float pdl[kQ];         // delta_t
    float dec;                         // exp2(cum_last)
};

__device__ __forceinline__ s16x4 ld4(const uint16_t *p) { return *(const s16x4 *)__builtin_assume_aligned(p, 8); }
// Transposed operand from a row-major tile: lane l gives the address of row
// 4 (l / 16) + (l % 16) / 4, columns 4 (l % 4) .. + 3 of the tile, and
// receives column l % 16 of rows 4 (l / 16) .. + 3.
__device__ __forceinline__ s16x4 ld_tr(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(__attribute__((address_space(3))) void *)p);
}
__device__ __forceinline__ bf16x8 cat(s16x4 lo, s16x4 hi) {
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ short to_bf16(float v) { return __builtin_bit_cast(short, (__bf16)v); }
__device__ __forceinline__ float from_bf16(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ s16x4 pack4(f32x4 v) {
    return s16x4{to_bf16(v[0]), to_bf16(v[1]), to_bf16(v[2]), to_bf16(v[3])};
}
__device__ __forceinline__ s16x4 scale4(s16x4 x, f32x4 s) {
    s16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = to_bf16(from_bf16((uint16_t)x[e]) * s[e]);
    return r;
}

// v plus the value of lane (lane - S) of its row of 16 (0 below it).
template <int S>
__device__ __forceinline__ float shr_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + S, 0xF, 0xF,
                                                                      false));
}
// Inclusive prefix sum over the 64 lanes: within rows of 16, then the last
// lane of each row carried into the rows after it.
__device__ __forceinline__ float wave_prefix_sum(float v) {
    v = shr_add<1>(v);
    v = shr_add<2>(v);
    v = shr_add<4>(v);
    v = shr_add<8>(v);
    // row_bcast:15 (rows 1 and 3 take lane 15 of the row before), then
    // row_bcast:31 (rows 2 and 3 take lane 31)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
    return v;
}

// v_permlane32_swap (lanes 32-63 of a trade places with lanes 0-31 of b) and
// v_permlane16_swap (the odd 16-lane rows of a trade places with the even
// rows of b), with the wait states a VALU-written source needs.
__device__ __forceinline__ void swap_halves_u(uint32_t &a, uint32_t &b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_odd_even_rows_u(uint32_t &a, uint32_t &b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Index of the M^T tile pair (token tile tt of the output, token tiles 2 pp
// and 2 pp + 1 of the sum) among the six the lower triangle needs.
__host__ __device__ constexpr int mslot(int tt, int pp) { return tt < 2 ? tt : 2 + 2 * (tt - 2) + pp; }

struct Head {
    int64_t b, h, g, nchunks;
};

// Matrix-core layouts of the 16 x 16 x 32 product: lane r + 16 q holds row r
// of the A operand (column r of the B operand) at k = 8 q .. 8 q + 7; result
// element e of lane l is row 4 (l / 16) + e, column l % 16.

// Waves 0 and 1: y and the state of the head-dimension half p0 .. p0 + 31.
template <int N>
__device__ __forceinline__ void consume(SsdShared<N> &sh, const SsdArgs &a, const Head &hd, int w, int l) {
    constexpr int NT = N / 16, KB = N / 32;
    const int j = l & 15, q = l >> 4;
    const int tr_row = 4 * q + j / 4, tr_col = 4 * (j % 4);
    const int64_t H = a.H, L = a.L;
    const int p0 = 32 * w;
    // The state, transposed: tile (nt, pt) holds H^T[16 nt + 4 q + e][p0 + 16 pt + j].
    f32x4 Hacc[NT][2];
    const float *si = a.state_in ? a.state_in + ((hd.b * H + hd.h) * kP + p0 + j) * (int64_t)N + 4 * q : nullptr;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
            Hacc[nt][pt] = si ? *(const f32x4 *)(si + 16 * pt * N + 16 * nt) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    uint16_t *yp = (uint16_t *)a.y;
    for (int64_t c = 0; c < hd.nchunks; ++c) {
        const int64_t t0 = c * kQ;
        lds_barrier();  // x, B, C and the decay factors of the chunk are in LDS
        // x of the half, transposed: xf[ti][pt] = x[16 ti + 4 q + e][p0 + 16 pt + j]
        s16x4 xf[4][2];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) xf[ti][pt] = ld_tr(&sh.Xs[16 * ti + tr_row][p0 + 16 * pt + tr_col]);
        // y^T[p][t]: first (H C^T)[p][t] with K = n, the state as A operand
        f32x4 Y[2][4];
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) Y[pt][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < KB; ++m) {
            bf16x8 hop[2];
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) hop[pt] = cat(pack4(Hacc[2 * m][pt]), pack4(Hacc[2 * m + 1][pt]));
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const uint16_t *cr = &sh.Cs[16 * tt + j][32 * m + 4 * q];
                const bf16x8 cop = cat(ld4(cr), ld4(cr + 16));
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) Y[pt][tt] = mfma32(hop[pt], cop, Y[pt][tt]);
            }
        }
        // the decay since the chunk start, per token (column)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const float ec = sh.ecum[16 * tt + j];
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) Y[pt][tt] *= ec;
        }
        lds_barrier();  // M^T is in LDS
        // then x^T M^T over the lower triangle, K = tokens, pairs of tiles
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int pp = 0; pp <= tt / 2; ++pp) {
                const bf16x8 mop = *(const bf16x8 *)&sh.Mt[mslot(tt, pp)][l][0];
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
                    Y[pt][tt] = mfma32(cat(xf[2 * pp][pt], xf[2 * pp + 1][pt]), mop, Y[pt][tt]);
            }
        }
        // store: element e of tile (pt, tt) is p0 + 16 pt + 4 q + e of token
        // 16 tt + j. Two lane swaps gather p0 + 8 q .. + 7 in lane (q, j), so
        // that each lane stores 16 bytes.
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const u32x2 lv = __builtin_bit_cast(u32x2, pack4(Y[0][tt])), hv = __builtin_bit_cast(u32x2, pack4(Y[1][tt]));
            uint32_t lo0 = lv[0], lo1 = lv[1], hi0 = hv[0], hi1 = hv[1];
            swap_halves_u(lo0, hi0);
            swap_halves_u(lo1, hi1);
            swap_odd_even_rows_u(lo0, hi0);
            swap_odd_even_rows_u(lo1, hi1);
            const int64_t t = t0 + 16 * tt + j;
            if (t < L) *(u32x4 *)(yp + ((hd.b * L + t) * H + hd.h) * kP + p0 + 8 * q) = u32x4{lo0, lo1, hi0, hi1};
        }
        // the state: H^T = exp2(cum_last) H^T + B^T (w o x), K = tokens
        const float dec = sh.dec;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) Hacc[nt][pt] *= dec;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            const f32x4 w0 = *(const f32x4 *)&sh.wt[32 * mm + 4 * q];
            const f32x4 w1 = *(const f32x4 *)&sh.wt[32 * mm + 16 + 4 * q];
            bf16x8 xw[2];
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) xw[pt] = cat(scale4(xf[2 * mm][pt], w0), scale4(xf[2 * mm + 1][pt], w1));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bf16x8 bop = cat(ld_tr(&sh.Bs[32 * mm + tr_row][16 * nt + tr_col]),
                                       ld_tr(&sh.Bs[32 * mm + 16 + tr_row][16 * nt + tr_col]));
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) Hacc[nt][pt] = mfma32(bop, xw[pt], Hacc[nt][pt]);
            }
        }
        lds_barrier();  // every read of the chunk is done
    }
    if (a.state_out) {
        float *so = a.state_out + ((hd.b * H + hd.h) * kP + p0 + j) * (int64_t)N + 4 * q;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) *(f32x4 *)(so + 16 * pt * N + 16 * nt) = Hacc[nt][pt];
    }
}

// Waves 2 (PW = 0) and 3 (PW = 1): the chunk's data and its masked matrix.
// While the consumers work on a chunk, each holds the next chunk's loads in
// registers: wave 2 the B rows, wave 3 the C rows, each half of the x rows,
// all as whole rows (coalesced). Per chunk: barrier B (the consumers are done
// with the chunk before), the rows into LDS, the next chunk's loads, barrier S
// (the chunk is in LDS: the consumers start on H C^T), the G^T tiles from
// LDS, masked and weighted,
// into the M^T pairs, barrier A (M^T is in LDS). Wave 2 also loads delta and
// scans the decay; wave 3 reads the scan from LDS after barrier S. The next
// chunk's loads are issued between the stores and barrier S.
// Wave 2 forms the tiles (s, t) = (0..3, 3) and (0, 0), M^T pairs 0, 4, 5;
// wave 3 forms (0..1, 1) and (0..2, 2), pairs 1, 2, 3.
template <int N, int PW>
__device__ __forceinline__ void prepare(SsdShared<N> &sh, const SsdArgs &a, const Head &hd, int l, float A2,
                                        float dsk) {
    constexpr int KB = N / 32;
    constexpr int PR = N / 8;      // 16-byte pieces per row of Bt or Ct
    constexpr int TPI = 64 / PR;   // rows per load instruction
    constexpr int NR = kQ / TPI;   // load instructions per chunk
    const int j = l & 15, q = l >> 4;
    const int64_t H = a.H, L = a.L, G = a.G;
    u32x4 raw[NR];  // rows TPI i + l / PR of Bt (wave 2) or Ct (wave 3), piece l % PR
    u32x4 xr[4];    // x rows 32 PW + 8 i + l / 8, piece l % 8
    uint16_t dlr = 0;
    float ecv = 0.0f, wv = 0.0f, decv = 0.0f;

    // Tokens past L read token L - 1 (finite values; their delta is taken as
    // 0). Offsets from the chunk's first token are 32-bit: the host keeps 64
    // tokens of x and of Bt, Ct below 4 GiB.
    auto load = [&](int64_t t0) {
        const int64_t rem = L - 1 - t0;
        const uint32_t last = rem < kQ - 1 ? (uint32_t)rem : (uint32_t)(kQ - 1);
        auto tok = [&](uint32_t r) { return r < last ? r : last; };
        const int64_t tokrow = (hd.b * L + t0) * H + hd.h;  // (token t0, head h)
        if constexpr (PW == 0) dlr = ((const uint16_t *)a.delta)[tokrow + tok((uint32_t)l) * (uint32_t)H];
        const uint32_t bs = (uint32_t)(G * N * 2);  // bytes between tokens of Bt, Ct
        const char *src = (const char *)(PW == 0 ? a.Bt : a.Ct) + ((hd.b * L + t0) * G + hd.g) * (N * 2) +
                          16 * (l % PR);
#pragma unroll
        for (int i = 0; i < NR; ++i) raw[i] = *(const u32x4 *)(src + tok(TPI * i + l / PR) * bs);
        const char *xp = (const char *)a.x + tokrow * (kP * 2) + 16 * (l & 7);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            xr[i] = *(const u32x4 *)(xp + tok(32 * PW + 8 * i + (l >> 3)) * (uint32_t)(H * kP * 2));
    };

    // The decay of the chunk at t0, lane = token (wave 2); cum and delta go
    // to LDS for both waves' masks.
    auto decay = [&](int64_t t0) {
        const float dl = t0 + l < L ? from_bf16(dlr) : 0.0f;
        const float cum = wave_prefix_sum(dl * A2);
        const float cl = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cum), 63));
        ecv = fast_exp2(cum);
        wv = dl * fast_exp2(cl - cum);
        decv = fast_exp2(cl);
        sh.pcum[l] = cum;
        sh.pdl[l] = dl;
    };

    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int r = TPI * i + l / PR, c0 = 8 * (l % PR);
            if constexpr (PW == 0) {
                *(u32x4 *)&sh.Bs[r][c0] = raw[i];
            } else {
                *(u32x2 *)&sh.Cs[r][c0] = u32x2{raw[i][0], raw[i][1]};
                *(u32x2 *)&sh.Cs[r][c0 + 4] = u32x2{raw[i][2], raw[i][3]};
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4 *)&sh.Xs[32 * PW + 8 * i + (l >> 3)][8 * (l & 7)] = xr[i];
        if constexpr (PW == 0) {
            sh.ecum[l] = ecv;
            sh.wt[l] = wv;
            if (l == 0) sh.dec = decv;
        }
    };

    // G^T tile (s tile si, t tile tt) of the chunk in LDS: A operand the B
    // rows of the s tile, B operand the C rows of the t tile (cf), both with
    // k = n in order.
    auto cfrag = [&](int tt, bf16x8 (&cf)[KB]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const uint16_t *cr = &sh.Cs[16 * tt + j][32 * kb + 8 * q];
            cf[kb] = cat(ld4(cr), ld4(cr + 4));
        }
    };
    auto gtile = [&](int si, const bf16x8 (&cf)[KB]) {
        f32x4 gt = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) gt = mfma32(*(const bf16x8 *)&sh.Bs[16 * si + j][32 * kb + 8 * q], cf[kb], gt);
        return gt;
    };
    // The decay mask and weight of M^T tile (si, tt), as four bfloat16 per lane.
    auto mask = [&](f32x4 gt, int si, int tt) -> u32x2 {
        const float ct = sh.pcum[16 * tt + j];
        const f32x4 cs = *(const f32x4 *)&sh.pcum[16 * si + 4 * q];
        const f32x4 ds = *(const f32x4 *)&sh.pdl[16 * si + 4 * q];
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = gt[e] * fast_exp2(ct - cs[e]) * ds[e];
            if (si == tt) {
                // the diagonal tile: s <= t only (the select drops any
                // overflow above it), and D on s = t
                v[e] = 4 * q + e <= j ? v[e] : 0.0f;
                if (4 * q + e == j) v[e] += dsk;
            }
        }
        return __builtin_bit_cast(u32x2, pack4(v));
    };
    auto put = [&](int slot, u32x2 lo, u32x2 hi) { *(u32x4 *)&sh.Mt[slot][l][0] = u32x4{lo[0], lo[1], hi[0], hi[1]}; };
    // Every product first (the C fragments of a t tile are read once), then
    // the masks, then the stores.
    auto form = [&]() {
        const u32x2 zero = u32x2{0u, 0u};
        bf16x8 cf[KB];
        if constexpr (PW == 0) {
            cfrag(3, cf);
            const f32x4 g03 = gtile(0, cf), g13 = gtile(1, cf), g23 = gtile(2, cf), g33 = gtile(3, cf);
            cfrag(0, cf);
            const f32x4 g00 = gtile(0, cf);
            const u32x2 m03 = mask(g03, 0, 3), m13 = mask(g13, 1, 3), m23 = mask(g23, 2, 3), m33 = mask(g33, 3, 3);
            const u32x2 m00 = mask(g00, 0, 0);
            put(4, m03, m13);
            put(5, m23, m33);
            put(0, m00, zero);
        } else {
            cfrag(1, cf);
            const f32x4 g01 = gtile(0, cf), g11 = gtile(1, cf);
            cfrag(2, cf);
            const f32x4 g02 = gtile(0, cf), g12 = gtile(1, cf), g22 = gtile(2, cf);
            const u32x2 m01 = mask(g01, 0, 1), m11 = mask(g11, 1, 1), m02 = mask(g02, 0, 2), m12 = mask(g12, 1, 2);
            const u32x2 m22 = mask(g22, 2, 2);
            put(1, m01, m11);
            put(2, m02, m12);
            put(3, m22, zero);
        }
    };

    const int64_t nc = hd.nchunks;
    load(0);
    for (int64_t c = 0; c < nc; ++c) {
        if constexpr (PW == 0) decay(c * kQ);
        if (c > 0) lds_barrier();  // B: the consumers are done with chunk c - 1
        stage();
        // the registers are free only after the stores: keep the loads below them
        __builtin_amdgcn_sched_barrier(0);
        if (c + 1 < nc) load((c + 1) * kQ);
        lds_barrier();  // S: chunk c is in LDS
        form();
        lds_barrier();  // A: its M^T too
    }
    lds_barrier();  // B of the last chunk
}

template <int N>
__global__ __launch_bounds__(kThreads, 3) void ssd_kernel(SsdArgs a) {
    __shared__ SsdShared<N> sh;
    const int l = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, kept scalar
    const int64_t H = a.H, G = a.G;
    // Workgroups are dealt to the 8 XCDs in turn (block id mod 8). When the
    // count divides evenly, XCD x takes the x-th eighth of the (b, h) pairs in
    // order, so the heads of a batch row, which read the same Bt and Ct,
    // share one XCD's L2.
    const int64_t nwg = (int64_t)gridDim.x;
    const int64_t pair = nwg % 8 == 0 ? (int64_t)(blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;
    Head hd;
    hd.b = pair / H;
    hd.h = pair % H;
    hd.g = hd.h / (H / G);
    hd.nchunks = (a.L + kQ - 1) / kQ;
    if (w < 2) {
        consume<N>(sh, a, hd, w, l);
    } else {
        const float A2 = a.A[hd.h] * kLog2e;
        const float dsk = a.Dskip ? a.Dskip[hd.h] : 0.0f;
        if (w == 2) prepare<N, 0>(sh, a, hd, l, A2, dsk);
        else prepare<N, 1>(sh, a, hd, l, A2, dsk);
    }
}

template <int N>
hipError_t launch_ssd_n(const SsdArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((ssd_kernel<N>), dim3((unsigned)(a.batch * a.H)), dim3(kThreads), 0, s, a);
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
