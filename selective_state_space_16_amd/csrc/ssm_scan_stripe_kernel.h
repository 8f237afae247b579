// Selective scan (S6) forward for gfx950, organised by stripes: the kernel and
// its launch, included by the two files that instantiate it (a delta given
// after, and before, its activation).
//
// The recurrence h <- dA*h + dBx runs along the sequence independently for
// every (batch row, channel, state) ("Notas sobre Mamba", section "A varredura
// paralela ciente do hardware": an associative scan over (A-bar_t, B-bar_t
// x_t) pairs, kept on chip, only y written back). Here a wave owns CPW
// channels (16 for N = 16: four rows of 16 lanes, NL = 4 states per lane) and
// walks the tokens of its stripe in order with the state in registers, so the
// scan itself needs no communication at all: per token and state it is one
// exponential, dA*h + B*(delta*x), and C*h accumulated into the readout.
//
// Work units. A workgroup of four waves covers a tile column of TCH = 4*CPW
// channels of one batch row and a stripe of the sequence. When there are at
// least as many tile columns as workgroup slots, a stripe is the whole
// sequence and each unit is one pass. Otherwise every column is cut into S
// stripes that run at the same time, and the carried-in state of a stripe is
// found with the associative composition of affine maps: applying a run of
// tokens to a state is the pair (P, S) with P = exp(A * sum delta) and S the
// run's end state from a zero start. Pass 1 walks the stripe to get its own
// (sum delta, S) and publishes it; a look-back then finds the nearest earlier
// stripe whose end state is out and folds the pairs in between (the chain of
// a handful of records, once per stripe); pass 2 walks the stripe again from
// that state and writes y. Every record is a set of 64-bit words tagged with
// the call's epoch, so a reader can validate each word without flags or
// completion waits. The replay uses the same arithmetic each stripe uses for
// its own end state, so results do not depend on timing.
//
// Long stripes take another order (early mode). The carried-in state enters
// the stripe's states only as exp(A * summed delta) * h_in, which shrinks
// token by token when A <= 0 and delta >= 0 (as the method draws them: A the
// negative exponential of a parameter, delta a softplus). So pass 1 runs the
// whole scan from a zero start, writing y and the (sum delta, S) pair; after
// the look-back, pass 2 walks again from the carried-in state only until, at
// the end of a tile, every lane's decayed carried-in state is below 2^-24
// (float32 outputs: their unit roundoff) or 2^-16 (bfloat16 outputs: 1/256 of
// theirs) times the largest of its states; from there on pass 1's y stands.
// The test is taken from the data alone, so the results do not depend on
// timing either; a lane whose A or delta has the other sign, or whose
// carried-in state is not finite, never passes it.
//
// Memory. Tiles of TT tokens x TCH channels of x, delta (and z, for pass 2),
// and the TT tokens of Bt (and Ct) are loaded into LDS with global_load_lds,
// double-buffered so that the next tile streams in while this one is scanned;
// channel rows are whole 128-byte lines (64 bfloat16 or, as two lines, 64
// float channels). Waves 1..3 issue the loads; wave 0 writes the finished y
// tile back as whole lines, so no wave ever waits for its own stores. A tile
// column's A rows and skip weights live in registers.
//
// Scheduling. Units are handed out from one counter per list (eight lists, a
// workgroup serves the list of its blockIdx modulo 8, i.e. its XCD; tile
// columns are dealt to the lists round robin). Units are handed out in list
// order with the stripes of a column in sequence order, so a stripe only ever
// waits for stripes already held by running workgroups: the launch needs no
// co-residency.
#pragma once

#include <atomic>
#include <cstddef>

#include "ssm_common.h"
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kWaves = 4;   // waves per workgroup (one per channel group)
constexpr int kLists = 8;   // unit lists (one per XCD of an MI355X)
constexpr int kReplay = 4;  // stripe records loaded per round trip of a look-back replay
constexpr int kSlotsPerList = 64;  // workgroups a list is planned for (2 per CU on 256 CUs)
constexpr int64_t kEarlyMinTokens = 16384;  // stripes at least this long take early mode
// options of a stripe walk: sum delta, track its minimum, stop early
constexpr int kSum = 1, kMin = 2, kStop = 4;

// dot_row for four states per lane when `c` came straight from an LDS read
// (the high-half loads): a DPP read needs no wait states after an LDS read,
// only after a VALU write, so the s_nop of dot_row is left out.
template <int S0>
__device__ __forceinline__ void dot_row_lds(float &acc, float c, const float (&h)[4]) {
    asm volatile("v_mul_f32_dpp %0, %1, %2 row_newbcast:%6 row_mask:0xf bank_mask:0xf"
                 "\n\tv_fmac_f32_dpp %0, %1, %3 row_newbcast:%7 row_mask:0xf bank_mask:0xf"
                 "\n\tv_fmac_f32_dpp %0, %1, %4 row_newbcast:%8 row_mask:0xf bank_mask:0xf"
                 "\n\tv_fmac_f32_dpp %0, %1, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf"
                 : "=&v"(acc)
                 : "v"(c), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "i"(S0), "i"(S0 + 1), "i"(S0 + 2),
                   "i"(S0 + 3));
}

// swap_halves(a0, a2) and swap_halves(a1, a3) behind one pair of wait states
// (the second swap's sources are older than the first's).
__device__ __forceinline__ void swap_halves2(float &a0, float &a2, float &a1, float &a3) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3"
                 : "+v"(a0), "+v"(a2), "+v"(a1), "+v"(a3));
}

template <int N, int DT>
struct Geo {
    using T = typename Act<DT>::T;
    static constexpr int NL = N < 4 ? N : 4;       // states per lane
    static constexpr int NGR = N / NL;             // rows per channel
    static constexpr int CPW = (4 / NGR) * 16;     // channels per wave
    static constexpr int TCH = kWaves * CPW;       // channels per tile column
    static constexpr int TPV = 16 / NL;            // tokens per broadcast register
    static constexpr int GROUP = TPV > 8 ? TPV : 8;  // tokens per register group
    static constexpr int BREGS = GROUP / TPV;      // broadcast registers per group
    static constexpr int OWN = GROUP / NGR;        // tokens of a group each lane finishes
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int VEC = 16 / ESZ;           // elements per 16-byte piece
    // tokens per tile: three activation tiles of at most 24 KB
    static constexpr int TT_RAW = 8192 / (TCH * ESZ);
    static constexpr int TT = TT_RAW < 16 ? 16 : (TT_RAW > 64 ? 64 : TT_RAW);
    static constexpr int PPR = TCH / VEC;           // pieces per tile row
    static constexpr int ACT_PIECES = TT * PPR;     // pieces per activation tile (a multiple of 64)
    static constexpr int BC_PIECES = TT * N / VEC;  // pieces per Bt/Ct tile
    static constexpr int BC_SLOTS = (BC_PIECES + 63) / 64 * 64;
    static_assert(ACT_PIECES % 64 == 0, "activation tiles are loaded in whole waves of pieces");
};

// An LDS array of R rows of C elements that exists only when ON: otherwise
// an empty member that takes no space, so that the buffers of the modes
// without it keep their layout.
template <class E, int R, int C, bool ON>
struct OptRows {
    alignas(16) E v[R][C];
};
template <class E, int R, int C>
struct OptRows<E, R, C, false> {};

// TRAP: the exponential-trapezoidal rule, which also needs the weight lam of
// each token and the delta and lam of the token after the tile. CONV: the x
// branch ahead of the scan; x holds the raw input and xc the tile's x after
// the convolution and SiLU, which the scan reads.
template <int N, int DT, bool TRAP = false, bool CONV = false>
struct TileBuf {
    using G = Geo<N, DT>;
    using T = typename G::T;
    // 16-byte aligned: pieces land here as whole 16-byte writes and y is read
    // back as 16-byte reads
    alignas(16) T x[G::TT][G::TCH];
    // delta; pass 2 writes y here once a token's delta is used. TRAP: row TT
    // holds the token after the tile.
    alignas(16) T dl[G::TT + (TRAP ? 1 : 0)][G::TCH];
    alignas(16) T z[G::TT][G::TCH];
    alignas(16) T B[G::BC_SLOTS * G::VEC];  // Bt rows of the tile's tokens (padded to whole waves of pieces)
    alignas(16) T C[G::BC_SLOTS * G::VEC];
    alignas(16) T lam[TRAP ? G::TT + 1 : 1][TRAP ? G::TCH : G::VEC];  // TRAP: rows as dl (else a stub)
    [[no_unique_address]] OptRows<T, G::TT, G::TCH, CONV> xc;  // CONV: rows as x
};

template <int N, int DT, bool TRAP = false, bool CONV = false>
struct Shared {
    TileBuf<N, DT, TRAP, CONV> buf[2];
    float cb[TRAP ? Geo<N, DT>::TT : 1];  // TRAP, pass 2: sum_n Ct[t,n] Bt[t,n] per token of the current tile
    // CONV: the taps (rows 0..3) and the bias (row 4) of the unit's channels
    [[no_unique_address]] OptRows<float, 5, Geo<N, DT>::TCH, CONV> cw;
    int unit;      // the unit handed to this workgroup
    uint32_t tag;  // this call's tag (see kHdrEpoch)
    int stop[2][kWaves];  // early mode, pass 2: each wave's vote to stop, by tile parity
};

template <int N, int DT, bool TRAP, bool CONV = false>
constexpr int stripe_min_blocks() { return 2 * sizeof(Shared<N, DT, TRAP, CONV>) <= 160 * 1024 ? 2 : 1; }

// An activation element of an LDS tile row, widened to float. A bfloat16 is
// read as the 32-bit word holding it and its neighbour, and moved into the
// high half of the result with one byte permute (`sel` depends only on the
// element's parity): the loads then go straight to their own registers.
__device__ __forceinline__ float lds_act(const float *row, int i, uint32_t) { return row[i]; }
__device__ __forceinline__ float lds_act(const uint16_t *row, int i, uint32_t sel) {
    const uint32_t w = reinterpret_cast<const uint32_t *>(row)[i >> 1];
    return __uint_as_float(__builtin_amdgcn_perm(w, w, sel));
}
// Byte selector of lds_act for an element of this parity: bytes 1,0 (even) or
// 3,2 (odd) of the word into bytes 3,2 of the result, zeros below.
__device__ __forceinline__ uint32_t half_sel(int i) { return (i & 1) ? 0x03020c0cu : 0x01000c0cu; }

// bfloat16 reads of an LDS tile straight into the high half of a register
// whose low half is zero (it last held a value read this way, or 0.0f): the
// register then holds the exact float, with no VALU work (the compiler does
// not form these loads itself). Each block waits for its own loads, so no
// register is read while its load is in flight. Addresses are a per-lane LDS
// byte address plus immediate offsets, so a fully unrolled walk over a tile
// needs no address arithmetic.
//
// Pass-1 loads of one 8-token group (bfloat16, state size 16): x and delta of
// the 8 tokens (b0 + OX / OD + k * ROWB) and the two Bt registers (b1 + OB +
// {0, SB}), as one block with one wait.
template <int ROWB, int OX, int OD, int SB, int OB>
__device__ __forceinline__ void lds_bf16_p1(float (&xv)[8], float (&dv)[8], float (&bq)[2], uint32_t b0,
                                            uint32_t b1) {
    asm volatile(
        "ds_read_u16_d16_hi %0, %18 offset:%20\n\tds_read_u16_d16_hi %1, %18 offset:%21\n\t"
        "ds_read_u16_d16_hi %2, %18 offset:%22\n\tds_read_u16_d16_hi %3, %18 offset:%23\n\t"
        "ds_read_u16_d16_hi %4, %18 offset:%24\n\tds_read_u16_d16_hi %5, %18 offset:%25\n\t"
        "ds_read_u16_d16_hi %6, %18 offset:%26\n\tds_read_u16_d16_hi %7, %18 offset:%27\n\t"
        "ds_read_u16_d16_hi %8, %18 offset:%28\n\tds_read_u16_d16_hi %9, %18 offset:%29\n\t"
        "ds_read_u16_d16_hi %10, %18 offset:%30\n\tds_read_u16_d16_hi %11, %18 offset:%31\n\t"
        "ds_read_u16_d16_hi %12, %18 offset:%32\n\tds_read_u16_d16_hi %13, %18 offset:%33\n\t"
        "ds_read_u16_d16_hi %14, %18 offset:%34\n\tds_read_u16_d16_hi %15, %18 offset:%35\n\t"
        "ds_read_u16_d16_hi %16, %19 offset:%36\n\tds_read_u16_d16_hi %17, %19 offset:%37\n\t"
        "s_waitcnt lgkmcnt(0)"
        :"+v"(xv[0]), "+v"(xv[1]), "+v"(xv[2]), "+v"(xv[3]), "+v"(xv[4]), "+v"(xv[5]), "+v"(xv[6]), "+v"(xv[7]), "+v"(dv[0]),
         "+v"(dv[1]), "+v"(dv[2]), "+v"(dv[3]), "+v"(dv[4]), "+v"(dv[5]), "+v"(dv[6]), "+v"(dv[7]), "+v"(bq[0]), "+v"(bq[1])
        :"v"(b0), "v"(b1), "i"(OX), "i"(OX + 1 * ROWB), "i"(OX + 2 * ROWB), "i"(OX + 3 * ROWB), "i"(OX + 4 * ROWB),
         "i"(OX + 5 * ROWB), "i"(OX + 6 * ROWB), "i"(OX + 7 * ROWB), "i"(OD), "i"(OD + 1 * ROWB), "i"(OD + 2 * ROWB),
         "i"(OD + 3 * ROWB), "i"(OD + 4 * ROWB), "i"(OD + 5 * ROWB), "i"(OD + 6 * ROWB), "i"(OD + 7 * ROWB), "i"(OB),
         "i"(OB + 1 * SB)
        : "memory");
}

// Pass-2 loads of one 8-token group: as lds_bf16_p1, plus the Ct registers
// (b1 + OC + {0, SB}) and x and z of the two tokens this lane finishes
// (b2 + OXO / OZO + {0, SO}).
template <int ROWB, int OX, int OD, int SB, int OB, int OC, int SO, int OXO, int OZO>
__device__ __forceinline__ void lds_bf16_p2(float (&xv)[8], float (&dv)[8], float (&bq)[2], float (&cq)[2],
                                            float (&xo)[2], float (&zo)[2], uint32_t b0, uint32_t b1, uint32_t b2) {
    asm volatile(
        "ds_read_u16_d16_hi %0, %24 offset:%27\n\tds_read_u16_d16_hi %1, %24 offset:%28\n\t"
        "ds_read_u16_d16_hi %2, %24 offset:%29\n\tds_read_u16_d16_hi %3, %24 offset:%30\n\t"
        "ds_read_u16_d16_hi %4, %24 offset:%31\n\tds_read_u16_d16_hi %5, %24 offset:%32\n\t"
        "ds_read_u16_d16_hi %6, %24 offset:%33\n\tds_read_u16_d16_hi %7, %24 offset:%34\n\t"
        "ds_read_u16_d16_hi %8, %24 offset:%35\n\tds_read_u16_d16_hi %9, %24 offset:%36\n\t"
        "ds_read_u16_d16_hi %10, %24 offset:%37\n\tds_read_u16_d16_hi %11, %24 offset:%38\n\t"
        "ds_read_u16_d16_hi %12, %24 offset:%39\n\tds_read_u16_d16_hi %13, %24 offset:%40\n\t"
        "ds_read_u16_d16_hi %14, %24 offset:%41\n\tds_read_u16_d16_hi %15, %24 offset:%42\n\t"
        "ds_read_u16_d16_hi %16, %25 offset:%43\n\tds_read_u16_d16_hi %17, %25 offset:%44\n\t"
        "ds_read_u16_d16_hi %18, %25 offset:%45\n\tds_read_u16_d16_hi %19, %25 offset:%46\n\t"
        "ds_read_u16_d16_hi %20, %26 offset:%47\n\tds_read_u16_d16_hi %21, %26 offset:%48\n\t"
        "ds_read_u16_d16_hi %22, %26 offset:%49\n\tds_read_u16_d16_hi %23, %26 offset:%50\n\t"
        "s_waitcnt lgkmcnt(0)"
        :"+v"(xv[0]), "+v"(xv[1]), "+v"(xv[2]), "+v"(xv[3]), "+v"(xv[4]), "+v"(xv[5]), "+v"(xv[6]), "+v"(xv[7]), "+v"(dv[0]),
         "+v"(dv[1]), "+v"(dv[2]), "+v"(dv[3]), "+v"(dv[4]), "+v"(dv[5]), "+v"(dv[6]), "+v"(dv[7]), "+v"(bq[0]), "+v"(bq[1]),
         "+v"(cq[0]), "+v"(cq[1]), "+v"(xo[0]), "+v"(xo[1]), "+v"(zo[0]), "+v"(zo[1])
        :"v"(b0), "v"(b1), "v"(b2), "i"(OX), "i"(OX + 1 * ROWB), "i"(OX + 2 * ROWB), "i"(OX + 3 * ROWB), "i"(OX + 4 * ROWB),
         "i"(OX + 5 * ROWB), "i"(OX + 6 * ROWB), "i"(OX + 7 * ROWB), "i"(OD), "i"(OD + 1 * ROWB), "i"(OD + 2 * ROWB),
         "i"(OD + 3 * ROWB), "i"(OD + 4 * ROWB), "i"(OD + 5 * ROWB), "i"(OD + 6 * ROWB), "i"(OD + 7 * ROWB), "i"(OB),
         "i"(OB + 1 * SB), "i"(OC), "i"(OC + 1 * SB), "i"(OXO), "i"(OXO + 1 * SO), "i"(OZO), "i"(OZO + 1 * SO)
        : "memory");
}

// Trapezoidal rule, pass 1: as lds_bf16_p1, plus lam of the 8 tokens (b0 +
// OL + k * ROWB) and delta and lam of the token after them (b0 + OD / OL + 8 *
// ROWB).
template <int ROWB, int OX, int OD, int OL, int SB, int OB>
__device__ __forceinline__ void lds_bf16_t1(float (&xv)[8], float (&dv)[8], float (&lv)[8], float &dn, float &ln,
                                            float (&bq)[2], uint32_t b0, uint32_t b1) {
    asm volatile(
        "ds_read_u16_d16_hi %0, %28 offset:%30\n\tds_read_u16_d16_hi %1, %28 offset:%31\n\t"
        "ds_read_u16_d16_hi %2, %28 offset:%32\n\tds_read_u16_d16_hi %3, %28 offset:%33\n\t"
        "ds_read_u16_d16_hi %4, %28 offset:%34\n\tds_read_u16_d16_hi %5, %28 offset:%35\n\t"
        "ds_read_u16_d16_hi %6, %28 offset:%36\n\tds_read_u16_d16_hi %7, %28 offset:%37\n\t"
        "ds_read_u16_d16_hi %8, %28 offset:%38\n\tds_read_u16_d16_hi %9, %28 offset:%39\n\t"
        "ds_read_u16_d16_hi %10, %28 offset:%40\n\tds_read_u16_d16_hi %11, %28 offset:%41\n\t"
        "ds_read_u16_d16_hi %12, %28 offset:%42\n\tds_read_u16_d16_hi %13, %28 offset:%43\n\t"
        "ds_read_u16_d16_hi %14, %28 offset:%44\n\tds_read_u16_d16_hi %15, %28 offset:%45\n\t"
        "ds_read_u16_d16_hi %16, %28 offset:%46\n\tds_read_u16_d16_hi %17, %28 offset:%47\n\t"
        "ds_read_u16_d16_hi %18, %28 offset:%48\n\tds_read_u16_d16_hi %19, %28 offset:%49\n\t"
        "ds_read_u16_d16_hi %20, %28 offset:%50\n\tds_read_u16_d16_hi %21, %28 offset:%51\n\t"
        "ds_read_u16_d16_hi %22, %28 offset:%52\n\tds_read_u16_d16_hi %23, %28 offset:%53\n\t"
        "ds_read_u16_d16_hi %24, %28 offset:%54\n\tds_read_u16_d16_hi %25, %28 offset:%55\n\t"
        "ds_read_u16_d16_hi %26, %29 offset:%56\n\tds_read_u16_d16_hi %27, %29 offset:%57\n\t"
        "s_waitcnt lgkmcnt(0)"
        :"+v"(xv[0]), "+v"(xv[1]), "+v"(xv[2]), "+v"(xv[3]), "+v"(xv[4]), "+v"(xv[5]), "+v"(xv[6]), "+v"(xv[7]), "+v"(dv[0]),
         "+v"(dv[1]), "+v"(dv[2]), "+v"(dv[3]), "+v"(dv[4]), "+v"(dv[5]), "+v"(dv[6]), "+v"(dv[7]), "+v"(lv[0]), "+v"(lv[1]),
         "+v"(lv[2]), "+v"(lv[3]), "+v"(lv[4]), "+v"(lv[5]), "+v"(lv[6]), "+v"(lv[7]), "+v"(dn), "+v"(ln), "+v"(bq[0]),
         "+v"(bq[1])
        :"v"(b0), "v"(b1), "i"(OX), "i"(OX + 1 * ROWB), "i"(OX + 2 * ROWB), "i"(OX + 3 * ROWB), "i"(OX + 4 * ROWB),
         "i"(OX + 5 * ROWB), "i"(OX + 6 * ROWB), "i"(OX + 7 * ROWB), "i"(OD), "i"(OD + 1 * ROWB), "i"(OD + 2 * ROWB),
         "i"(OD + 3 * ROWB), "i"(OD + 4 * ROWB), "i"(OD + 5 * ROWB), "i"(OD + 6 * ROWB), "i"(OD + 7 * ROWB), "i"(OL),
         "i"(OL + 1 * ROWB), "i"(OL + 2 * ROWB), "i"(OL + 3 * ROWB), "i"(OL + 4 * ROWB), "i"(OL + 5 * ROWB),
         "i"(OL + 6 * ROWB), "i"(OL + 7 * ROWB), "i"(OD + 8 * ROWB), "i"(OL + 8 * ROWB), "i"(OB), "i"(OB + 1 * SB)
        : "memory");
}

// Trapezoidal rule, pass 2: as lds_bf16_t1, plus the Ct registers, x and z of
// the two finished tokens and delta and lam of the token after each (b2 +
// OXO / OZO / ODO / OLO + {0, SO}), and the float C . B of each finished token
// (b3 + OCB + {0, SCB}).
template <int ROWB, int OX, int OD, int OL, int SB, int OB, int OC, int SO, int OXO, int OZO, int ODO, int OLO, int SCB, int OCB>
__device__ __forceinline__ void lds_bf16_t2(float (&xv)[8], float (&dv)[8], float (&lv)[8], float &dn, float &ln,
                                            float (&bq)[2], float (&cq)[2], float (&xo)[2], float (&zo)[2],
                                            float (&dno)[2], float (&lno)[2], float (&cbo)[2], uint32_t b0,
                                            uint32_t b1, uint32_t b2, uint32_t b3) {
    asm volatile(
        "ds_read_u16_d16_hi %0, %40 offset:%44\n\tds_read_u16_d16_hi %1, %40 offset:%45\n\t"
        "ds_read_u16_d16_hi %2, %40 offset:%46\n\tds_read_u16_d16_hi %3, %40 offset:%47\n\t"
        "ds_read_u16_d16_hi %4, %40 offset:%48\n\tds_read_u16_d16_hi %5, %40 offset:%49\n\t"
        "ds_read_u16_d16_hi %6, %40 offset:%50\n\tds_read_u16_d16_hi %7, %40 offset:%51\n\t"
        "ds_read_u16_d16_hi %8, %40 offset:%52\n\tds_read_u16_d16_hi %9, %40 offset:%53\n\t"
        "ds_read_u16_d16_hi %10, %40 offset:%54\n\tds_read_u16_d16_hi %11, %40 offset:%55\n\t"
        "ds_read_u16_d16_hi %12, %40 offset:%56\n\tds_read_u16_d16_hi %13, %40 offset:%57\n\t"
        "ds_read_u16_d16_hi %14, %40 offset:%58\n\tds_read_u16_d16_hi %15, %40 offset:%59\n\t"
        "ds_read_u16_d16_hi %16, %40 offset:%60\n\tds_read_u16_d16_hi %17, %40 offset:%61\n\t"
        "ds_read_u16_d16_hi %18, %40 offset:%62\n\tds_read_u16_d16_hi %19, %40 offset:%63\n\t"
        "ds_read_u16_d16_hi %20, %40 offset:%64\n\tds_read_u16_d16_hi %21, %40 offset:%65\n\t"
        "ds_read_u16_d16_hi %22, %40 offset:%66\n\tds_read_u16_d16_hi %23, %40 offset:%67\n\t"
        "ds_read_u16_d16_hi %24, %40 offset:%68\n\tds_read_u16_d16_hi %25, %40 offset:%69\n\t"
        "ds_read_u16_d16_hi %26, %41 offset:%70\n\tds_read_u16_d16_hi %27, %41 offset:%71\n\t"
        "ds_read_u16_d16_hi %28, %41 offset:%72\n\tds_read_u16_d16_hi %29, %41 offset:%73\n\t"
        "ds_read_u16_d16_hi %30, %42 offset:%74\n\tds_read_u16_d16_hi %31, %42 offset:%75\n\t"
        "ds_read_u16_d16_hi %32, %42 offset:%76\n\tds_read_u16_d16_hi %33, %42 offset:%77\n\t"
        "ds_read_u16_d16_hi %34, %42 offset:%78\n\tds_read_u16_d16_hi %35, %42 offset:%79\n\t"
        "ds_read_u16_d16_hi %36, %42 offset:%80\n\tds_read_u16_d16_hi %37, %42 offset:%81\n\t"
        "ds_read_b32 %38, %43 offset:%82\n\tds_read_b32 %39, %43 offset:%83\n\ts_waitcnt lgkmcnt(0)"
        :"+v"(xv[0]), "+v"(xv[1]), "+v"(xv[2]), "+v"(xv[3]), "+v"(xv[4]), "+v"(xv[5]), "+v"(xv[6]), "+v"(xv[7]), "+v"(dv[0]),
         "+v"(dv[1]), "+v"(dv[2]), "+v"(dv[3]), "+v"(dv[4]), "+v"(dv[5]), "+v"(dv[6]), "+v"(dv[7]), "+v"(lv[0]), "+v"(lv[1]),
         "+v"(lv[2]), "+v"(lv[3]), "+v"(lv[4]), "+v"(lv[5]), "+v"(lv[6]), "+v"(lv[7]), "+v"(dn), "+v"(ln), "+v"(bq[0]),
         "+v"(bq[1]), "+v"(cq[0]), "+v"(cq[1]), "+v"(xo[0]), "+v"(xo[1]), "+v"(zo[0]), "+v"(zo[1]), "+v"(dno[0]),
         "+v"(dno[1]), "+v"(lno[0]), "+v"(lno[1]), "=&v"(cbo[0]), "=&v"(cbo[1])
        :"v"(b0), "v"(b1), "v"(b2), "v"(b3), "i"(OX), "i"(OX + 1 * ROWB), "i"(OX + 2 * ROWB), "i"(OX + 3 * ROWB),
         "i"(OX + 4 * ROWB), "i"(OX + 5 * ROWB), "i"(OX + 6 * ROWB), "i"(OX + 7 * ROWB), "i"(OD), "i"(OD + 1 * ROWB),
         "i"(OD + 2 * ROWB), "i"(OD + 3 * ROWB), "i"(OD + 4 * ROWB), "i"(OD + 5 * ROWB), "i"(OD + 6 * ROWB),
         "i"(OD + 7 * ROWB), "i"(OL), "i"(OL + 1 * ROWB), "i"(OL + 2 * ROWB), "i"(OL + 3 * ROWB), "i"(OL + 4 * ROWB),
         "i"(OL + 5 * ROWB), "i"(OL + 6 * ROWB), "i"(OL + 7 * ROWB), "i"(OD + 8 * ROWB), "i"(OL + 8 * ROWB), "i"(OB),
         "i"(OB + 1 * SB), "i"(OC), "i"(OC + 1 * SB), "i"(OXO), "i"(OXO + 1 * SO), "i"(OZO), "i"(OZO + 1 * SO), "i"(ODO),
         "i"(ODO + 1 * SO), "i"(OLO), "i"(OLO + 1 * SO), "i"(OCB), "i"(OCB + 1 * SCB)
        : "memory");
}

// An empty volatile statement that reads and rewrites `st` and `x`: every
// computation of those values comes before it and every use after it, and it
// stays in order with the other volatile statements (the tile loads).
template <int NL>
__device__ __forceinline__ void order_point(float (&st)[NL], float &x) {
    if constexpr (NL == 4) asm volatile("" : "+v"(st[0]), "+v"(st[1]), "+v"(st[2]), "+v"(st[3]), "+v"(x));
    else if constexpr (NL == 2) asm volatile("" : "+v"(st[0]), "+v"(st[1]), "+v"(x));
    else asm volatile("" : "+v"(st[0]), "+v"(x));
}

__device__ __forceinline__ uint32_t take_unit(uint32_t *ctr) {
    return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The per-piece path of load_tile_w, with addresses clamped into the sequence.
template <int N, int DT, int NACT, int NBC, bool HAS_Z, bool TRAP, class TB>
__device__ __forceinline__ void load_tile_clamped(TB &tb, const StripeArgs &a, int64_t b,
                                                  int64_t ch0, int64_t tt0, int w, int lane) {
    using G = Geo<N, DT>;
    using T = typename G::T;
    const int64_t D = a.D, L = a.L;
    for (int base = (w - 1) * 64; base < NACT * G::ACT_PIECES; base += 3 * 64) {
        const int arr = base / G::ACT_PIECES;
        const int pa = base - arr * G::ACT_PIECES + lane;
        const int r = pa / G::PPR, c = (pa % G::PPR) * G::VEC;
        int64_t t = tt0 + r;
        t = t < L ? t : L - 1;
        int64_t ch = ch0 + c;
        ch = ch + G::VEC <= D ? ch : D - G::VEC;
        const bool is_z = arr == 2 && HAS_Z;
        const T *src = arr == 0 ? (const T *)a.x : arr == 1 ? (const T *)a.delta : is_z ? (const T *)a.z : (const T *)a.lam;
        T *dst = arr == 0 ? &tb.x[0][0] : arr == 1 ? &tb.dl[0][0] : is_z ? &tb.z[0][0] : &tb.lam[0][0];
        dma16(src + (b * L + t) * D + ch, lds_addr(dst + (int64_t)(base - arr * G::ACT_PIECES) * G::VEC));
    }
    for (int base = (w - 1) * 64; base < NBC * G::BC_SLOTS; base += 3 * 64) {
        const int arr = base / G::BC_SLOTS;
        int pq = base - arr * G::BC_SLOTS + lane;
        pq = pq < G::BC_PIECES ? pq : G::BC_PIECES - 1;  // padding slots repeat the last piece
        const int r = pq * G::VEC / N, c = pq * G::VEC % N;
        int64_t t = tt0 + r;
        t = t < L ? t : L - 1;
        const T *src = arr == 0 ? (const T *)a.Bt : (const T *)a.Ct;
        T *dst = arr == 0 ? tb.B : tb.C;
        dma16(src + (b * L + t) * N + c, lds_addr(dst + (int64_t)(base - arr * G::BC_SLOTS) * G::VEC));
    }
}

// Load the tile of TT tokens starting at tt0 of tile column (b, ch0) into
// LDS, spread over waves 1..3. Pass 1 needs x, delta and Bt; pass 2 also z
// and Ct. Each wave moves slots of 64 16-byte pieces; a slot of an activation
// array covers whole tile rows, so a piece's address is a wave-uniform row
// address (SGPRs) plus the lane's offset within the slot, `act_off`, which is
// the same for every tile of a unit. Only the last tile of a sequence, whose
// rows may run past L, takes the per-piece path: pieces past the end of the
// sequence are read from the last token instead, and the tokens are given
// delta = 0 afterwards. Channels past D (a last, partial column) are read
// from the last whole piece of the row and never stored. TRAP adds lam, and
// the delta (wave 1) and lam (wave 2) row of the token after the tile, read
// from the last token when there is none.
template <int N, int DT, bool GATE, int PASS, int WV, bool TRAP, class TB>
__device__ __forceinline__ void load_tile_w(TB &tb, const StripeArgs &a, int64_t b, int64_t ch0,
                                            int64_t tt0, int lane, uint32_t act_off) {
    using G = Geo<N, DT>;
    using T = typename G::T;
    constexpr bool HAS_Z = PASS == 2 && GATE;
    constexpr int NACT = 2 + (HAS_Z ? 1 : 0) + (TRAP ? 1 : 0);  // x, delta, [z], [lam]
    constexpr int NBC = PASS == 2 ? 2 : 1;
    const int64_t D = a.D, L = a.L;
    if (tt0 + G::TT <= L) {
        const uint32_t rowb = (uint32_t)(D * G::ESZ);
        const int64_t off = ((b * L + tt0) * D + ch0) * G::ESZ;
        const uint32_t lds_tb = lds_addr(&tb);
        // the wave's slots: pieces (WV - 1) * 64 + 192 * k
        static_for<0, (NACT * G::ACT_PIECES - (WV - 1) * 64 + 191) / 192>([&](auto kc) {
            constexpr int base = (WV - 1) * 64 + 192 * decltype(kc)::value;
            constexpr int arr = base / G::ACT_PIECES;
            constexpr int pa0 = base - arr * G::ACT_PIECES;  // first piece of the slot
            constexpr bool is_z = arr == 2 && HAS_Z;
            const void *p = arr == 0 ? a.x : arr == 1 ? a.delta : is_z ? a.z : a.lam;
            constexpr int dst = (arr == 0   ? offsetof(TB, x)
                                 : arr == 1 ? offsetof(TB, dl)
                                 : is_z     ? offsetof(TB, z)
                                            : offsetof(TB, lam)) +
                                pa0 * 16;
            dma16_s((const char *)p + off + (uint64_t)(pa0 / G::PPR) * rowb, act_off, lds_tb + dst);
        });
        const int64_t boff = (b * L + tt0) * N * G::ESZ;
        static_for<0, (NBC * G::BC_SLOTS - (WV - 1) * 64 + 191) / 192>([&](auto kc) {
            constexpr int base = (WV - 1) * 64 + 192 * decltype(kc)::value;
            constexpr int arr = base / G::BC_SLOTS;
            constexpr int pq0 = base - arr * G::BC_SLOTS;
            const int pq = pq0 + lane < G::BC_PIECES ? pq0 + lane : G::BC_PIECES - 1;  // padding repeats the last piece
            constexpr int dst = (arr == 0 ? offsetof(TB, B) : offsetof(TB, C)) + pq0 * 16;
            dma16_s((const char *)(arr == 0 ? a.Bt : a.Ct) + boff, (uint32_t)pq * 16, lds_tb + dst);
        });
    } else {
        load_tile_clamped<N, DT, NACT, NBC, HAS_Z, TRAP>(tb, a, b, ch0, tt0, WV, lane);
    }
    if constexpr (TRAP && (WV == 1 || WV == 2)) {
        if (lane < G::PPR) {
            int64_t t = tt0 + G::TT;
            t = t < L ? t : L - 1;
            int64_t ch = ch0 + (int64_t)lane * G::VEC;
            ch = ch + G::VEC <= D ? ch : D - G::VEC;
            const T *src = WV == 1 ? (const T *)a.delta : (const T *)a.lam;
            dma16(src + (b * L + t) * D + ch, lds_addr(WV == 1 ? &tb.dl[G::TT][0] : &tb.lam[G::TT][0]));
        }
    }
}

template <int N, int DT, bool GATE, int PASS, bool TRAP, class TB>
__device__ __forceinline__ void load_tile(TB &tb, const StripeArgs &a, int64_t b, int64_t ch0,
                                          int64_t tt0, int w, int lane, uint32_t act_off) {
    if (w == 1) load_tile_w<N, DT, GATE, PASS, 1, TRAP>(tb, a, b, ch0, tt0, lane, act_off);
    else if (w == 2) load_tile_w<N, DT, GATE, PASS, 2, TRAP>(tb, a, b, ch0, tt0, lane, act_off);
    else load_tile_w<N, DT, GATE, PASS, 3, TRAP>(tb, a, b, ch0, tt0, lane, act_off);
}

// Step-size activation for a raw step: once a tile has landed, the
// workgroup's threads share its delta pieces (piece p goes to thread
// p mod 256) and replace each value by softplus(delta + dt_bias), so every
// (token, channel) is activated once. A thread's pieces all sit in the same
// piece column (256 is a multiple of the pieces per row), so `dtb` holds the
// bias of its VEC channels.
template <int N, int DT, class TB>
__device__ __forceinline__ void activate_delta(TB &tb, const float (&dtb)[Geo<N, DT>::VEC]) {
    using G = Geo<N, DT>;
    using T = typename G::T;
    using VT = uint32_t __attribute__((ext_vector_type(4)));
    static_assert((64 * kWaves) % G::PPR == 0, "a thread's pieces share one column");
    static_assert(G::ACT_PIECES % (64 * kWaves) == 0, "every thread has the same number of pieces");
#pragma unroll
    for (int k0 = 0; k0 < G::ACT_PIECES / (64 * kWaves); ++k0) {
        T *p = &tb.dl[0][0] + (int64_t)(threadIdx.x + k0 * 64 * kWaves) * G::VEC;
        VT v = *(const VT *)__builtin_assume_aligned(p, 16);
        T e[G::VEC];
        __builtin_memcpy(e, &v, sizeof(v));
#pragma unroll
        for (int k = 0; k < G::VEC; ++k) {
            const float f = softplus(ld_act(e, k) + dtb[k]);
            if constexpr (DT == 0) e[k] = f;
            else e[k] = __builtin_bit_cast(uint16_t, (__bf16)f);
        }
        __builtin_memcpy(&v, e, sizeof(v));
        *(VT *)__builtin_assume_aligned(p, 16) = v;
    }
}

// The x branch ahead of the scan, once a tile has landed: xc = SiLU of the
// causal width-4 convolution of the raw x rows, per channel. A thread takes
// one channel over RPT consecutive rows, so every LDS access of a wave covers
// one row of 64 channels (no bank conflicts); it reads the three rows before
// its own too, all in one round. Rows before the tile are the last three raw
// rows of `prev`, the other buffer, which holds the previous tile (its next
// load is issued only after the barrier that follows this) or, for the first
// tile of a pass, the raw x of the three tokens before the stripe (staged by
// the walk). Writes go to xc only, so no thread overwrites a row another
// still reads. `cw` holds the taps and bias of the tile column's channels.
template <int N, int DT, class TB>
__device__ __forceinline__ void conv_tile(TB &tb, const TB &prev, const float (&cw)[5][Geo<N, DT>::TCH]) {
    using G = Geo<N, DT>;
    constexpr int TCH = G::TCH, TT = G::TT;
    constexpr int TPC = 64 * kWaves / TCH;  // threads per channel
    constexpr int RPT = TT / TPC;           // rows per thread
    static_assert((64 * kWaves) % TCH == 0 && TT % TPC == 0, "whole rows per thread");
    const int c = threadIdx.x % TCH, r0 = (threadIdx.x / TCH) * RPT;
    float raw[RPT + 3];
#pragma unroll
    for (int k = 0; k < RPT + 3; ++k) {
        const int r = r0 - 3 + k;
        raw[k] = ld_act(r >= 0 ? &tb.x[r][0] : &prev.x[TT + r][0], c);
    }
    const float w0 = cw[0][c], w1 = cw[1][c], w2 = cw[2][c], w3 = cw[3][c], bias = cw[4][c];
#pragma unroll
    for (int k = 0; k < RPT; ++k)
        st_act(&tb.xc.v[r0 + k][0], c, conv_silu(w0, w1, w2, w3, bias, raw[k], raw[k + 1], raw[k + 2], raw[k + 3]));
}

// One stripe record: NL state words per lane (and, for an aggregate, one
// summed-delta word per lane), epoch-tagged. Word j of lane l sits at j*64 + l,
// so each store instruction of a wave writes 512 contiguous bytes.
template <int NL>
__device__ __forceinline__ void publish_state(uint64_t *rec, int l, const float (&S)[NL], uint32_t epoch) {
#pragma unroll
    for (int j = 0; j < NL; ++j) st_tagged(rec + j * 64 + l, S[j], epoch);
}

// What the scan computes besides the exponential-Euler recurrence on an
// activated step size; each is a separate instance, so that the kernels for
// the plain rule carry none of that code.
//  kSoftplus: delta holds the step size before its activation (softplus(delta
//    + dt_bias), applied to each tile as it lands).
//  kTrap: the exponential-trapezoidal rule ("Notas sobre Mamba", section
//    "Recorrência trapezoidal"): h_t = a_t h_{t-1} + mu_t a_t v_{t-1} +
//    lam_t delta_t v_t, with a_t = exp(delta_t A), v_t = B_t x_t and mu_t =
//    (1 - lam_t) delta_t. The kernel runs the same recurrence on
//    k_t = h_t + mu_{t+1} v_t, which is
//      k_t = a_t k_{t-1} + (lam_t delta_t + mu_{t+1}) v_t,
//    the exponential-Euler form with the input weight lam_t delta_t +
//    mu_{t+1} in place of delta_t; so a state update costs what it costs
//    there, and stripes compose as before. Then
//      y_t = C_t . k_t - mu_{t+1} x_t (C_t . B_t) + D x_t   (before the gate),
//    k starts from h_in + mu_0 v_{-1}, and mu_L = 0 (no token after the call)
//    makes the final k the final h.
//  kConv: as kSoftplus, and x holds the raw input of the x branch ahead of
//    the scan ("Notas sobre Mamba", section "O bloco Mamba"): the scan uses
//    SiLU of its causal width-4 convolution per channel (conv_tile), rounded
//    to the activation dtype, in both passes and in the D skip.
enum ScanMode { kEuler = 0, kSoftplus = 1, kTrap = 2, kConv = 3 };

template <int N, int DT, bool GATE, bool SKIP, int MODE>
__global__ __launch_bounds__(64 * kWaves, (stripe_min_blocks<N, DT, MODE == kTrap, MODE == kConv>())) void scan_stripe_kernel(
    StripeArgs a) {
    using G = Geo<N, DT>;
    using T = typename G::T;
    constexpr int NL = G::NL, NGR = G::NGR, CPW = G::CPW, TCH = G::TCH, TPV = G::TPV, BREGS = G::BREGS;
    constexpr int TT = G::TT, GROUP = G::GROUP;
    constexpr bool CONV = MODE == kConv, SP = MODE == kSoftplus || CONV, TRAP = MODE == kTrap;
    using TBT = TileBuf<N, DT, TRAP, CONV>;

    __shared__ Shared<N, DT, TRAP, CONV> sh;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, kept scalar
    const int l = threadIdx.x & 63;
    const int row = l >> 4, k16 = l & 15;
    const int g = row % NGR;                            // state group of this lane
    const int nstate0 = g * NL;
    const int cl = w * CPW + (row / NGR) * 16 + k16;    // channel within the tile column
    const uint32_t sel_ch = half_sel(cl);                 // lds_act selectors: this lane's channel
    const uint32_t sel_st = half_sel(k16 % NL);           // and its Bt/Ct element (nstate0 is even)
    const int64_t D = a.D, L = a.L;
    const int64_t n_whole = a.n_whole, n_split = a.cols_per_list - a.n_whole;

    const int list = blockIdx.x % kLists;
    uint32_t *const counter = a.hdr + kHdrCounters + list;
    uint32_t *const err = a.hdr + kHdrError;
    // This call's tag: one past that of the last finished call (skipping 0,
    // the value of a cleared workspace). Every workgroup reads it before it
    // counts itself finished, and only the last to finish advances it.
    if (threadIdx.x == 0) {
        const uint32_t e = ld_flag(a.hdr + kHdrEpoch) + 1u;
        sh.tag = e == 0u ? 1u : e;
    }
    lds_barrier();
    const uint32_t epoch = (uint32_t)__builtin_amdgcn_readfirstlane(sh.tag);
    const uint32_t units = (uint32_t)(n_whole + n_split * a.S);
    // every workgroup takes units until it is handed one past the end, so a
    // call makes exactly (units + workgroups of the list) takes; the last one
    // puts the counter back to zero for the next call
    const uint32_t last_take = units + gridDim.x / kLists - 1;

    while (true) {
        if (w == 0 && l == 0) {
            const uint32_t u = take_unit(counter);
            if (u == last_take) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sh.unit = (int)u;
        }
        lds_barrier();
        const uint32_t u = (uint32_t)__builtin_amdgcn_readfirstlane(sh.unit);
        if (u >= units) break;
        // The list's first n_whole columns are whole-sequence units; each of
        // the others is cut into S stripes (which fill the last round).
        const bool whole = u < n_whole;
        const int64_t S = whole ? 1 : a.S;
        const int64_t SL = whole ? L : a.SL;
        const int64_t cs = whole ? 0 : (u - n_whole) / S;       // split column index
        const int64_t j = whole ? 0 : (u - n_whole) % S;        // stripe
        const int64_t col = list + (int64_t)kLists * (whole ? u : n_whole + cs);  // tile column
        if (col >= a.ncol) {
            lds_barrier();  // sh.unit is rewritten at the top
            continue;
        }
        const int64_t b = col / a.ntpb;
        const int64_t ch0 = (col % a.ntpb) * TCH;
        const int64_t d = ch0 + cl;
        const bool valid = d < D;
        // this lane's byte offset within an activation slot of a tile (see load_tile)
        int64_t lane_ch = ch0 + (l % G::PPR) * G::VEC;
        lane_ch = lane_ch + G::VEC <= D ? lane_ch : D - G::VEC;
        const uint32_t act_off = (uint32_t)((l / G::PPR) * D + (lane_ch - ch0)) * G::ESZ;
        // bias of the raw step size for the channels of this thread's delta pieces
        float dtb[G::VEC];
#pragma unroll
        for (int k = 0; k < G::VEC; ++k) dtb[k] = (SP && a.dt_bias) ? a.dt_bias[lane_ch + k] : 0.0f;
        const int64_t dc = valid ? d : D - 1;
        if constexpr (CONV) {
            // taps and bias of the tile column's channels (past D: the last
            // channel's; those results are never stored)
            for (int q = threadIdx.x; q < 5 * TCH; q += 64 * kWaves) {
                const int jj = q / TCH, c = q % TCH;
                const int64_t ch = ch0 + c < D ? ch0 + c : D - 1;
                sh.cw.v[jj][c] = jj < 4 ? a.conv_w[ch * 4 + jj] : (a.conv_b ? a.conv_b[ch] : 0.0f);
            }
        }
        const int64_t t0 = j * SL;
        const int64_t t1 = t0 + SL < L ? t0 + SL : L;
        const int ntiles = (int)((t1 - t0 + TT - 1) / TT);
        const bool has_next = j + 1 < S;  // a later stripe needs this one's end state

        float A2[NL];
#pragma unroll
        for (int q = 0; q < NL; ++q) A2[q] = a.A[dc * N + nstate0 + q] * kLog2e;
        const float dskip = SKIP ? a.Dskip[dc] : 0.0f;
        // records of stripe jj of this column, for this wave
        const int64_t rec0 = ((int64_t)list * n_split + cs) * S;
        auto rec_of = [&](int64_t jj) { return (rec0 + jj) * kWaves + w; };
        const int64_t rec = rec_of(j);

        // Walk the stripe's tiles: PASS 1 folds (dA, dBx) from a zero start,
        // PASS 2 runs the recurrence from h and writes y.
        float h[NL];
        // The finished y of tile i (pass 2): every wave writes a share of it back
        // as whole lines from the tile's delta area.
        auto store_y = [&](const TBT &tb, int i) {
            using VT = uint32_t __attribute__((ext_vector_type(4)));
            const int64_t tt0 = t0 + (int64_t)i * TT;
            const int64_t rows = t1 - tt0;  // tokens of the tile inside the stripe
            T *yptr = (T *)a.y;
#pragma unroll
            for (int p = threadIdx.x; p < G::ACT_PIECES; p += 64 * kWaves) {
                const int r = p / G::PPR, c = (p % G::PPR) * G::VEC;
                if (r < rows && ch0 + c < D) {
                    const VT v = *(const VT *)__builtin_assume_aligned(&tb.dl[r][c], 16);
                    *(VT *)(yptr + (b * L + tt0 + r) * D + ch0 + c) = v;
                }
            }
        };
        // First tile of a pass, loaded ahead (before the look-back, for pass 2).
        auto prefetch = [&](auto pass_c) {
            constexpr int PASS = decltype(pass_c)::value;
            if (w > 0) load_tile<N, DT, GATE, PASS, TRAP>(sh.buf[0], a, b, ch0, t0, w, l, act_off);
        };
        // TRAP, pass 2: C_t . B_t of every token of a landed tile, into sh.cb.
        // PARTS consecutive threads share a token, SPP states each, and sum
        // their parts with lane exchanges.
        auto tile_cb = [&](const TBT &tb) {
            constexpr int PARTS = 64 * kWaves / TT;
            if constexpr (N % PARTS == 0) {
                constexpr int SPP = N / PARTS;
                const int t = threadIdx.x / PARTS, n0 = (threadIdx.x % PARTS) * SPP;
                const T *Br = &tb.B[t * N], *Cr = &tb.C[t * N];
                float cbv = 0.0f;
#pragma unroll
                for (int n = n0; n < n0 + SPP; ++n)
                    cbv = __builtin_fmaf(lds_act(Cr, n, half_sel(n)), lds_act(Br, n, half_sel(n)), cbv);
#pragma unroll
                for (int m = 1; m < PARTS; m <<= 1) cbv += __shfl_xor(cbv, m);
                if (n0 == 0) sh.cb[t] = cbv;
            } else if (threadIdx.x < TT) {
                const T *Br = &tb.B[threadIdx.x * N], *Cr = &tb.C[threadIdx.x * N];
                float cbv = 0.0f;
#pragma unroll
                for (int n = 0; n < N; ++n)
                    cbv = __builtin_fmaf(lds_act(Cr, n, half_sel(n)), lds_act(Br, n, half_sel(n)), cbv);
                sh.cb[threadIdx.x] = cbv;
            }
        };
        // Early mode, pass 2: the carried-in state, and whether this lane may
        // vote to stop (see the file comment).
        float hin[NL];
        bool lane_ok = false;
        // OPT (kSum, kMin, kStop): pass 2 also sums delta into dsum, tracks its
        // minimum in dmin, or stops at the first tile end where every lane of
        // the workgroup votes to (pass 1 always sums).
        auto walk = [&](auto pass_c, auto opt_c, float (&st)[NL], float &dsum, float &dmin) {
            constexpr int PASS = decltype(pass_c)::value;
            constexpr int OPT = decltype(opt_c)::value;
            // bfloat16 groups of 8 tokens with two broadcast registers and two
            // finished tokens per lane take the high-half loads
            constexpr bool kHiLoads = DT == 1 && GROUP == 8 && BREGS == 2 && G::OWN == 2;
            float xv[GROUP], dv[GROUP], Bq[BREGS], Cq[BREGS], xo[G::OWN], zo[G::OWN];
            // TRAP: lam of the group's tokens, delta and lam of the token after
            // the group, and of the token after each finished token
            float lv[GROUP], dn = 0.0f, ln = 0.0f, dno[G::OWN], lno[G::OWN], cbo[G::OWN];
#pragma unroll
            for (int t = 0; t < GROUP; ++t) xv[t] = dv[t] = lv[t] = 0.0f;
#pragma unroll
            for (int q = 0; q < G::OWN; ++q) dno[q] = lno[q] = 0.0f;
#pragma unroll
            for (int q = 0; q < BREGS; ++q) Bq[q] = Cq[q] = 0.0f;
#pragma unroll
            for (int q = 0; q < G::OWN; ++q) xo[q] = zo[q] = 0.0f;
            if constexpr (CONV) {
                // the raw x of the three tokens before the stripe, as the last
                // rows of the buffer the first tile's convolution takes as the
                // previous one (before token 0: conv_state, or zeros); the
                // prefetch fills the other buffer
                for (int q = threadIdx.x; q < 3 * TCH; q += 64 * kWaves) {
                    const int jj = q / TCH, c = q % TCH;
                    const int64_t ch = ch0 + c < D ? ch0 + c : D - 1;
                    const int64_t t = t0 - 3 + jj;
                    T v = T(0);
                    if (t >= 0) v = ((const T *)a.x)[(b * L + t) * D + ch];
                    else if (a.conv_state) v = ((const T *)a.conv_state)[(b * D + ch) * 3 + (t + 3)];
                    sh.buf[1].x[TT - 3 + jj][c] = v;
                }
            }
            if (w > 0) vm_wait();  // the first tile (prefetch) has landed
            lds_barrier();
            int last = ntiles - 1;  // the last tile walked
            for (int i = 0; i < ntiles; ++i) {
                TBT &tb = sh.buf[i & 1];
                const int64_t tt0 = t0 + (int64_t)i * TT;
                if constexpr (PASS == 2) {
                    // y of the previous tile goes out now, so that the stores
                    // complete behind this tile's scan; its buffer is loaded next
                    if (i > 0) store_y(sh.buf[(i - 1) & 1], i - 1);
                }
                if constexpr (SP) activate_delta<N, DT>(tb, dtb);  // this tile has landed for every wave
                if constexpr (CONV) conv_tile<N, DT>(tb, sh.buf[(i + 1) & 1], sh.cw.v);
                if constexpr (TRAP && PASS == 2) tile_cb(tb);
                if (SP || (PASS == 2 && (TRAP || i > 0))) lds_barrier();
                if (w > 0 && i + 1 < ntiles)
                    load_tile<N, DT, GATE, PASS, TRAP>(sh.buf[(i + 1) & 1], a, b, ch0, tt0 + TT, w, l, act_off);
                // tokens past the end were loaded from the last token; give
                // them delta = 0 so that they leave the state unchanged
                if constexpr (TRAP) {
                    // The call's last tile, with the token after it: rows from
                    // L - tt0 through TT. (Stripes are whole tiles, so any other
                    // tile is full and its next token is real.) mu is then 0
                    // from token L on.
                    if (tt0 + TT >= L) {
                        const int first = (int)(L - tt0);
                        for (int q = threadIdx.x; q < (TT + 1 - first) * TCH; q += 64 * kWaves)
                            tb.dl[first + q / TCH][q % TCH] = T(0.0f);
                        lds_barrier();
                    }
                } else {
                    const int64_t tail = t1 - tt0;  // tokens of this tile inside the stripe
                    if (tail < TT) {
                        for (int q = threadIdx.x; q < (TT - (int)tail) * TCH; q += 64 * kWaves)
                            tb.dl[tail + q / TCH][q % TCH] = T(0.0f);
                        lds_barrier();
                    }
                }
                // per-lane LDS byte addresses in this tile: the lane's channel
                // column, its Bt/Ct element and its first owned token's row
                using TB = TBT;
                constexpr int ROWB = TCH * G::ESZ, BCB = N * G::ESZ;
                constexpr int OFF_DL = offsetof(TB, dl), OFF_Z = offsetof(TB, z), OFF_LAM = offsetof(TB, lam);
                constexpr int OFF_B = offsetof(TB, B), OFF_C = offsetof(TB, C);
                constexpr int OFF_X = CONV ? offsetof(TB, xc) : offsetof(TB, x);  // the x the scan reads
                const uint32_t a_ch = lds_addr(&tb) + cl * G::ESZ;
                const uint32_t a_bc = lds_addr(&tb) + OFF_B + ((k16 / NL) * N + nstate0 + (k16 % NL)) * G::ESZ;
                const uint32_t a_own = a_ch + g * ROWB;
                const uint32_t a_cb = lds_addr(&sh.cb[0]) + g * 4;  // TRAP: C . B of the lane's first finished token
                // row r of the x the scan reads (generic loads)
                [[maybe_unused]] auto xrow = [&](int r) -> const T * {
                    if constexpr (CONV) return &tb.xc.v[r][0];
                    else return &tb.x[r][0];
                };
                static_for<0, TT / GROUP>([&](auto gc) {
                    constexpr int tg = decltype(gc)::value * GROUP;
                    // Keep the groups in order: the previous group's state
                    // and summed delta pass through here before this group's
                    // loads are issued, so the compiler cannot hoist the
                    // loads of later groups above earlier arithmetic (which
                    // would keep every group's values live at once). The
                    // activation code of SP made the compiler do that.
                    if constexpr (SP) order_point<NL>(st, dsum);
                    if constexpr (kHiLoads) {
                        // bfloat16: loads into the high halves of the registers
                        // that held the previous group's values, one wait per group
                        constexpr int OX = OFF_X + tg * ROWB, OD = OFF_DL + tg * ROWB, OL = OFF_LAM + tg * ROWB;
                        constexpr int SB = TPV * BCB, OB = tg * BCB, OC = OFF_C - OFF_B + tg * BCB;
                        constexpr int SO = NGR * ROWB, OXO = OFF_X + tg * ROWB, OZO = OFF_Z + tg * ROWB;
                        if constexpr (TRAP && PASS == 2)
                            lds_bf16_t2<ROWB, OX, OD, OL, SB, OB, OC, SO, OXO, OZO, OFF_DL + (tg + 1) * ROWB,
                                        OFF_LAM + (tg + 1) * ROWB, NGR * 4, tg * 4>(
                                xv, dv, lv, dn, ln, Bq, Cq, xo, zo, dno, lno, cbo, a_ch, a_bc, a_own, a_cb);
                        else if constexpr (TRAP)
                            lds_bf16_t1<ROWB, OX, OD, OL, SB, OB>(xv, dv, lv, dn, ln, Bq, a_ch, a_bc);
                        else if constexpr (PASS == 2)
                            lds_bf16_p2<ROWB, OX, OD, SB, OB, OC, SO, OXO, OZO>(xv, dv, Bq, Cq, xo, zo, a_ch, a_bc,
                                                                                a_own);
                        else
                            lds_bf16_p1<ROWB, OX, OD, SB, OB>(xv, dv, Bq, a_ch, a_bc);
                    } else {
#pragma unroll
                        for (int t = 0; t < GROUP; ++t) {
                            xv[t] = lds_act(xrow(tg + t), cl, sel_ch);
                            dv[t] = lds_act(&tb.dl[tg + t][0], cl, sel_ch);
                            if constexpr (TRAP) lv[t] = lds_act(&tb.lam[tg + t][0], cl, sel_ch);
                        }
                        if constexpr (TRAP) {
                            dn = lds_act(&tb.dl[tg + GROUP][0], cl, sel_ch);
                            ln = lds_act(&tb.lam[tg + GROUP][0], cl, sel_ch);
                        }
#pragma unroll
                        for (int q = 0; q < BREGS; ++q) {
                            const int tw = tg + q * TPV + k16 / NL;
                            Bq[q] = lds_act(&tb.B[tw * N], nstate0 + (k16 % NL), sel_st);
                            if constexpr (PASS == 2) Cq[q] = lds_act(&tb.C[tw * N], nstate0 + (k16 % NL), sel_st);
                        }
                        if constexpr (PASS == 2) {
                            // x and z of the tokens this lane finishes (token NGR*q + g of the group)
#pragma unroll
                            for (int q = 0; q < G::OWN; ++q) {
                                const int tw = tg + NGR * q + g;
                                xo[q] = (SKIP || TRAP) ? lds_act(xrow(tw), cl, sel_ch) : 0.0f;
                                zo[q] = GATE ? lds_act(&tb.z[tw][0], cl, sel_ch) : 0.0f;
                                if constexpr (TRAP) {
                                    dno[q] = lds_act(&tb.dl[tw + 1][0], cl, sel_ch);
                                    lno[q] = lds_act(&tb.lam[tw + 1][0], cl, sel_ch);
                                    cbo[q] = sh.cb[tw];
                                }
                            }
                        }
                    }
                    // input weight times x of token t of the group: delta x, or
                    // for TRAP (lam delta + mu of the next token) x
                    auto in_x = [&](auto tc) {
                        constexpr int t = decltype(tc)::value;
                        if constexpr (TRAP) {
                            float dnx, lnx;
                            if constexpr (t + 1 < GROUP) {
                                dnx = dv[t + 1];
                                lnx = lv[t + 1];
                            } else {
                                dnx = dn;
                                lnx = ln;
                            }
                            const float mu = __builtin_fmaf(-lnx, dnx, dnx);
                            return __builtin_fmaf(lv[t], dv[t], mu) * xv[t];
                        } else {
                            return dv[t] * xv[t];
                        }
                    };
                    if constexpr (PASS == 1) {
                        static_for<0, GROUP>([&](auto tc) {
                            constexpr int t = decltype(tc)::value;
                            const float dx = in_x(tc);
                            dsum += dv[t];
                            static_for<0, NL>([&](auto jc) {
                                constexpr int q = decltype(jc)::value;
                                const float dA = fast_exp2(dv[t] * A2[q]);
                                st[q] = __builtin_fmaf(dA, st[q], row_bcast<(t % TPV) * NL + q>(Bq[t / TPV]) * dx);
                            });
                        });
                    } else {
                        float yp[GROUP];
                        static_for<0, GROUP>([&](auto tc) {
                            constexpr int t = decltype(tc)::value;
                            const float dx = in_x(tc);
                            if constexpr ((OPT & kSum) != 0) dsum += dv[t];
                            if constexpr ((OPT & kMin) != 0) dmin = __builtin_fminf(dmin, dv[t]);
                            static_for<0, NL>([&](auto jc) {
                                constexpr int q = decltype(jc)::value;
                                const float dA = fast_exp2(dv[t] * A2[q]);
                                st[q] = __builtin_fmaf(dA, st[q], row_bcast<(t % TPV) * NL + q>(Bq[t / TPV]) * dx);
                            });
                            if constexpr (kHiLoads)
                                dot_row_lds<(t % TPV) * NL>(yp[t], Cq[t / TPV], st);
                            else
                                dot_row<NL, (t % TPV) * NL>(yp[t], Cq[t / TPV], st);
                        });
                        // Sum the partial readouts over a channel's rows; afterwards
                        // row r holds the finished token NGR*q + (r % NGR) of group q.
                        float yo[G::OWN];
                        if constexpr (NGR == 4) {
#pragma unroll
                            for (int q = 0; q < GROUP / 4; ++q) {
                                float a0 = yp[4 * q + 0], a2 = yp[4 * q + 2], a1 = yp[4 * q + 1], a3 = yp[4 * q + 3];
                                // rows 0,1: token 0 | rows 2,3: token 2, and tokens 1 | 3
                                swap_halves2(a0, a2, a1, a3);
                                float s02 = a0 + a2, s13 = a1 + a3;
                                swap_odd_even_rows(s02, s13);
                                yo[q] = s02 + s13;
                            }
                        } else if constexpr (NGR == 2) {
#pragma unroll
                            for (int q = 0; q < GROUP / 2; ++q) {
                                float a0 = yp[2 * q + 0], a1 = yp[2 * q + 1];
                                swap_odd_even_rows(a0, a1);
                                yo[q] = a0 + a1;
                            }
                        } else {
#pragma unroll
                            for (int q = 0; q < GROUP; ++q) yo[q] = yp[q];
                        }
                        // Finish the owned tokens (D skip, silu gate) into the tile.
#pragma unroll
                        for (int q = 0; q < G::OWN; ++q) {
                            const int tw = tg + NGR * q + g;
                            float yv = yo[q];
                            if constexpr (TRAP) {
                                // h = k - mu_{t+1} v_t: subtract mu_{t+1} x_t (C_t . B_t)
                                const float mu = __builtin_fmaf(-lno[q], dno[q], dno[q]);
                                yv = __builtin_fmaf(-mu * xo[q], cbo[q], yv);
                            }
                            if (SKIP) yv = __builtin_fmaf(dskip, xo[q], yv);
                            if (GATE) yv *= silu(zo[q]);
                            st_act(&tb.dl[tw][0], cl, yv);
                        }
                    }
                });
                if constexpr ((OPT & kStop) != 0) {
                    // this lane's vote: its carried-in state, decayed to the
                    // end of this tile, below the rounding unit of its states
                    constexpr float kRel = DT == 0 ? 0x1p-24f : 0x1p-16f;
                    float em = 0.0f, hm = 0.0f;
#pragma unroll
                    for (int q = 0; q < NL; ++q) {
                        em = __builtin_fmaxf(em, __builtin_fabsf(hin[q]) * fast_exp2(A2[q] * dsum));
                        hm = __builtin_fmaxf(hm, __builtin_fabsf(st[q]));
                    }
                    const bool ok = lane_ok && em <= kRel * hm;
                    const uint64_t against = __builtin_amdgcn_ballot_w64(!ok);  // every lane, before the branch
                    if (l == 0) sh.stop[i & 1][w] = against == 0 ? 1 : 0;
                }
                vm_wait();  // the next tile has landed (and this wave's earlier y stores are out)
                lds_barrier();
                if constexpr ((OPT & kStop) != 0) {
                    int all = 1;
#pragma unroll
                    for (int v = 0; v < kWaves; ++v) all &= sh.stop[i & 1][v];
                    if (__builtin_amdgcn_readfirstlane(all)) {
                        last = i;
                        break;
                    }
                }
            }
            if constexpr (PASS == 2) store_y(sh.buf[last & 1], last);
        };

        using P1 = std::integral_constant<int, 1>;
        using P2 = std::integral_constant<int, 2>;
        float agg[NL], dagg = 0.0f, dmin = __builtin_inff(), unused = 0.0f;
#pragma unroll
        for (int q = 0; q < NL; ++q) agg[q] = 0.0f;
        // early mode: stripe 0 walks once from its known state; every later
        // stripe runs the scan from zero first (fold), then the short pass 2
        const bool early = a.early != 0 && S > 1;
        const bool fold = early && j > 0;
        if (fold) {
            prefetch(P2{});
            walk(P2{}, std::integral_constant<int, kSum | (SP ? 0 : kMin)>{}, agg, dagg, dmin);
            if (has_next) {
                uint64_t *ar = a.agg + rec * (64 * (NL + 1));
                publish_state<NL>(ar, l, agg, epoch);
                st_tagged(ar + 64 * NL + l, dagg, epoch);
            }
            lds_barrier();  // every wave has read its share of the last y tile before the prefetch lands
        } else if (!early && has_next) {
            prefetch(P1{});
            walk(P1{}, std::integral_constant<int, 0>{}, agg, dagg, unused);
            if (j > 0) {  // (stripe 0: its end state goes out directly)
                uint64_t *ar = a.agg + rec * (64 * (NL + 1));
                publish_state<NL>(ar, l, agg, epoch);
                st_tagged(ar + 64 * NL + l, dagg, epoch);
            }
        }
        prefetch(P2{});  // lands during the look-back

        // Carried-in state of this stripe.
        if (j == 0) {
            const float *si = a.state_in ? a.state_in + (b * D + dc) * N + nstate0 : nullptr;
#pragma unroll
            for (int q = 0; q < NL; ++q) h[q] = si ? si[q] : 0.0f;
            if constexpr (TRAP) {
                // k starts from h_in + mu_0 v_{-1}, v_{-1} = B_prev x_prev
                if (a.x_prev) {
                    const int64_t r0 = b * L * D + dc;  // token 0
                    const float d0 = ld_act((const T *)a.delta, r0), l0 = ld_act((const T *)a.lam, r0);
                    const float px = __builtin_fmaf(-l0, d0, d0) * ld_act((const T *)a.x_prev, b * D + dc);
#pragma unroll
                    for (int q = 0; q < NL; ++q)
                        h[q] = __builtin_fmaf(px, ld_act((const T *)a.B_prev, b * N + nstate0 + q), h[q]);
                }
            }
        } else {
            // Look back over the earlier stripes of this column: the nearest
            // one whose end state is out, with the aggregates of all stripes
            // after it out. A wait that gives up (the spin limit, or another
            // wait of this call gave up first: then this one does not wait at
            // all) leaves a NaN state, so that every output depending on it
            // is NaN, and marks the header's error word with this call's tag.
            int64_t j0 = -1;
            long spin = 0;
            bool failed = (uint32_t)__builtin_amdgcn_readfirstlane(ld_flag(err)) == epoch;
            while (!failed) {
                const int64_t jj = j - 1 - l;  // stripe examined by this lane
                bool inc = false, ag = false;
                if (jj >= 0) {
                    // the first word of a record stands for all of it; the
                    // replay below still checks every word it reads
                    const int64_t r2 = rec_of(jj);
                    inc = (uint32_t)(ld_tagged(a.incl + r2 * (64 * NL)) >> 32) == epoch;
                    ag = inc || (uint32_t)(ld_tagged(a.agg + r2 * (64 * (NL + 1))) >> 32) == epoch;
                }
                const uint64_t m_inc = __builtin_amdgcn_ballot_w64(inc);
                const uint64_t m_agg = __builtin_amdgcn_ballot_w64(ag);
                if (m_inc) {
                    const int i0 = __builtin_ctzll(m_inc);
                    const uint64_t below = i0 == 0 ? 0 : (~0ull >> (64 - i0));
                    if ((m_agg & below) == below) {
                        j0 = j - 1 - i0;
                        break;
                    }
                }
                if (++spin > kSpinLimit ||
                    (spin % 64 == 0 && (uint32_t)__builtin_amdgcn_readfirstlane(ld_flag(err)) == epoch)) {
                    failed = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(4);
            }
            if (!failed) {
                // Replay forward from that state with the arithmetic each
                // stripe uses for its own end state, kReplay records per
                // round trip. A word still not of this call after its own
                // bounded wait fails the replay.
                bool bad = false;
                auto value = [&](uint64_t v) {
                    bad |= (uint32_t)(v >> 32) != epoch;
                    return __uint_as_float((uint32_t)v);
                };
                const uint64_t *src = a.incl + rec_of(j0) * (64 * NL) + l;
#pragma unroll
                for (int q = 0; q < NL; ++q) h[q] = value(ld_valid(src + q * 64, epoch));
                for (int64_t jj = j0 + 1; jj < j; jj += kReplay) {
                    uint64_t sv[kReplay][NL], dv2[kReplay];
#pragma unroll
                    for (int r = 0; r < kReplay; ++r) {
                        if (jj + r < j) {
                            const uint64_t *ar = a.agg + rec_of(jj + r) * (64 * (NL + 1));
#pragma unroll
                            for (int q = 0; q < NL; ++q) sv[r][q] = ld_tagged(ar + q * 64 + l);
                            dv2[r] = ld_tagged(ar + 64 * NL + l);
                        }
                    }
#pragma unroll
                    for (int r = 0; r < kReplay; ++r) {
                        if (jj + r < j) {
                            const uint64_t *ar = a.agg + rec_of(jj + r) * (64 * (NL + 1));
                            const float dd = value(recheck(dv2[r], ar + 64 * NL + l, epoch));
#pragma unroll
                            for (int q = 0; q < NL; ++q)
                                h[q] = __builtin_fmaf(fast_exp2(A2[q] * dd), h[q],
                                                      value(recheck(sv[r][q], ar + q * 64 + l, epoch)));
                        }
                    }
                }
                failed = __builtin_amdgcn_ballot_w64(bad) != 0;
            }
            if (failed) {
                if (l == 0) __hip_atomic_store(err, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                for (int q = 0; q < NL; ++q) h[q] = __builtin_nanf("");
            }
        }
        // this stripe's end state, from the pair (for the stripes after it,
        // and the final state of a folded last stripe)
        float e[NL];
#pragma unroll
        for (int q = 0; q < NL; ++q) e[q] = __builtin_fmaf(fast_exp2(A2[q] * dagg), h[q], agg[q]);
        if (has_next && !(early && j == 0)) publish_state<NL>(a.incl + rec * (64 * NL), l, e, epoch);
        const bool final_state = !has_next && a.state_out && valid;
        float *const so = final_state ? a.state_out + (b * D + d) * N + nstate0 : nullptr;
        if (fold && final_state) {
#pragma unroll
            for (int q = 0; q < NL; ++q) so[q] = e[q];
        }

        if (fold) {
            bool ok = SP || dmin >= 0.0f;
#pragma unroll
            for (int q = 0; q < NL; ++q) {
                hin[q] = h[q];
                ok = ok && __builtin_isfinite(h[q]) && A2[q] <= 0.0f;
            }
            lane_ok = ok;
            float dsum = 0.0f;
            walk(P2{}, std::integral_constant<int, kSum | kStop>{}, h, dsum, unused);
        } else {
            walk(P2{}, std::integral_constant<int, 0>{}, h, unused, unused);
            if (early && has_next) publish_state<NL>(a.incl + rec * (64 * NL), l, h, epoch);  // stripe 0
        }
        if (!fold && final_state) {
#pragma unroll
            for (int q = 0; q < NL; ++q) so[q] = h[q];
        }
    }
    // The last workgroup to finish publishes this call's tag as the last
    // finished call's and clears the count for the next call.
    if (threadIdx.x == 0) {
        uint32_t *const done = a.hdr + kHdrDone;
        if (__hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
            __hip_atomic_store(a.hdr + kHdrEpoch, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int N, int DT, bool GATE, bool SKIP, int MODE>
hipError_t launch_stripe_typed(const StripeArgs &a, hipStream_t s) {
    auto kern = scan_stripe_kernel<N, DT, GATE, SKIP, MODE>;
    constexpr int kMaxDevices = 64;
    // CU count and resident workgroups per CU, queried once per device:
    // (cus << 32 | per_cu), 0 = not queried yet
    static std::atomic<uint64_t> cache[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    uint64_t packed = dev < kMaxDevices ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (packed == 0) {
        int cus = 0, per_cu = 0;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * kWaves, 0)) != hipSuccess) return e;
        if (per_cu < 1 || cus < 1) return hipErrorInvalidConfiguration;
        packed = (uint64_t)cus << 32 | (uint32_t)per_cu;
        if (dev < kMaxDevices) cache[dev].store(packed, std::memory_order_relaxed);
    }
    const int cus = (int)(packed >> 32), per_cu = (int)(uint32_t)packed;
    int64_t per_list = (int64_t)cus * per_cu / kLists;
    const int64_t units = a.n_whole + (a.cols_per_list - a.n_whole) * a.S;
    if (per_list > units) per_list = units;
    if (per_list < 1) per_list = 1;
    StripeArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel((const void *)kern, dim3((unsigned)(per_list * kLists)), dim3(64 * kWaves), params, 0, s);
}

template <int N, int DT, int MODE>
hipError_t launch_stripe_flags(const StripeArgs &a, hipStream_t s) {
    const bool gate = a.z != nullptr, skip = a.Dskip != nullptr;
    if (gate && skip) return launch_stripe_typed<N, DT, true, true, MODE>(a, s);
    if (gate) return launch_stripe_typed<N, DT, true, false, MODE>(a, s);
    if (skip) return launch_stripe_typed<N, DT, false, true, MODE>(a, s);
    return launch_stripe_typed<N, DT, false, false, MODE>(a, s);
}

template <int N, int MODE>
hipError_t launch_stripe_dtype(const StripeArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch_stripe_flags<N, 0, MODE>(a, s) : launch_stripe_flags<N, 1, MODE>(a, s);
}

template <int MODE>
hipError_t launch_stripe_n(const StripeArgs &a, int N, int dtype, hipStream_t s) {
    switch (N) {
        case 1: return launch_stripe_dtype<1, MODE>(a, dtype, s);
        case 2: return launch_stripe_dtype<2, MODE>(a, dtype, s);
        case 4: return launch_stripe_dtype<4, MODE>(a, dtype, s);
        case 8: return launch_stripe_dtype<8, MODE>(a, dtype, s);
        case 16: return launch_stripe_dtype<16, MODE>(a, dtype, s);
        default: return hipErrorInvalidValue;
    }
}

template <int N, int DT>
void stripe_geometry(int64_t batch, int64_t L, int64_t D, StripePlan *p) {
    using G = Geo<N, DT>;
    p->nl = G::NL;
    p->tch = G::TCH;
    p->tt = G::TT;
    p->vec = G::VEC;
    p->ntpb = (D + G::TCH - 1) / G::TCH;
    p->ncol = batch * p->ntpb;
    p->cols_per_list = (p->ncol + kLists - 1) / kLists;
    // Columns that fill whole rounds of the planned workgroup slots run as
    // whole-sequence units; the rest are cut into S stripes each, so that
    // the last round is full too.
    const int64_t C = p->cols_per_list;
    const int64_t tiles = (L + G::TT - 1) / G::TT;
    const int64_t rem = C >= kSlotsPerList ? C % kSlotsPerList : C;
    int64_t S = rem > 0 ? kSlotsPerList / rem : 1;
    if (S > 64) S = 64;  // the look-back examines at most 64 earlier stripes at once
    if (S > tiles) S = tiles;
    if (S < 1) S = 1;
    const int64_t tiles_per_stripe = (tiles + S - 1) / S;
    S = tiles > 0 ? (tiles + tiles_per_stripe - 1) / tiles_per_stripe : 1;
    p->SL = tiles_per_stripe * G::TT;
    p->S = S;
    p->early = S > 1 && p->SL >= kEarlyMinTokens;
    p->n_whole = S > 1 ? C - rem : C;
}

}  // namespace

}  // namespace ssm
