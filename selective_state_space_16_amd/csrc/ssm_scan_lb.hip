// Single-pass selective scan (S6) forward for gfx950: persistent workgroups,
// register-resident chunk scans, and a decoupled look-back between chunks.
//
// The recurrence h <- dA*h + dBx is an associative composition of affine maps
// ("Notas sobre Mamba", section "A varredura paralela ciente do hardware":
// the scan over (A-bar_t, B-bar_t x_t) pairs). Applying a run of tokens to a
// state equals one pair (P, S): P = prod dA = exp(A * sum delta) and S = the
// run's end state from a zero start. The kernel uses this at two levels.
//
// Work items. An item is one chunk of 64 tokens of one block of CPW channels
// (CPW = 16 for N = 16). A workgroup of 4 waves scans an item: wave w owns
// tokens 16w..16w+15. Phase A computes dA = exp2(delta * A*log2(e)) once per
// (token, state) and keeps it in registers, with delta*x per token, while
// folding dA and dBx = B*(delta*x) into the wave's segment pair; the four
// segment pairs are combined through LDS. Phase C rescans the wave's tokens
// from its carried-in state using those registers (no second exponential;
// dBx is one multiply again) and reads out y.
//
// Between items of the same channel block the carried-in state comes from a
// decoupled look-back: every item publishes its inclusive end state as
// 64-bit words tagged with the call's epoch (readers validate each word, so a
// workgroup can fetch its predecessor's state before phase A and use it
// after). When the predecessor's state is not out yet the item publishes its
// own aggregate (sum delta, S) so that later items can skip over it, then
// scans back over the flags of earlier items to the nearest inclusive state
// and replays the chain forward from it with the same arithmetic every item
// uses for its own inclusive state; results therefore do not depend on
// timing. Every wait is bounded: on timeout the kernel records an error word
// in the workspace header and continues with a zero state.
//
// Memory. HBM rows are read in whole 128-byte lines: a workgroup loads tiles
// of 64 tokens x TCH channels (TCH = 64 bfloat16 or 32 float channels) of x,
// delta, z and the 64 tokens of Bt, Ct into LDS with global_load_lds (no
// registers involved), double-buffered so that the next tile streams in while
// the TCH/CPW items of the current tile are scanned. y is written into the
// tile's delta area (delta is dead after phase A) and stored as whole lines.
// Workgroups are persistent (as many as fit at once) and take tiles from one
// counter per XCD (the workgroup's blockIdx modulo 8): each XCD works through
// a contiguous range of channel blocks chunk-major, so that the look-back
// words a tile reads were written in the same L2. Tiles are handed out in that
// order, so a workgroup only ever waits for tiles already held by running
// workgroups: the launch is an ordinary one.
//
// Lanes. A wave is 4 rows of 16 lanes. A channel's N states are split over
// NGR = N/NL rows (NL = min(N, 4) states per lane); the 16 lanes of a row are
// 16 consecutive channels. Bt[t,:] and Ct[t,:] are the same for every
// channel, so a row keeps the values of its state group for 16/NL tokens in
// one register and broadcasts them with DPP row_newbcast. The readout sum over
// a channel's rows uses permlane16/32 swaps, which also scatter the finished
// tokens over the rows so that each lane finishes 16/NGR of the 16 tokens.
#include <atomic>
#include <type_traits>

#include "ssm_common.h"
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

namespace {

constexpr int kSegT = 16;        // tokens per wave segment
constexpr int kWaves = 4;        // waves (segments) per workgroup
constexpr int kChunk = kSegT * kWaves;
constexpr int kXcds = 8;         // XCDs of an MI355X
constexpr int kReplay = 2;       // aggregates loaded per round trip of a look-back replay

template <int N, int DT>
struct Geo {
    using T = typename Act<DT>::T;
    static constexpr int NL = N < 4 ? N : 4;       // states per lane
    static constexpr int NGR = N / NL;             // rows per channel
    static constexpr int CPW = (4 / NGR) * 16;     // channels per wave
    static constexpr int TPV = 16 / NL;            // tokens per broadcast register
    static constexpr int BREGS = kSegT / TPV;      // broadcast registers per segment
    static constexpr int OWN = kSegT / NGR;        // tokens each lane finishes
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int LINE_CH = 128 / ESZ;      // channels in a 128-byte line
    static constexpr int TCH = CPW > LINE_CH ? CPW : LINE_CH;  // tile channels
    static constexpr int SUBS = TCH / CPW;         // items per tile
    static constexpr int VEC = 16 / ESZ;           // elements per 16-byte piece
};

template <int N, int DT>
struct TileBuf {
    using G = Geo<N, DT>;
    using T = typename G::T;
    T x[kChunk][G::TCH];
    T dl[kChunk][G::TCH];  // delta; y is written here once delta is dead
    T z[kChunk][G::TCH];
    T B[kChunk][N];
    T C[kChunk][N];
    float A[G::TCH][N];    // state matrix rows of the tile's channels
    float Dsk[G::TCH];     // skip weights of the tile's channels
};

template <int N, int DT>
struct Shared {
    using G = Geo<N, DT>;
    TileBuf<N, DT> buf[2];
    float seg_s[kWaves][64][G::NL];  // segment end states (read only between the two item barriers)
    float seg_d[kWaves][64];         // segment summed deltas
    float carry[64][G::NL];          // the item's carried-in state
    int64_t tiles[1];                // the next tile handed to this workgroup
    uint64_t early[G::NL >= 2 ? G::NL / 2 : 1][64][2];  // predecessor's inclusive state, fetched early
};

// Workgroups per CU the kernel is built for: two when two copies of the LDS
// layout fit in the CU's 160 KB, else one (float tiles with N <= 4).
template <int N, int DT>
constexpr int min_blocks() { return 2 * sizeof(Shared<N, DT>) <= 160 * 1024 ? 2 : 1; }

// An item's segments 0..upto-1 folded from a zero start, in order: the end
// state from a zero start and the summed delta. Every wave that needs an
// item's aggregate (or a prefix of it) uses this, so that they agree bit for
// bit; the look-back replay folds with the same arithmetic.
template <int NL>
__device__ __forceinline__ void fold_segments(const float (&seg_s)[kWaves][64][NL], const float (&seg_d)[kWaves][64],
                                              int l, int upto, const float (&A2)[NL], float (&S)[NL], float &d) {
#pragma unroll
    for (int j = 0; j < NL; ++j) S[j] = 0.0f;
    d = 0.0f;
    for (int v = 0; v < upto; ++v) {
        const float dd = seg_d[v][l];
#pragma unroll
        for (int j = 0; j < NL; ++j) S[j] = __builtin_fmaf(fast_exp2(A2[j] * dd), S[j], seg_s[v][l][j]);
        d += dd;
    }
}

// An item's aggregate as epoch-tagged words: NL state words per lane, then one
// summed-delta word per lane.
template <int NL>
__device__ __forceinline__ void publish_aggregate(uint64_t *ag, int l, const float (&S)[NL], float d, uint32_t epoch) {
#pragma unroll
    for (int j = 0; j < NL; ++j) st_tagged(ag + l * NL + j, S[j], epoch);
    st_tagged(ag + 64 * NL + l, d, epoch);
}

// Issue the loads of one tile into LDS, spread over waves 1..3 (wave 0 keeps
// its memory counter free for the look-back). Pieces past the end of the
// sequence or of the channels are read from an in-bounds location instead;
// their LDS slots are never used for a stored result.
template <int N, int DT, bool GATE>
__device__ __forceinline__ void issue_tile_loads(TileBuf<N, DT> &tb, const LbArgs &a, int64_t b, int64_t ch0,
                                                 int64_t k, int w, int lane) {
    using G = Geo<N, DT>;
    using T = typename G::T;
    constexpr int PPR = G::TCH / G::VEC;            // pieces per tile row
    constexpr int ACT_PIECES = kChunk * PPR;        // pieces per activation tile (a multiple of 64)
    constexpr int BC_PIECES = kChunk * N / G::VEC;  // pieces per Bt/Ct tile (a multiple of 64)
    constexpr int NACT = GATE ? 3 : 2;              // x, delta (, z)
    const int64_t D = a.D, L = a.L;
    // activation tiles, in whole waves of 64 pieces
    for (int base = (w - 1) * 64; base < NACT * ACT_PIECES; base += 3 * 64) {
        const int arr = base / ACT_PIECES;
        const int pa = base - arr * ACT_PIECES + lane;
        const int r = pa / PPR, c = (pa % PPR) * G::VEC;
        int64_t t = k * kChunk + r;
        t = t < L ? t : L - 1;
        int64_t ch = ch0 + c;
        ch = ch + G::VEC <= D ? ch : D - G::VEC;
        const T *src = arr == 0 ? (const T *)a.x : arr == 1 ? (const T *)a.delta : (const T *)a.z;
        T *dst = arr == 0 ? &tb.x[0][0] : arr == 1 ? &tb.dl[0][0] : &tb.z[0][0];
        dma16(src + (b * L + t) * D + ch, lds_addr(dst + (int64_t)(base - arr * ACT_PIECES) * G::VEC));
    }
    // A rows of the tile's channels (contiguous), and the skip weights
    constexpr int A_PIECES = G::TCH * N / 4;        // 16-byte pieces of float
    for (int base = (w - 1) * 64; base < A_PIECES; base += 3 * 64) {
        int64_t ch = ch0 + (base + lane) * 4 / N;
        const int c = (base + lane) * 4 % N;
        ch = ch < D ? ch : D - 1;
        dma16(a.A + ch * N + c, lds_addr(&tb.A[0][0] + (int64_t)base * 4));
    }
    if (a.Dskip && w == 3) {
        // 4-byte pieces: lane i loads channel ch0 + i (TCH <= 64)
        int64_t ch = ch0 + lane;
        ch = ch < D ? ch : D - 1;
        if (lane < G::TCH) dma4(a.Dskip + ch, lds_addr(&tb.Dsk[0]));
    }
    // Bt and Ct tiles: the 64 tokens are contiguous rows of N values
    for (int base = (w - 1) * 64; base < 2 * BC_PIECES; base += 3 * 64) {
        const int arr = base / BC_PIECES;
        const int pq = base - arr * BC_PIECES + lane;
        const int r = pq * G::VEC / N, c = pq * G::VEC % N;
        int64_t t = k * kChunk + r;
        t = t < L ? t : L - 1;
        const T *src = arr == 0 ? (const T *)a.Bt : (const T *)a.Ct;
        T *dst = arr == 0 ? &tb.B[0][0] : &tb.C[0][0];
        dma16(src + (b * L + t) * N + c, lds_addr(dst + (int64_t)(base - arr * BC_PIECES) * G::VEC));
    }
}

// The next tile of one XCD's list. Tiles are handed out in list order, so
// every tile a workgroup waits for has already been handed to a running
// workgroup: no workgroup needs another one to be resident, and the launch
// needs no co-residency. Each workgroup takes tiles until it is handed one
// past the end, so a call makes exactly (tiles + workgroups of the list) takes;
// the last one puts the counter back to zero for the next call.
__device__ __forceinline__ uint32_t take_tile(uint32_t *ctr) {
    return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void after_take(uint32_t *ctr, uint32_t t, uint32_t last) {
    if (t == last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int N, int DT, bool GATE, bool SKIP>
__global__ __launch_bounds__(64 * kWaves, (min_blocks<N, DT>())) void scan_lb_kernel(LbArgs a) {
    using G = Geo<N, DT>;
    using T = typename G::T;
    constexpr int NL = G::NL, NGR = G::NGR, CPW = G::CPW, TPV = G::TPV, BREGS = G::BREGS;
    constexpr int TCH = G::TCH, SUBS = G::SUBS;

    __shared__ Shared<N, DT> sh;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, kept scalar
    const int l = threadIdx.x & 63;
    const int row = l >> 4, k16 = l & 15;
    const int g = row % NGR;           // state group of this lane
    const int nstate0 = g * NL;
    const int64_t D = a.D, L = a.L;

    // Tiles: (batch row, tile column) x chunk. XCD x owns tile columns
    // [x*tpx, (x+1)*tpx) and hands its tiles out chunk-major.
    const int64_t ntpb = (D + TCH - 1) / TCH;          // tile columns per batch row
    const int64_t ntcol = a.batch * ntpb;
    const int64_t tpx = (ntcol + kXcds - 1) / kXcds;
    const int64_t nlocal = tpx * a.K;
    const int xcd = blockIdx.x % kXcds;
    uint32_t *const counter = a.tiles + xcd;
    const uint32_t last_take = (uint32_t)(nlocal + gridDim.x / kXcds - 1);

    auto tile_of = [&](int64_t s, int64_t &tcol, int64_t &k) {
        k = s / tpx;
        tcol = xcd * tpx + s % tpx;
        return tcol < ntcol;
    };

    // Prologue: the first tile, loaded before the loop.
    if (w == 0 && l == 0) {
        const uint32_t t = take_tile(counter);
        after_take(counter, t, last_take);
        sh.tiles[0] = t;
    }
    lds_barrier();
    // tile indices of a list stay below 2^30 (checked when planning)
    int64_t s = __builtin_amdgcn_readfirstlane((int)sh.tiles[0]);
    {
        int64_t tcol, k;
        if (s < nlocal && tile_of(s, tcol, k) && w > 0)
            issue_tile_loads<N, DT, GATE>(sh.buf[0], a, tcol / ntpb, (tcol % ntpb) * TCH, k, w, l);
        vm_wait();
        lds_barrier();
    }

    int it = 0;        // tile counter (LDS buffer parity)
    while (s < nlocal) {
        TileBuf<N, DT> &tb = sh.buf[it & 1];
        int64_t tcol, k;
        const bool real = tile_of(s, tcol, k);
        // Ask for the next tile now (wave 1). Wave 1 hands the answer over
        // between the first item's two barriers; after the second, waves 1..3
        // start loading that tile into the other buffer (free since the end of
        // the previous tile) while this one is scanned. Tiles are thus taken
        // one ahead and processed in the order they are handed out.
        uint32_t nxt;  // assigned and read by wave 1, lane 0 only
        if (w == 1 && l == 0) nxt = take_tile(counter);
        int64_t s_next = nlocal;
        auto hand_over = [&]() {
            if (w == 1 && l == 0) {
                asm volatile("" : "+v"(nxt));  // read (and wait for) it here, in wave 1 only
                after_take(counter, nxt, last_take);
                sh.tiles[0] = nxt;
            }
        };
        auto start_next = [&]() {
            s_next = __builtin_amdgcn_readfirstlane((int)sh.tiles[0]);
            int64_t tcol2, k2;
            if (w > 0 && s_next < nlocal && tile_of(s_next, tcol2, k2))
                issue_tile_loads<N, DT, GATE>(sh.buf[(it + 1) & 1], a, tcol2 / ntpb, (tcol2 % ntpb) * TCH, k2, w, l);
        };
        if (real) {
            const int64_t b = tcol / ntpb;
            const int64_t ch0 = (tcol % ntpb) * TCH;
            const int64_t tail = L - k * kChunk;  // tokens of this chunk that exist
            if (tail < kChunk) {
                // Tokens past the end were loaded from the last token; give them
                // delta = 0 so that they leave the state unchanged.
                for (int i = threadIdx.x; i < (kChunk - (int)tail) * TCH; i += 64 * kWaves)
                    tb.dl[tail + i / TCH][i % TCH] = T(0.0f);
                lds_barrier();
            }
#pragma unroll 1
            for (int sub = 0; sub < SUBS; ++sub) {
                if (ch0 + sub * CPW >= D) break;                    // no channel of this item exists
                const int cl = sub * CPW + (row / NGR) * 16 + k16;  // channel within the tile
                const int64_t d = ch0 + cl;
                const bool valid = d < D;
                const int64_t dc = valid ? d : D - 1;
                const int64_t icol = tcol * SUBS + sub;            // item column
                const int64_t item = k * a.nicol + icol;

                float A2[NL];
#pragma unroll
                for (int j = 0; j < NL; ++j) A2[j] = tb.A[cl][nstate0 + j] * kLog2e;

                // Early look-back: fetch the predecessor's inclusive state (if it
                // is already out) into LDS; it is checked after phase A. Going
                // through LDS keeps these loads out of the registers and waits
                // of the other waves.
                uint64_t early1 = 0;  // N = 1: one 8-byte word, loaded directly
                if (w == 0 && k > 0) {
                    const uint64_t *src = a.incl + ((k - 1) * a.nicol + icol) * (64 * NL) + l * NL;
                    if constexpr (NL >= 2) {
#pragma unroll
                        for (int p = 0; p < NL / 2; ++p) dma16_coherent(src + 2 * p, lds_addr(&sh.early[p][0][0]));
                    } else {
                        early1 = ld_tagged(src);
                    }
                }

                // Inputs of this wave's segment from the tile (tokens past the
                // end have delta = 0 there: the identity map).
                float xv[kSegT], dv[kSegT];
#pragma unroll
                for (int t = 0; t < kSegT; ++t) {
                    const int tw = w * kSegT + t;
                    xv[t] = ld_act(&tb.x[tw][0], cl);
                    dv[t] = ld_act(&tb.dl[tw][0], cl);
                }
                float Bq[BREGS], Cq[BREGS];
#pragma unroll
                for (int q = 0; q < BREGS; ++q) {
                    const int tw = w * kSegT + q * TPV + k16 / NL;
                    Bq[q] = ld_act(&tb.B[tw][0], nstate0 + (k16 % NL));
                    Cq[q] = ld_act(&tb.C[tw][0], nstate0 + (k16 % NL));
                }

                // Phase A: discretise, keep dA (the exponentials) and delta*x,
                // fold the segment. dBx = B*(delta*x) is one multiply and is
                // formed again in phase C rather than held in registers.
                float dA[kSegT][NL], dx[kSegT], S[NL];
                float dsum = 0.0f;
#pragma unroll
                for (int j = 0; j < NL; ++j) S[j] = 0.0f;
                static_for<0, kSegT>([&](auto tc) {
                    constexpr int t = decltype(tc)::value;
                    dx[t] = dv[t] * xv[t];
                    dsum += dv[t];
                    static_for<0, NL>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        dA[t][j] = fast_exp2(dv[t] * A2[j]);
                        const float u = row_bcast<(t % TPV) * NL + j>(Bq[t / TPV]) * dx[t];
                        S[j] = __builtin_fmaf(dA[t][j], S[j], u);
                    });
                });
#pragma unroll
                for (int j = 0; j < NL; ++j) sh.seg_s[w][l][j] = S[j];
                sh.seg_d[w][l] = dsum;
                lds_barrier();

                // Earlier segments of this item folded from a zero start; read
                // between the two barriers, so the segment buffers need no copy.
                float pre_s[NL], pre_d;
                fold_segments<NL>(sh.seg_s, sh.seg_d, l, w, A2, pre_s, pre_d);
                const bool publish = k + 1 < a.K;  // a later chunk reads this item's words

                // With several chunks of a column in flight at once, every item
                // publishes its aggregate right away (wave 2), so that its
                // successors can fold it in without waiting for its state.
                if (a.agg_early && w == 2 && publish) {
                    float Sagg[NL], dagg;
                    fold_segments<NL>(sh.seg_s, sh.seg_d, l, kWaves, A2, Sagg, dagg);
                    publish_aggregate<NL>(a.agg + item * (64 * (NL + 1)), l, Sagg, dagg, a.epoch);
                }

                if (sub == 0) hand_over();

                if (w == 0) {
                    float H[NL];
                    if (k == 0) {
                        const float *si = a.state_in ? a.state_in + (b * D + dc) * N + nstate0 : nullptr;
#pragma unroll
                        for (int j = 0; j < NL; ++j) H[j] = si ? si[j] : 0.0f;
                    } else {
                        uint64_t early[NL];
                        if constexpr (NL >= 2) {
                            vm_wait();
#pragma unroll
                            for (int j = 0; j < NL; ++j) early[j] = sh.early[j / 2][l][j % 2];
                        } else {
                            early[0] = early1;
                        }
                        bool ok = true;
#pragma unroll
                        for (int j = 0; j < NL; ++j) ok = ok && (uint32_t)(early[j] >> 32) == a.epoch;
                        if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
#pragma unroll
                            for (int j = 0; j < NL; ++j) H[j] = __uint_as_float((uint32_t)early[j]);
                        } else {
                            // Slow path. Publish this item's aggregate (unless wave 2
                            // has) so that later items can fold it in without waiting
                            // for it, then find the nearest earlier item whose
                            // inclusive state is out with the aggregates of all items
                            // after it out.
                            if (publish && !a.agg_early) {
                                float Sagg[NL], dagg;
                                fold_segments<NL>(sh.seg_s, sh.seg_d, l, kWaves, A2, Sagg, dagg);
                                publish_aggregate<NL>(a.agg + item * (64 * (NL + 1)), l, Sagg, dagg, a.epoch);
                            }
                            int64_t base = k - 1;  // chunk examined by lane 0
                            int64_t j0 = -1;
                            long spin = 0;
                            while (true) {
                                const int64_t jj = base - l;  // chunk examined by this lane
                                bool inc = false, agg = false;
                                if (jj >= 0) {
                                    // the first word of an item's record stands for all of it;
                                    // the replay below still checks every word it reads
                                    const int64_t it2 = jj * a.nicol + icol;
                                    inc = (uint32_t)(ld_tagged(a.incl + it2 * (64 * NL)) >> 32) == a.epoch;
                                    agg = inc || (uint32_t)(ld_tagged(a.agg + it2 * (64 * (NL + 1))) >> 32) == a.epoch;
                                }
                                const uint64_t m_inc = __builtin_amdgcn_ballot_w64(inc);
                                const uint64_t m_agg = __builtin_amdgcn_ballot_w64(agg);
                                if (m_inc) {
                                    const int i0 = __builtin_ctzll(m_inc);
                                    const uint64_t below = i0 == 0 ? 0 : (~0ull >> (64 - i0));
                                    if ((m_agg & below) == below) {
                                        j0 = base - i0;
                                        break;
                                    }
                                } else if (m_agg == ~0ull) {
                                    base -= 64;  // 64 aggregates and no inclusive state yet: look further back
                                    spin = 0;
                                    continue;
                                }
                                if (++spin > kSpinLimit ||
                                    (spin % 64 == 0 && __builtin_amdgcn_readfirstlane(ld_flag(a.error)) != 0)) {
                                    if (l == 0) __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                    break;
                                }
                                __builtin_amdgcn_s_sleep(2);
                            }
                            if (j0 < 0) {
#pragma unroll
                                for (int j = 0; j < NL; ++j) H[j] = 0.0f;
                            } else {
                                // Replay the chain forward from that state with the
                                // arithmetic each item uses for its own inclusive
                                // state, kReplay aggregates per round trip.
                                const uint64_t *src = a.incl + (j0 * a.nicol + icol) * (64 * NL) + l * NL;
#pragma unroll
                                for (int j = 0; j < NL; ++j) H[j] = __uint_as_float((uint32_t)ld_valid(src + j, a.epoch));
                                for (int64_t jj = j0 + 1; jj < k; jj += kReplay) {
                                    uint64_t sv[kReplay][NL], dv2[kReplay];
#pragma unroll
                                    for (int q = 0; q < kReplay; ++q) {
                                        if (jj + q < k) {
                                            const uint64_t *ag = a.agg + ((jj + q) * a.nicol + icol) * (64 * (NL + 1));
#pragma unroll
                                            for (int j = 0; j < NL; ++j) sv[q][j] = ld_tagged(ag + l * NL + j);
                                            dv2[q] = ld_tagged(ag + 64 * NL + l);
                                        }
                                    }
#pragma unroll
                                    for (int q = 0; q < kReplay; ++q) {
                                        if (jj + q < k) {
                                            const uint64_t *ag = a.agg + ((jj + q) * a.nicol + icol) * (64 * (NL + 1));
                                            const float dd = __uint_as_float((uint32_t)recheck(dv2[q], ag + 64 * NL + l, a.epoch));
#pragma unroll
                                            for (int j = 0; j < NL; ++j)
                                                H[j] = __builtin_fmaf(fast_exp2(A2[j] * dd), H[j],
                                                                      __uint_as_float((uint32_t)recheck(sv[q][j], ag + l * NL + j, a.epoch)));
                                        }
                                    }
                                }
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < NL; ++j) sh.carry[l][j] = H[j];
                }
                lds_barrier();
                if (sub == 0) start_next();

                // This wave's carried-in state: the item's, pushed through the
                // earlier segments (folded above, before the barrier).
                float h[NL], H[NL];
#pragma unroll
                for (int j = 0; j < NL; ++j) {
                    H[j] = sh.carry[l][j];
                    h[j] = __builtin_fmaf(fast_exp2(A2[j] * pre_d), H[j], pre_s[j]);
                }
                // The last wave publishes the item's inclusive state (its own
                // segment completes the aggregate in its registers); wave 0's
                // memory queue stays free for the next item's look-back.
                if (w == kWaves - 1 && publish) {
                    uint64_t *dst = a.incl + item * (64 * NL) + l * NL;
                    const float dagg = pre_d + dsum;
#pragma unroll
                    for (int j = 0; j < NL; ++j) {
                        const float sagg = __builtin_fmaf(fast_exp2(A2[j] * dsum), pre_s[j], S[j]);
                        st_tagged(dst + j, __builtin_fmaf(fast_exp2(A2[j] * dagg), H[j], sagg), a.epoch);
                    }
                }

                // Phase C: rescan from registers; partial readout over this lane's states.
                float yp[kSegT];
                static_for<0, kSegT>([&](auto tc) {
                    constexpr int t = decltype(tc)::value;
                    yp[t] = 0.0f;
                    static_for<0, NL>([&](auto jc) {
                        constexpr int j = decltype(jc)::value;
                        const float u = row_bcast<(t % TPV) * NL + j>(Bq[t / TPV]) * dx[t];
                        h[j] = __builtin_fmaf(dA[t][j], h[j], u);
                        fmac_bcast<(t % TPV) * NL + j>(yp[t], Cq[t / TPV], h[j]);
                    });
                });

                if (k == a.K - 1 && w == kWaves - 1 && a.state_out && valid) {
                    float *so = a.state_out + (b * D + d) * N + nstate0;
#pragma unroll
                    for (int j = 0; j < NL; ++j) so[j] = h[j];
                }

                // Sum the partial readouts over a channel's rows. Afterwards
                // row r holds the finished token t = NGR*q + (r % NGR) of group q.
                float yo[G::OWN];
                if constexpr (NGR == 4) {
#pragma unroll
                    for (int q = 0; q < kSegT / 4; ++q) {
                        float a0 = yp[4 * q + 0], a2 = yp[4 * q + 2], a1 = yp[4 * q + 1], a3 = yp[4 * q + 3];
                        swap_halves(a0, a2);  // rows 0,1: token 0 | rows 2,3: token 2
                        swap_halves(a1, a3);  // rows 0,1: token 1 | rows 2,3: token 3
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

                // Finish the owned tokens (D skip, silu gate) into the tile.
                const float dskip = SKIP ? tb.Dsk[cl] : 0.0f;
#pragma unroll
                for (int q = 0; q < G::OWN; ++q) {
                    const int t = NGR * q + g;
                    const int tw = w * kSegT + t;
                    const float xt = ld_act(&tb.x[tw][0], cl);
                    float yv = yo[q];
                    if (SKIP) yv = __builtin_fmaf(dskip, xt, yv);
                    if (GATE) yv *= silu(ld_act(&tb.z[tw][0], cl));
                    st_act(&tb.dl[tw][0], cl, yv);
                }
            }
        }
        if (!real) {
            hand_over();
            lds_barrier();
            start_next();
        }
        lds_barrier();
        // Store the finished y tile as whole lines (waves 1..3), then make sure
        // the next tile has landed before anyone reads it.
        if (real && w > 0) {
            using VT = uint32_t __attribute__((ext_vector_type(4)));
            constexpr int PPR = TCH / G::VEC;
            const int64_t b = tcol / ntpb, ch0 = (tcol % ntpb) * TCH;
            T *yptr = (T *)a.y;
            for (int p = (w - 1) * 64 + l; p < kChunk * PPR; p += 3 * 64) {
                const int r = p / PPR, c = (p % PPR) * G::VEC;
                const int64_t t = k * kChunk + r;
                if (t < L && ch0 + c < D) {
                    const VT v = *(const VT *)&tb.dl[r][c];
                    *(VT *)(yptr + (b * L + t) * D + ch0 + c) = v;
                }
            }
        }
        if (w > 0) vm_wait();
        lds_barrier();
        s = s_next;
        ++it;
    }
}

template <int N, int DT, bool GATE, bool SKIP>
hipError_t launch_lb_typed(const LbArgs &a, hipStream_t s) {
    auto kern = scan_lb_kernel<N, DT, GATE, SKIP>;
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
    using G = Geo<N, DT>;
    const int64_t ntcol = a.batch * ((a.D + G::TCH - 1) / G::TCH);
    const int64_t tpx = (ntcol + kXcds - 1) / kXcds;
    const int64_t need = tpx * a.K * kXcds;  // one workgroup per tile is the most that helps
    int64_t grid = (int64_t)cus * per_cu / kXcds * kXcds;
    if (grid > need) grid = need;
    if (grid < kXcds) grid = kXcds;
    LbArgs args = a;
    // more workgroups per XCD than tile columns: chunks of a column overlap
    args.agg_early = grid / kXcds > tpx;
    void *params[] = {&args};
    return hipLaunchKernel((const void *)kern, dim3((unsigned)grid), dim3(64 * kWaves), params, 0, s);
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

template <int N, int DT>
void lb_geometry(int64_t batch, int64_t L, int64_t D, LbPlan *p) {
    using G = Geo<N, DT>;
    p->nl = G::NL;
    p->nicol = batch * ((D + G::TCH - 1) / G::TCH) * G::SUBS;
    p->K = (L + kChunk - 1) / kChunk;
    p->vec = G::VEC;
    p->tiles_per_list = (batch * ((D + G::TCH - 1) / G::TCH) + kXcds - 1) / kXcds * p->K;
}

}  // namespace

bool lb_plan(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype, LbPlan *p) {
    const bool bf = dtype == 1;
    switch (N) {
        case 1: bf ? lb_geometry<1, 1>(batch, L, D, p) : lb_geometry<1, 0>(batch, L, D, p); break;
        case 2: bf ? lb_geometry<2, 1>(batch, L, D, p) : lb_geometry<2, 0>(batch, L, D, p); break;
        case 4: bf ? lb_geometry<4, 1>(batch, L, D, p) : lb_geometry<4, 0>(batch, L, D, p); break;
        case 8: bf ? lb_geometry<8, 1>(batch, L, D, p) : lb_geometry<8, 0>(batch, L, D, p); break;
        case 16: bf ? lb_geometry<16, 1>(batch, L, D, p) : lb_geometry<16, 0>(batch, L, D, p); break;
        default: return false;
    }
    p->chunk = kChunk;
    // Tiles are read as 16-byte pieces: channel rows must be whole pieces and
    // Bt/Ct rows at least one piece.
    const int esz = bf ? 2 : 4;
    p->supported = (D % p->vec == 0) && (N * esz >= 16);
    // tile indices of one XCD's list must fit the counters (and a 32-bit lane)
    if (p->tiles_per_list >= (int64_t(1) << 30)) p->supported = false;
    const int64_t items = p->nicol * p->K;
    // header (error word, tile counters) | incl | agg, all words epoch-tagged:
    // per item, incl holds 64 lanes x NL state words and agg 64 x NL state
    // words followed by 64 summed-delta words
    size_t off = 256;
    p->off_incl = off;
    off += (size_t)items * 64 * p->nl * sizeof(uint64_t);
    p->off_agg = off;
    off += (size_t)items * 64 * (p->nl + 1) * sizeof(uint64_t);
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
