// Selective scan (S6) forward organised by stripes: the plan, and the
// instances for a delta given after its activation.
#include "ssm_scan_stripe_kernel.h"

namespace ssm {

bool stripe_plan(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype, StripePlan *p) {
    const bool bf = dtype == 1;
    switch (N) {
        case 1: bf ? stripe_geometry<1, 1>(batch, L, D, p) : stripe_geometry<1, 0>(batch, L, D, p); break;
        case 2: bf ? stripe_geometry<2, 1>(batch, L, D, p) : stripe_geometry<2, 0>(batch, L, D, p); break;
        case 4: bf ? stripe_geometry<4, 1>(batch, L, D, p) : stripe_geometry<4, 0>(batch, L, D, p); break;
        case 8: bf ? stripe_geometry<8, 1>(batch, L, D, p) : stripe_geometry<8, 0>(batch, L, D, p); break;
        case 16: bf ? stripe_geometry<16, 1>(batch, L, D, p) : stripe_geometry<16, 0>(batch, L, D, p); break;
        default: return false;
    }
    // Tiles are read as 16-byte pieces: channel rows must be whole pieces
    // (and at least one), and Bt/Ct rows at least one piece.
    const int esz = bf ? 2 : 4;
    p->supported = (D % p->vec == 0) && (D >= p->vec) && (N * esz >= 16) &&
                   (p->cols_per_list * p->S < (int64_t(1) << 30));
    const int64_t n_split = p->cols_per_list - p->n_whole;
    // header (error word, unit counters) | incl | agg: per record 64 lanes x
    // NL end-state words, and 64 x NL state words followed by 64 summed-delta
    // words; one record per (tile column, stripe, wave)
    const int64_t recs = p->S > 1 ? kLists * n_split * p->S * kWaves : 0;
    size_t off = 256;
    p->off_incl = off;
    off += (size_t)recs * 64 * p->nl * sizeof(uint64_t);
    p->off_agg = off;
    off += (size_t)recs * 64 * (p->nl + 1) * sizeof(uint64_t);
    p->bytes = (off + 255) / 256 * 256;
    return true;
}

hipError_t launch_scan_stripe(const StripeArgs &a, int N, int dtype, hipStream_t s) {
    if (a.lam) return launch_scan_stripe_trap(a, N, dtype, s);
    if (a.conv_w) return launch_scan_stripe_conv(a, N, dtype, s);
    if (a.delta_softplus) return launch_scan_stripe_act(a, N, dtype, s);
    return launch_stripe_n<kEuler>(a, N, dtype, s);
}

}  // namespace ssm
