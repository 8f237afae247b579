// Gradient of the selective scan (S6): the instances for the exponential-Euler
// rule (step size given, or given before its activation) and the dispatch.
#include "ssm_scan_bwd_kernel.h"

namespace ssm {

namespace {

template <int N, int DT>
hipError_t launch_bwd_act(const BwdArgs &a, hipStream_t s) {
    return a.delta_softplus ? launch_bwd_flags<N, DT, kBwdSoftplus>(a, s) : launch_bwd_flags<N, DT, kBwdEuler>(a, s);
}

template <int N>
hipError_t launch_bwd_dtype(const BwdArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch_bwd_act<N, 0>(a, s) : launch_bwd_act<N, 1>(a, s);
}

}  // namespace

hipError_t launch_scan_bwd(const BwdArgs &a, int N, int dtype, hipStream_t s) {
    if (a.lam) return launch_scan_bwd_trap(a, N, dtype, s);
    switch (N) {
        case 1: return launch_bwd_dtype<1>(a, dtype, s);
        case 2: return launch_bwd_dtype<2>(a, dtype, s);
        case 4: return launch_bwd_dtype<4>(a, dtype, s);
        case 8: return launch_bwd_dtype<8>(a, dtype, s);
        case 16: return launch_bwd_dtype<16>(a, dtype, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
