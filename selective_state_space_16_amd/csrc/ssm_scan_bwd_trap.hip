// Gradient of the selective scan (S6): the instances for the
// exponential-trapezoidal rule.
#include "ssm_scan_bwd_kernel.h"

namespace ssm {

namespace {

template <int N>
hipError_t launch_bwd_trap_dtype(const BwdArgs &a, int dtype, hipStream_t s) {
    return dtype == 0 ? launch_bwd_flags<N, 0, kBwdTrap>(a, s) : launch_bwd_flags<N, 1, kBwdTrap>(a, s);
}

}  // namespace

hipError_t launch_scan_bwd_trap(const BwdArgs &a, int N, int dtype, hipStream_t s) {
    switch (N) {
        case 1: return launch_bwd_trap_dtype<1>(a, dtype, s);
        case 2: return launch_bwd_trap_dtype<2>(a, dtype, s);
        case 4: return launch_bwd_trap_dtype<4>(a, dtype, s);
        case 8: return launch_bwd_trap_dtype<8>(a, dtype, s);
        case 16: return launch_bwd_trap_dtype<16>(a, dtype, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssm
