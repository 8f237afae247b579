// Selective scan (S6) forward organised by stripes: the instances for the
// exponential-trapezoidal rule.
#include "ssm_scan_stripe_kernel.h"

namespace ssm {

hipError_t launch_scan_stripe_trap(const StripeArgs &a, int N, int dtype, hipStream_t s) {
    return launch_stripe_n<kTrap>(a, N, dtype, s);
}

}  // namespace ssm
