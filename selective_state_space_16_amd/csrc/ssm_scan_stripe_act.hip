// Selective scan (S6) forward organised by stripes: the instances for a
// delta given before its activation (softplus(delta + dt_bias)).
#include "ssm_scan_stripe_kernel.h"

namespace ssm {

hipError_t launch_scan_stripe_act(const StripeArgs &a, int N, int dtype, hipStream_t s) {
    return launch_stripe_n<kSoftplus>(a, N, dtype, s);
}

}  // namespace ssm
