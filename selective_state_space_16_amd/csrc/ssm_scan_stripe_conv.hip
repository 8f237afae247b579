// Selective scan (S6) forward organised by stripes: the instances for the x
// branch ahead of the scan (SiLU of a causal width-4 convolution of x) with a
// delta given before its activation.
#include "ssm_scan_stripe_kernel.h"

namespace ssm {

hipError_t launch_scan_stripe_conv(const StripeArgs &a, int N, int dtype, hipStream_t s) {
    return launch_stripe_n<kConv>(a, N, dtype, s);
}

}  // namespace ssm
