// Internal interfaces between the C ABI (ssm_abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

// Everything one scan launch needs. Pointers are device pointers.
struct ScanArgs {
    int64_t batch, L, D;
    const void *x, *delta, *Bt, *Ct, *z;
    const float *A, *Dskip, *state_in;
    const float *dt_bias;  // per-channel bias of the raw step size (NULL = 0)
    int delta_softplus;    // delta holds the raw step size: use softplus(delta + dt_bias)
    // exponential-trapezoidal rule: per-token weight lam (NULL = the Euler
    // rule) and the token before the first (x_prev, B_prev; NULL = none)
    const void *lam, *x_prev, *B_prev;
    // the x branch ahead of the scan: x holds the raw input of a causal
    // depthwise convolution with taps conv_w (D, 4) (tap 3 on the token itself)
    // and bias conv_b (D; NULL = 0), followed by SiLU; conv_state (batch, D, 3,
    // activation dtype; NULL = zeros) is the raw x of the three tokens before
    // token 0. conv_w NULL: x is used as given.
    const float *conv_w, *conv_b;
    const void *conv_state;
    float *state_out;
    void *y;
    float *ws_state;   // (batch, K, D, N) chunk end states, then carried-in states
    float *ws_dsum;    // (batch, K, D)    summed delta per chunk
    int64_t K;         // number of sequence chunks
    int64_t Lc;        // tokens per chunk (the last chunk may be shorter)
};

// Header of a scan workspace: the first kHdrBytes bytes, as 32-bit words.
// The kernels keep it consistent from call to call; it must be zero before the
// workspace is first used.
//  [kHdrError]    tag of the last call in which a wait for another workgroup's
//                 words gave up (0: none)
//  [kHdrEpoch]    tag of the last call that finished (0: none yet). A call tags
//                 the words it publishes with this value plus one (skipping 0),
//                 read on the device, so a launch replayed from a graph gets a
//                 new tag like any other.
//  [kHdrDone]     workgroups of the running call that have finished (0 between
//                 calls); the last one advances kHdrEpoch and clears this word
//  [kHdrCounters] eight unit counters (0 between calls)
constexpr int kHdrError = 0, kHdrEpoch = 1, kHdrDone = 2, kHdrCounters = 16;
constexpr size_t kHdrBytes = 256;

// Stripe scan: every wave walks its channels along a stripe of the sequence.
struct StripeArgs {
    int64_t batch, L, D;
    const void *x, *delta, *Bt, *Ct, *z;
    const float *A, *Dskip, *state_in;
    const float *dt_bias;  // per-channel bias of the raw step size (NULL = 0)
    int delta_softplus;    // delta holds the raw step size: use softplus(delta + dt_bias)
    // exponential-trapezoidal rule: per-token weight lam (NULL = the Euler
    // rule) and the token before the first (x_prev, B_prev; NULL = none)
    const void *lam, *x_prev, *B_prev;
    // the x branch ahead of the scan (as in ScanArgs)
    const float *conv_w, *conv_b;
    const void *conv_state;
    float *state_out;
    void *y;
    int64_t ntpb;           // tile columns per batch row
    int64_t ncol;           // tile columns
    int64_t cols_per_list;  // tile columns per unit list
    int64_t n_whole;        // columns per list run as one whole-sequence unit each
    int64_t S;              // stripes per remaining column
    int64_t SL;             // tokens per stripe (the last one may be shorter)
    int early;              // cut stripes take early mode (scan from zero first, then a pass 2 that may stop early)
    uint32_t *hdr;          // the workspace header (kHdr* words)
    uint64_t *incl;         // per (column, stripe, wave): end state, epoch-tagged words
    uint64_t *agg;          // per (column, stripe, wave): end state from zero and summed delta
};

struct StripePlan {
    int64_t nl, tch, tt, vec, ntpb, ncol, cols_per_list, n_whole, S, SL;
    bool early;         // stripes are long enough for early mode
    bool supported;     // shape meets the tile-load requirements
    size_t off_incl, off_agg, bytes;
};

struct StepArgs {
    int64_t batch, D;
    const void *x, *delta, *Bt, *Ct, *z;
    const float *A, *Dskip;
    const float *dt_bias;  // per-channel bias of the raw step size (NULL = 0)
    int delta_softplus;    // delta holds the raw step size: use softplus(delta + dt_bias)
    // exponential-trapezoidal rule: per-token weight lam (NULL = the Euler
    // rule) and the token before the first (x_prev, B_prev; NULL = none)
    const void *lam, *x_prev, *B_prev;
    // the x branch ahead of the step (as in ScanArgs): taps conv_w (D, 4),
    // bias conv_b (D; NULL = 0) and conv_state (batch, D, 3, activation
    // dtype), the raw x of the three tokens before this one, which the step
    // shifts in place to end with this token's raw x. conv_w NULL: x is used
    // as given.
    const float *conv_w, *conv_b;
    void *conv_state;
    float *state;
    void *y;
};

// Mamba-2 SSD layer: x, y (batch, L, H, P); delta (batch, L, H); Bt, Ct
// (batch, L, G, N); A, Dskip (H); state (batch, H, P, N); bfloat16 activations.
struct SsdArgs {
    int64_t batch, L, H, G;
    const void *x, *delta, *Bt, *Ct;
    const float *A, *Dskip, *state_in;
    float *state_out;
    void *y;
};
bool ssd_supported(int64_t P, int64_t N);

// Mamba-2 SSD decode step: x, y (batch, H, P); delta (batch, H); Bt, Ct
// (batch, G, N); A, Dskip (H); state (batch, H, P, N) float, in place.
struct SsdStepArgs {
    int64_t batch, H, G;
    const void *x, *delta, *Bt, *Ct;
    const float *A, *Dskip;
    float *state;
    void *y;
};
bool ssd_step_supported(int64_t P, int64_t N);
hipError_t launch_ssd_step(const SsdStepArgs &a, int N, int dtype, hipStream_t s);
hipError_t launch_ssd(const SsdArgs &a, int N, hipStream_t s);

// Gradient of the scan (Euler rule, delta after its activation). Pointers are
// device pointers; dx, ddelta, dz in the activation dtype, the rest float.
constexpr int64_t kBwdChunk = 32;  // tokens per chunk of the gradient
constexpr int kBwdSub = 8;         // tokens per recomputed block of a chunk
constexpr int kBwdCk = (int)(kBwdChunk / kBwdSub) - 1;  // block entries inside a chunk
// State elements per lane in the gradient's chunk kernel: 8 (two lanes per
// channel at N = 16), and 4 for the trapezoidal rule, whose reverse step
// keeps one more vector per lane (measured faster with four lanes).
constexpr int bwd_np(int64_t N, bool trap) { return (int)(N < (trap ? 4 : 8) ? N : (trap ? 4 : 8)); }
struct BwdArgs {
    int64_t batch, L, D, K;  // K = ceil(L / kBwdChunk) chunks
    const void *x, *delta, *Bt, *Ct, *z, *dy;
    const float *A, *Dskip, *state_in, *dstate;
    const float *dt_bias;  // per-channel bias of the raw step size (NULL = 0)
    int delta_softplus;    // delta holds the raw step size: the scan used softplus(delta + dt_bias)
    void *dx, *ddelta, *dz;  // with delta_softplus, ddelta is the gradient of the raw step size
    float *dA, *dBt, *dCt, *dDskip, *dstate_in;
    float *ddt_bias;       // gradient of dt_bias (NULL = not written)
    // exponential-trapezoidal rule: the weight lam (NULL = the Euler rule) and
    // the token before the first (x_prev, B_prev; NULL = none); the gradients
    // of lam (dtype) and of the token before (dx_prev dtype, dB_prev float;
    // NULL = not written)
    const void *lam, *x_prev, *B_prev;
    void *dlam, *dx_prev;
    float *dB_prev;
    // workspace
    float *hst;         // (batch, K, D, N) state entering each chunk
    float *dsum;        // (batch, K, D)    summed delta per chunk
    float *gq;          // (batch, K, D, N) gradient entering each chunk from its end
    float *pdB, *pdC;   // (bwd_channel_blocks, batch, L, N) per-block partial sums
    float *pdA;         // (batch, K, D, N) per-chunk partial sums
    float *pdD;         // (batch, K, D)
    float *pdT;         // (batch, K, D)    partial sums of ddt_bias
    float *pdBp;        // (bwd_channel_blocks, batch, N) partial sums of dB_prev
    float *ckp;         // (batch, K, kBwdCk, D, N) state at each block entry inside a chunk, from a zero chunk start
    float *ckd;         // (batch, K, kBwdCk, D)    summed delta from the chunk start to each block entry
};
hipError_t launch_scan_bwd(const BwdArgs &a, int N, int dtype, hipStream_t s);
// The instances for the exponential-trapezoidal rule (called by launch_scan_bwd).
hipError_t launch_scan_bwd_trap(const BwdArgs &a, int N, int dtype, hipStream_t s);
// Channel blocks of the gradient's chunk kernel (256 lanes, N / bwd_np lanes
// per channel): the number of partials of dBt and dCt.
inline int64_t bwd_channel_blocks(int64_t D, int64_t N, bool trap) {
    const int64_t cpb = 256 / (N / bwd_np(N, trap));
    return (D + cpb - 1) / cpb;
}

// Sequence split used for a scan of these sizes (deterministic).
void scan_plan(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t *K, int64_t *Lc);

bool stripe_plan(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype, StripePlan *p);

// The gradient through the x branch ahead of the scan (ssm_conv_bwd.hip).
// Pointers are device pointers; x_raw, conv_state, xc, gx, dx_raw and
// dconv_state in the activation dtype, the rest float.
struct ConvBwdArgs {
    int64_t batch, L, D;
    int64_t chunk, nchunk;  // tokens per chunk of conv_bwd_kernel, chunks per batch row
    const void *x_raw, *conv_state;  // the branch's input; the raw x of the three tokens before (NULL = 0)
    const float *conv_w, *conv_b;    // taps (D, 4), bias (D; NULL = 0)
    void *xc;                        // (batch, L, D) the branch's output (conv_fwd_kernel)
    const void *gx;                  // (batch, L, D) the gradient of that output
    void *dx_raw, *dconv_state;      // gradients of x_raw and conv_state (NULL: not written)
    float *dconv_w, *dconv_b;        // gradients of the taps and bias (dconv_b NULL: not written)
    float *part;                     // (batch * nchunk, D, 5) partial sums of the taps' and bias' gradients
};
void conv_bwd_plan(int64_t batch, int64_t L, int64_t D, int64_t *chunk, int64_t *nchunk);
hipError_t launch_conv_fwd(const ConvBwdArgs &a, int dtype, hipStream_t s);
hipError_t launch_conv_bwd(const ConvBwdArgs &a, int dtype, hipStream_t s);

// Launchers; return hipSuccess or the launch error.// Launchers; return hipSuccess or the launch error.
hipError_t launch_scan_stripe(const StripeArgs &a, int N, int dtype, hipStream_t s);
// The instances for a delta given before its activation (called by launch_scan_stripe).
hipError_t launch_scan_stripe_act(const StripeArgs &a, int N, int dtype, hipStream_t s);
// The instances for the x branch ahead of the scan, with a delta given before
// its activation (called by launch_scan_stripe).
hipError_t launch_scan_stripe_conv(const StripeArgs &a, int N, int dtype, hipStream_t s);
// The instances for the exponential-trapezoidal rule (called by launch_scan_stripe).
hipError_t launch_scan_stripe_trap(const StripeArgs &a, int N, int dtype, hipStream_t s);
hipError_t launch_scan(const ScanArgs &a, int N, int dtype, hipStream_t s);
// ssm_scan_fwd's checks and launches (ssm_abi.cpp), for the entry points that
// bring their own workspace; launch = false runs the checks only.
int scan_fwd_euler(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype, const void *x, const void *delta,
                   const float *A, const void *Bt, const void *Ct, const float *Dskip, const void *z,
                   const float *state_in, float *state_out, void *y, void *workspace, size_t workspace_bytes,
                   void *stream, bool launch);
hipError_t launch_state_copy(const float *src, float *dst, int64_t n, hipStream_t s);
hipError_t launch_step(const StepArgs &a, int N, int dtype, hipStream_t s);

}  // namespace ssm
