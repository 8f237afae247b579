// C ABI of libssm.so: argument checks on the host, then kernel dispatch.
// Every check runs before any HIP call, so a rejected call launches nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/ssm.h"
#include "ssm_internal.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 46;  // keeps every byte offset far from overflow

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool supported_n(int64_t N) { return N == 1 || N == 2 || N == 4 || N == 8 || N == 16; }

// Product of non-negative sizes, or -1 when it exceeds kMaxElems.
int64_t checked_mul(int64_t a, int64_t b) {
    if (a == 0 || b == 0) return 0;
    if (a > kMaxElems / b) return -1;
    return a * b;
}

int64_t checked_mul3(int64_t a, int64_t b, int64_t c) {
    const int64_t ab = checked_mul(a, b);
    return ab < 0 ? -1 : checked_mul(ab, c);
}

size_t round_up256(size_t n) { return (n + 255) / 256 * 256; }

// Both scans keep a header of ssm::kHdrBytes at the start of the workspace
// (its words are described in ssm_internal.h); the chunked scan leaves it alone.
constexpr size_t kHeader = ssm::kHdrBytes;

// Workspace of the chunked three-launch scan:
// [header | chunk states (batch,K,D,N) | summed deltas (batch,K,D)].
size_t twopass_workspace(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t *K, int64_t *Lc) {
    ssm::scan_plan(batch, L, D, N, K, Lc);
    if (*K <= 1) return 0;
    return kHeader + round_up256((size_t)batch * *K * D * N * sizeof(float)) +
           round_up256((size_t)batch * *K * D * sizeof(float));
}

// Workspace of the stripe scan.
size_t stripe_workspace(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype, ssm::StripePlan *p) {
    if (!ssm::stripe_plan(batch, L, D, N, dtype, p)) return 0;
    return p->bytes;
}

// Which scan runs. The stripe scan reads 16-byte pieces of channel rows and
// Bt/Ct rows; shapes it cannot take run the chunked three-launch scan, which
// SSM_SCAN_IMPL=twopass also selects (for comparison).
enum class Impl { kTwopass, kStripe };

Impl choose_impl(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype) {
    ssm::StripePlan sp;
    const bool stripe_ok = ssm::stripe_plan(batch, L, D, N, dtype, &sp) && sp.supported;
    const char *e = getenv("SSM_SCAN_IMPL");
    if (e && strcmp(e, "twopass") == 0) return Impl::kTwopass;
    return stripe_ok ? Impl::kStripe : Impl::kTwopass;
}

// Whether cut stripes take early mode: by their length, or as
// SSM_STRIPE_EARLY=0/1 says (for comparison and tests).
int stripe_early(const ssm::StripePlan &p) {
    const char *e = getenv("SSM_STRIPE_EARLY");
    if (e && (strcmp(e, "0") == 0 || strcmp(e, "1") == 0)) return e[0] == '1';
    return p.early ? 1 : 0;
}

size_t workspace_for(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype) {
    int64_t K, Lc;
    ssm::StripePlan sp;
    return choose_impl(batch, L, D, N, dtype) == Impl::kStripe ? stripe_workspace(batch, L, D, N, dtype, &sp)
                                                               : twopass_workspace(batch, L, D, N, &K, &Lc);
}

}  // namespace

extern "C" {

const char *ssm_status_string(int status) {
    switch (status) {
        case SSM_OK: return "ok";
        case SSM_ERR_NULL: return "a required pointer is NULL";
        case SSM_ERR_SHAPE: return "a size is negative or the tensor sizes overflow";
        case SSM_ERR_DTYPE: return "dtype must be SSM_F32 or SSM_BF16";
        case SSM_ERR_UNSUPPORTED: return "N must be 1, 2, 4, 8 or 16";
        case SSM_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case SSM_ERR_WORKSPACE: return "workspace is missing or too small";
        case SSM_ERR_HIP: return "a HIP launch failed";
        case SSM_ERR_TIMEOUT: return "a wait for another workgroup's results gave up; the outputs that depend on them are NaN";
        default: return "unknown status";
    }
}

const char *ssm_version(void) { return "ssm-gfx950 0.1"; }

int ssm_scan_workspace_status(const void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace || workspace_bytes < kHeader) return SSM_OK;  // no header: nothing can have failed
    if (!aligned16(workspace)) return SSM_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    uint32_t hdr[4] = {0, 0, 0, 0};
    if (hipMemcpyAsync(hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost, s) != hipSuccess) return SSM_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SSM_ERR_HIP;
    // the last call failed when the error word carries its tag
    return hdr[ssm::kHdrError] != 0 && hdr[ssm::kHdrError] == hdr[ssm::kHdrEpoch] ? SSM_ERR_TIMEOUT : SSM_OK;
}

size_t ssm_scan_workspace_bytes(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype) {
    if (batch < 0 || L < 0 || D < 0 || !supported_n(N)) return 0;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return 0;
    if (checked_mul3(batch, L, D) < 0 || checked_mul3(batch, D, N) < 0) return 0;
    if (batch == 0 || L == 0 || D == 0) return 0;
    return workspace_for(batch, L, D, N, dtype);
}

// Extra inputs of the exponential-trapezoidal rule: the per-token weight and
// the token before the first (both of x_prev and B_prev, or neither); and of
// the x branch ahead of the scan: the taps, bias and earlier raw x of its
// convolution (conv_w NULL: x is used as given).
struct TrapIn {
    const void *lam = nullptr, *x_prev = nullptr, *B_prev = nullptr;
    const float *conv_w = nullptr, *conv_b = nullptr;
    const void *conv_state = nullptr;
};

static int scan_fwd(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                    const void *x, const void *delta, const float *dt_bias, int softplus, const float *A,
                    const void *Bt, const void *Ct, const float *Dskip,
                    const void *z, const float *state_in, float *state_out,
                    void *y, void *workspace, size_t workspace_bytes, void *stream, TrapIn tr = {},
                    bool launch = true) {
    // launch = false: check the arguments only (every check below precedes
    // the first HIP call)
    if (batch < 0 || L < 0 || D < 0 || N < 0) return SSM_ERR_SHAPE;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (!supported_n(N)) return SSM_ERR_UNSUPPORTED;
    if (checked_mul3(batch, L, D) < 0 || checked_mul3(batch, L, N) < 0 || checked_mul3(batch, D, N) < 0)
        return SSM_ERR_SHAPE;
    if (batch == 0 || D == 0) return SSM_OK;
    hipStream_t s = (hipStream_t)stream;
    if (L == 0) {
        if (!state_out) return SSM_OK;
        if (!aligned16(state_out) || (state_in && !aligned16(state_in))) return SSM_ERR_ALIGN;
        if (state_in == state_out || !launch) return SSM_OK;
        return ssm::launch_state_copy(state_in, state_out, batch * D * N, s) == hipSuccess ? SSM_OK
                                                                                          : SSM_ERR_HIP;
    }
    if (!x || !delta || !A || !Bt || !Ct || !y) return SSM_ERR_NULL;
    const void *ptrs[] = {x, delta, A, Bt, Ct, Dskip, z, state_in, state_out, y, dt_bias, tr.lam, tr.x_prev,
                          tr.B_prev, tr.conv_w, tr.conv_b, tr.conv_state};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSM_ERR_ALIGN;

    const size_t need = workspace_for(batch, L, D, N, dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE;
        if (!aligned16(workspace)) return SSM_ERR_ALIGN;
    }
    if (!launch) return SSM_OK;
    const Impl impl = choose_impl(batch, L, D, N, dtype);
    if (impl == Impl::kStripe) {
        ssm::StripePlan p;
        stripe_workspace(batch, L, D, N, dtype, &p);
        ssm::StripeArgs a{};
        a.batch = batch;
        a.L = L;
        a.D = D;
        a.x = x;
        a.delta = delta;
        a.Bt = Bt;
        a.Ct = Ct;
        a.z = z;
        a.A = A;
        a.Dskip = Dskip;
        a.state_in = state_in;
        a.state_out = state_out;
        a.dt_bias = dt_bias;
        a.delta_softplus = softplus;
        a.lam = tr.lam;
        a.x_prev = tr.x_prev;
        a.B_prev = tr.B_prev;
        a.conv_w = tr.conv_w;
        a.conv_b = tr.conv_b;
        a.conv_state = tr.conv_state;
        a.y = y;
        a.ntpb = p.ntpb;
        a.ncol = p.ncol;
        a.cols_per_list = p.cols_per_list;
        a.n_whole = p.n_whole;
        a.S = p.S;
        a.SL = p.SL;
        a.early = stripe_early(p);
        char *w = (char *)workspace;
        a.hdr = (uint32_t *)w;
        a.incl = (uint64_t *)(w + p.off_incl);
        a.agg = (uint64_t *)(w + p.off_agg);
        return ssm::launch_scan_stripe(a, (int)N, dtype, s) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
    }
    ssm::ScanArgs a{};
    a.batch = batch;
    a.L = L;
    a.D = D;
    a.x = x;
    a.delta = delta;
    a.Bt = Bt;
    a.Ct = Ct;
    a.z = z;
    a.A = A;
    a.Dskip = Dskip;
    a.state_in = state_in;
    a.dt_bias = dt_bias;
    a.delta_softplus = softplus;
    a.lam = tr.lam;
    a.x_prev = tr.x_prev;
    a.B_prev = tr.B_prev;
    a.conv_w = tr.conv_w;
    a.conv_b = tr.conv_b;
    a.conv_state = tr.conv_state;
    a.state_out = state_out;
    a.y = y;
    if (twopass_workspace(batch, L, D, N, &a.K, &a.Lc) > 0) {
        char *w = (char *)workspace + kHeader;
        a.ws_state = (float *)w;
        a.ws_dsum = (float *)(w + round_up256((size_t)batch * a.K * D * N * sizeof(float)));
    }
    return ssm::launch_scan(a, (int)N, dtype, s) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

static int step(int64_t batch, int64_t D, int64_t N, int dtype,
                const void *x, const void *delta, const float *dt_bias, int softplus, const float *A,
                const void *Bt, const void *Ct, const float *Dskip,
                const void *z, float *state, void *y, void *stream, TrapIn tr = {}) {
    if (batch < 0 || D < 0 || N < 0) return SSM_ERR_SHAPE;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (!supported_n(N)) return SSM_ERR_UNSUPPORTED;
    if (checked_mul3(batch, D, N) < 0) return SSM_ERR_SHAPE;
    if (batch == 0 || D == 0) return SSM_OK;
    if (!x || !delta || !A || !Bt || !Ct || !state || !y) return SSM_ERR_NULL;
    const void *ptrs[] = {x, delta, A, Bt, Ct, Dskip, z, state, y, dt_bias, tr.lam, tr.x_prev, tr.B_prev,
                          tr.conv_w, tr.conv_b, tr.conv_state};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSM_ERR_ALIGN;
    ssm::StepArgs a{};
    a.batch = batch;
    a.D = D;
    a.x = x;
    a.delta = delta;
    a.Bt = Bt;
    a.Ct = Ct;
    a.z = z;
    a.A = A;
    a.Dskip = Dskip;
    a.state = state;
    a.y = y;
    a.dt_bias = dt_bias;
    a.delta_softplus = softplus;
    a.lam = tr.lam;
    a.x_prev = tr.x_prev;
    a.B_prev = tr.B_prev;
    a.conv_w = tr.conv_w;
    a.conv_b = tr.conv_b;
    a.conv_state = const_cast<void *>(tr.conv_state);
    return ssm::launch_step(a, (int)N, dtype, (hipStream_t)stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_scan_fwd(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                 const void *x, const void *delta, const float *A,
                 const void *Bt, const void *Ct, const float *Dskip,
                 const void *z, const float *state_in, float *state_out,
                 void *y, void *workspace, size_t workspace_bytes, void *stream) {
    return scan_fwd(batch, L, D, N, dtype, x, delta, nullptr, 0, A, Bt, Ct, Dskip, z, state_in, state_out, y,
                    workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_dt(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                    const void *x, const void *delta_raw, const float *dt_bias, const float *A,
                    const void *Bt, const void *Ct, const float *Dskip,
                    const void *z, const float *state_in, float *state_out,
                    void *y, void *workspace, size_t workspace_bytes, void *stream) {
    return scan_fwd(batch, L, D, N, dtype, x, delta_raw, dt_bias, 1, A, Bt, Ct, Dskip, z, state_in, state_out, y,
                    workspace, workspace_bytes, stream);
}

int ssm_scan_fwd_conv(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                      const void *x_raw, const float *conv_w, const float *conv_b, const void *conv_state,
                      const void *delta_raw, const float *dt_bias, const float *A,
                      const void *Bt, const void *Ct, const float *Dskip,
                      const void *z, const float *state_in, float *state_out,
                      void *y, void *workspace, size_t workspace_bytes, void *stream) {
    if (!conv_w && batch > 0 && L > 0 && D > 0) return SSM_ERR_NULL;
    TrapIn tr;
    tr.conv_w = conv_w;
    tr.conv_b = conv_b;
    tr.conv_state = conv_state;
    return scan_fwd(batch, L, D, N, dtype, x_raw, delta_raw, dt_bias, 1, A, Bt, Ct, Dskip, z, state_in, state_out,
                    y, workspace, workspace_bytes, stream, tr);
}

int ssm_scan_fwd_trap(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                      const void *x, const void *delta, const void *lam, const float *A,
                      const void *Bt, const void *Ct, const float *Dskip, const void *z,
                      const void *x_prev, const void *B_prev, const float *state_in, float *state_out,
                      void *y, void *workspace, size_t workspace_bytes, void *stream) {
    if (!lam && batch > 0 && L > 0 && D > 0) return SSM_ERR_NULL;
    if ((x_prev == nullptr) != (B_prev == nullptr)) return SSM_ERR_NULL;
    TrapIn tr;
    tr.lam = lam;
    tr.x_prev = x_prev;
    tr.B_prev = B_prev;
    return scan_fwd(batch, L, D, N, dtype, x, delta, nullptr, 0, A, Bt, Ct, Dskip, z, state_in, state_out, y,
                    workspace, workspace_bytes, stream, tr);
}

int ssm_step(int64_t batch, int64_t D, int64_t N, int dtype,
             const void *x, const void *delta, const float *A,
             const void *Bt, const void *Ct, const float *Dskip,
             const void *z, float *state, void *y, void *stream) {
    return step(batch, D, N, dtype, x, delta, nullptr, 0, A, Bt, Ct, Dskip, z, state, y, stream);
}

int ssm_step_dt(int64_t batch, int64_t D, int64_t N, int dtype,
                const void *x, const void *delta_raw, const float *dt_bias, const float *A,
                const void *Bt, const void *Ct, const float *Dskip,
                const void *z, float *state, void *y, void *stream) {
    return step(batch, D, N, dtype, x, delta_raw, dt_bias, 1, A, Bt, Ct, Dskip, z, state, y, stream);
}

int ssm_step_conv(int64_t batch, int64_t D, int64_t N, int dtype,
                  const void *x_raw, const float *conv_w, const float *conv_b, void *conv_state,
                  const void *delta_raw, const float *dt_bias, const float *A,
                  const void *Bt, const void *Ct, const float *Dskip,
                  const void *z, float *state, void *y, void *stream) {
    if ((!conv_w || !conv_state) && batch > 0 && D > 0) return SSM_ERR_NULL;
    TrapIn tr;
    tr.conv_w = conv_w;
    tr.conv_b = conv_b;
    tr.conv_state = conv_state;
    return step(batch, D, N, dtype, x_raw, delta_raw, dt_bias, 1, A, Bt, Ct, Dskip, z, state, y, stream, tr);
}

int ssm_step_trap(int64_t batch, int64_t D, int64_t N, int dtype,
                  const void *x, const void *delta, const void *lam, const float *A,
                  const void *Bt, const void *Ct, const float *Dskip, const void *z,
                  const void *x_prev, const void *B_prev, float *state, void *y, void *stream) {
    if (!lam && batch > 0 && D > 0) return SSM_ERR_NULL;
    if ((x_prev == nullptr) != (B_prev == nullptr)) return SSM_ERR_NULL;
    TrapIn tr;
    tr.lam = lam;
    tr.x_prev = x_prev;
    tr.B_prev = B_prev;
    return step(batch, D, N, dtype, x, delta, nullptr, 0, A, Bt, Ct, Dskip, z, state, y, stream, tr);
}

// Workspace of the gradient: [header | hst | dsum | gq | pdB | pdC | pdA | pdD | pdT | pdBp | ckp | ckd].
struct BwdLayout {
    int64_t K;
    size_t off[11], bytes;
};

static BwdLayout bwd_layout(int64_t batch, int64_t L, int64_t D, int64_t N) {
    BwdLayout w{};
    w.K = (L + ssm::kBwdChunk - 1) / ssm::kBwdChunk;
    const int64_t nDB = ssm::bwd_channel_blocks(D, N, true);  // the most blocks: the trapezoidal rule
    const size_t sz[11] = {(size_t)(batch * w.K * D * N), (size_t)(batch * w.K * D), (size_t)(batch * w.K * D * N),
                           (size_t)(nDB * batch * L * N), (size_t)(nDB * batch * L * N),
                           (size_t)(batch * w.K * D * N), (size_t)(batch * w.K * D), (size_t)(batch * w.K * D),
                           (size_t)(nDB * batch * N), (size_t)(batch * w.K * ssm::kBwdCk * D * N),
                           (size_t)(batch * w.K * ssm::kBwdCk * D)};
    size_t off = kHeader;
    for (int i = 0; i < 11; ++i) {
        w.off[i] = off;
        off += round_up256(sz[i] * sizeof(float));
    }
    w.bytes = off;
    return w;
}

// Sizes the gradient accepts: every count within kMaxElems and every flat
// grid within 2^32 work-items.
static bool bwd_sizes_ok(int64_t batch, int64_t L, int64_t D, int64_t N) {
    const int64_t K = (L + ssm::kBwdChunk - 1) / ssm::kBwdChunk;
    if (checked_mul3(batch, L, D) < 0 || checked_mul3(batch, L, N) < 0 || checked_mul3(batch, D, N) < 0)
        return false;
    const int64_t nDB = ssm::bwd_channel_blocks(D, N, true);  // the most blocks: the trapezoidal rule
    if (checked_mul3(checked_mul(batch, K), D, N) < 0 || checked_mul3(checked_mul(nDB, batch), L, N) < 0)
        return false;
    const int64_t blocks = checked_mul3(nDB, K, batch);
    // the flat grids of the chunk kernels, the carry (batch * D * N lanes)
    // and the sums of dBt, dCt (batch * L * N lanes), in 256-lane blocks
    const int64_t lanes = checked_mul3(batch, D, N) > checked_mul3(batch, L, N) ? checked_mul3(batch, D, N)
                                                                                : checked_mul3(batch, L, N);
    return blocks >= 0 && blocks < ((int64_t)1 << 24) && lanes / 256 < ((int64_t)1 << 31);
}

size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype) {
    if (batch <= 0 || L <= 0 || D <= 0 || !supported_n(N)) return 0;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return 0;
    if (!bwd_sizes_ok(batch, L, D, N)) return 0;
    return bwd_layout(batch, L, D, N).bytes;
}

// The gradient, for a step size given after its activation (softplus = 0) or
// before it (softplus = 1: delta holds delta_raw, ddelta receives its
// gradient, and ddt_bias, when given, the gradient of dt_bias).
// The trapezoidal rule's extra inputs and outputs.
struct TrapBwd {
    const void *lam = nullptr, *x_prev = nullptr, *B_prev = nullptr;
    void *dlam = nullptr, *dx_prev = nullptr;
    float *dB_prev = nullptr;
};

static int scan_bwd(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                    const void *x, const void *delta, const float *dt_bias, int softplus, const float *A,
                    const void *Bt, const void *Ct, const float *Dskip, const void *z, const float *state_in,
                    const void *dy, const float *dstate,
                    void *dx, void *ddelta, float *ddt_bias, float *dA, float *dBt, float *dCt, float *dDskip,
                    void *dz, float *dstate_in, void *workspace, size_t workspace_bytes, void *stream,
                    TrapBwd tr = {}, bool launch = true) {
    // launch = false: check the arguments only (every check below precedes
    // the first HIP call)
    if (batch < 0 || L < 0 || D < 0 || N < 0) return SSM_ERR_SHAPE;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (!supported_n(N)) return SSM_ERR_UNSUPPORTED;
    if (!bwd_sizes_ok(batch, L, D, N)) return SSM_ERR_SHAPE;
    if (D > 0 && !dA) return SSM_ERR_NULL;
    if (z && !dz) return SSM_ERR_NULL;
    const void *ptrs[] = {x, delta, A, Bt, Ct, Dskip, z, state_in, dy, dstate, dx, ddelta,
                          dA, dBt, dCt, dDskip, dz, dstate_in, workspace, dt_bias, ddt_bias,
                          tr.lam, tr.x_prev, tr.B_prev, tr.dlam, tr.dx_prev, tr.dB_prev};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSM_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (D == 0) return SSM_OK;
    if (batch == 0 || L == 0) {
        if (!launch) return SSM_OK;
        // nothing flows through the tokens: the parameter gradients are zero
        // and the gradient of the entering state is that of the leaving one
        if (ssm::launch_state_copy(nullptr, dA, D * N, s) != hipSuccess) return SSM_ERR_HIP;
        if (Dskip && dDskip && ssm::launch_state_copy(nullptr, dDskip, D, s) != hipSuccess) return SSM_ERR_HIP;
        if (ddt_bias && ssm::launch_state_copy(nullptr, ddt_bias, D, s) != hipSuccess) return SSM_ERR_HIP;

        if (dstate_in && dstate_in != dstate &&
            ssm::launch_state_copy(dstate, dstate_in, batch * D * N, s) != hipSuccess)
            return SSM_ERR_HIP;
        return SSM_OK;
    }
    if (!x || !delta || !A || !Bt || !Ct || !dy || !dx || !ddelta || !dBt || !dCt) return SSM_ERR_NULL;
    if (tr.lam && !tr.dlam) return SSM_ERR_NULL;
    const BwdLayout w = bwd_layout(batch, L, D, N);
    if (!workspace || workspace_bytes < w.bytes) return SSM_ERR_WORKSPACE;
    char *ws = (char *)workspace;
    ssm::BwdArgs a{};
    a.batch = batch;
    a.L = L;
    a.D = D;
    a.K = w.K;
    a.x = x;
    a.delta = delta;
    a.Bt = Bt;
    a.Ct = Ct;
    a.z = z;
    a.dy = dy;
    a.A = A;
    a.Dskip = Dskip;
    a.state_in = state_in;
    a.dstate = dstate;
    a.dx = dx;
    a.ddelta = ddelta;
    a.dz = dz;
    a.dA = dA;
    a.dBt = dBt;
    a.dCt = dCt;
    a.dDskip = Dskip ? dDskip : nullptr;
    a.dstate_in = dstate_in;
    a.dt_bias = dt_bias;
    a.delta_softplus = softplus;
    a.ddt_bias = softplus ? ddt_bias : nullptr;
    a.lam = tr.lam;
    a.x_prev = tr.x_prev;
    a.B_prev = tr.B_prev;
    a.dlam = tr.dlam;
    // the token before the first gets a gradient only when it is given, and
    // both of its outputs are asked for
    const bool prev_grad = tr.x_prev && tr.dx_prev && tr.dB_prev;
    a.dx_prev = prev_grad ? tr.dx_prev : nullptr;
    a.dB_prev = prev_grad ? tr.dB_prev : nullptr;
    a.hst = (float *)(ws + w.off[0]);
    a.dsum = (float *)(ws + w.off[1]);
    a.gq = (float *)(ws + w.off[2]);
    a.pdB = (float *)(ws + w.off[3]);
    a.pdC = (float *)(ws + w.off[4]);
    a.pdA = (float *)(ws + w.off[5]);
    a.pdD = (float *)(ws + w.off[6]);
    a.pdT = (float *)(ws + w.off[7]);
    a.pdBp = (float *)(ws + w.off[8]);
    a.ckp = (float *)(ws + w.off[9]);
    a.ckd = (float *)(ws + w.off[10]);
    if (!launch) return SSM_OK;
    return ssm::launch_scan_bwd(a, (int)N, dtype, s) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_scan_bwd(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                 const void *x, const void *delta, const float *A, const void *Bt, const void *Ct,
                 const float *Dskip, const void *z, const float *state_in,
                 const void *dy, const float *dstate,
                 void *dx, void *ddelta, float *dA, float *dBt, float *dCt, float *dDskip, void *dz,
                 float *dstate_in, void *workspace, size_t workspace_bytes, void *stream) {
    return scan_bwd(batch, L, D, N, dtype, x, delta, nullptr, 0, A, Bt, Ct, Dskip, z, state_in, dy, dstate, dx,
                    ddelta, nullptr, dA, dBt, dCt, dDskip, dz, dstate_in, workspace, workspace_bytes, stream);
}

int ssm_scan_bwd_trap(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                      const void *x, const void *delta, const void *lam, const float *A,
                      const void *Bt, const void *Ct, const float *Dskip, const void *z,
                      const void *x_prev, const void *B_prev, const float *state_in,
                      const void *dy, const float *dstate,
                      void *dx, void *ddelta, void *dlam, float *dA, float *dBt, float *dCt, float *dDskip, void *dz,
                      void *dx_prev, float *dB_prev, float *dstate_in, void *workspace, size_t workspace_bytes,
                      void *stream) {
    if (!lam && batch > 0 && L > 0 && D > 0) return SSM_ERR_NULL;
    if ((x_prev == nullptr) != (B_prev == nullptr)) return SSM_ERR_NULL;
    if ((dx_prev == nullptr) != (dB_prev == nullptr)) return SSM_ERR_NULL;
    TrapBwd tr;
    tr.lam = lam;
    tr.x_prev = x_prev;
    tr.B_prev = B_prev;
    tr.dlam = dlam;
    tr.dx_prev = dx_prev;
    tr.dB_prev = dB_prev;
    return scan_bwd(batch, L, D, N, dtype, x, delta, nullptr, 0, A, Bt, Ct, Dskip, z, state_in, dy, dstate, dx,
                    ddelta, nullptr, dA, dBt, dCt, dDskip, dz, dstate_in, workspace, workspace_bytes, stream, tr);
}

// Workspace of the gradient through the x branch: the scan gradient's, then
// the branch's output and its gradient (activation dtype) and the partial
// sums of the taps' and bias' gradients.
struct ConvBwdLayout {
    int64_t chunk, nchunk;
    size_t bwd, off_xc, off_gx, off_part, bytes;
};

static ConvBwdLayout conv_bwd_layout(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype) {
    ConvBwdLayout w{};
    ssm::conv_bwd_plan(batch, L, D, &w.chunk, &w.nchunk);
    w.bwd = bwd_layout(batch, L, D, N).bytes;
    const size_t act = (size_t)(batch * L * D) * (dtype == SSM_BF16 ? 2 : 4);
    w.off_xc = w.bwd;
    w.off_gx = w.off_xc + round_up256(act);
    w.off_part = w.off_gx + round_up256(act);
    w.bytes = w.off_part + round_up256((size_t)(batch * w.nchunk * D * 5) * sizeof(float));
    return w;
}

size_t ssm_scan_bwd_conv_workspace_bytes(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype) {
    if (batch <= 0 || L <= 0 || D <= 0 || !supported_n(N)) return 0;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return 0;
    if (!bwd_sizes_ok(batch, L, D, N)) return 0;
    return conv_bwd_layout(batch, L, D, N, dtype).bytes;
}

int ssm_scan_bwd_conv(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                      const void *x_raw, const float *conv_w, const float *conv_b, const void *conv_state,
                      const void *delta_raw, const float *dt_bias, const float *A,
                      const void *Bt, const void *Ct, const float *Dskip, const void *z, const float *state_in,
                      const void *dy, const float *dstate,
                      void *dx_raw, float *dconv_w, float *dconv_b, void *dconv_state,
                      void *ddelta_raw, float *ddt_bias, float *dA, float *dBt, float *dCt,
                      float *dDskip, void *dz, float *dstate_in, void *workspace, size_t workspace_bytes,
                      void *stream) {
    if (batch < 0 || L < 0 || D < 0 || N < 0) return SSM_ERR_SHAPE;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (!supported_n(N)) return SSM_ERR_UNSUPPORTED;
    if (!bwd_sizes_ok(batch, L, D, N)) return SSM_ERR_SHAPE;
    if (D > 0 && (!conv_w || !dconv_w)) return SSM_ERR_NULL;
    const void *ptrs[] = {conv_w, conv_b, conv_state, dconv_w, dconv_b, dconv_state};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSM_ERR_ALIGN;
    const bool tokens = batch > 0 && L > 0 && D > 0;
    if (tokens && (!x_raw || !dx_raw)) return SSM_ERR_NULL;
    if (x_raw && !aligned16(x_raw)) return SSM_ERR_ALIGN;
    if (dx_raw && !aligned16(dx_raw)) return SSM_ERR_ALIGN;
    const ConvBwdLayout w = tokens ? conv_bwd_layout(batch, L, D, N, dtype) : ConvBwdLayout{};
    if (tokens && (!workspace || workspace_bytes < w.bytes)) return SSM_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return SSM_ERR_ALIGN;
    char *ws = (char *)workspace;
    ssm::ConvBwdArgs c{};
    c.batch = batch;
    c.L = L;
    c.D = D;
    c.chunk = w.chunk;
    c.nchunk = w.nchunk;
    c.x_raw = x_raw;
    c.conv_state = conv_state;
    c.conv_w = conv_w;
    c.conv_b = conv_b;
    c.xc = tokens ? ws + w.off_xc : nullptr;
    c.gx = tokens ? ws + w.off_gx : nullptr;
    c.dx_raw = dx_raw;
    c.dconv_state = dconv_state;
    c.dconv_w = dconv_w;
    c.dconv_b = conv_b ? dconv_b : nullptr;
    c.part = tokens ? (float *)(ws + w.off_part) : nullptr;
    hipStream_t s = (hipStream_t)stream;
    // check the scan gradient's own arguments before launching anything: the
    // branch's output stands in for x (any aligned address passes the checks)
    const int chk = scan_bwd(batch, L, D, N, dtype, tokens ? c.xc : x_raw, delta_raw, dt_bias, 1, A, Bt, Ct, Dskip,
                             z, state_in, dy, dstate, tokens ? ws + w.off_gx : dx_raw, ddelta_raw, ddt_bias, dA,
                             dBt, dCt, dDskip, dz, dstate_in, workspace, tokens ? w.bwd : workspace_bytes, stream,
                             TrapBwd{}, /*launch=*/false);
    if (chk != SSM_OK) return chk;
    if (D == 0) return SSM_OK;
    if (ssm::launch_conv_fwd(c, dtype, s) != hipSuccess) return SSM_ERR_HIP;
    const int rc = scan_bwd(batch, L, D, N, dtype, tokens ? c.xc : x_raw, delta_raw, dt_bias, 1, A, Bt, Ct, Dskip,
                            z, state_in, dy, dstate, tokens ? ws + w.off_gx : dx_raw, ddelta_raw, ddt_bias, dA, dBt,
                            dCt, dDskip, dz, dstate_in, workspace, tokens ? w.bwd : workspace_bytes, stream);
    if (rc != SSM_OK) return rc;
    return ssm::launch_conv_bwd(c, dtype, s) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_scan_bwd_dt(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                    const void *x, const void *delta_raw, const float *dt_bias, const float *A,
                    const void *Bt, const void *Ct, const float *Dskip, const void *z, const float *state_in,
                    const void *dy, const float *dstate,
                    void *dx, void *ddelta_raw, float *ddt_bias, float *dA, float *dBt, float *dCt,
                    float *dDskip, void *dz, float *dstate_in, void *workspace, size_t workspace_bytes,
                    void *stream) {
    return scan_bwd(batch, L, D, N, dtype, x, delta_raw, dt_bias, 1, A, Bt, Ct, Dskip, z, state_in, dy, dstate,
                    dx, ddelta_raw, ddt_bias, dA, dBt, dCt, dDskip, dz, dstate_in, workspace, workspace_bytes,
                    stream);
}

int ssm_ssd_step(int64_t batch, int64_t H, int64_t P, int64_t G, int64_t N, int dtype,
                 const void *x, const void *delta, const float *A, const void *Bt, const void *Ct,
                 const float *Dskip, float *state, void *y, void *stream) {
    if (batch < 0 || H < 0 || P < 0 || G < 0 || N < 0) return SSM_ERR_SHAPE;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (!ssm::ssd_step_supported(P, N)) return SSM_ERR_UNSUPPORTED;
    if (H > 0 && (G < 1 || H % G != 0)) return SSM_ERR_SHAPE;
    if (checked_mul3(checked_mul(batch, H), P, N) < 0 || checked_mul3(batch, G, N) < 0 ||
        checked_mul(batch, H) >= ((int64_t)1 << 31))
        return SSM_ERR_SHAPE;
    if (batch == 0 || H == 0) return SSM_OK;
    if (!x || !delta || !A || !Bt || !Ct || !state || !y) return SSM_ERR_NULL;
    const void *ptrs[] = {x, delta, A, Bt, Ct, Dskip, state, y};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSM_ERR_ALIGN;
    ssm::SsdStepArgs a{};
    a.batch = batch;
    a.H = H;
    a.G = G;
    a.x = x;
    a.delta = delta;
    a.Bt = Bt;
    a.Ct = Ct;
    a.A = A;
    a.Dskip = Dskip;
    a.state = state;
    a.y = y;
    return ssm::launch_ssd_step(a, (int)N, dtype, (hipStream_t)stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_ssd_fwd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int dtype,
                const void *x, const void *delta, const float *A, const void *Bt, const void *Ct,
                const float *Dskip, const float *state_in, float *state_out, void *y, void *stream) {
    if (batch < 0 || L < 0 || H < 0 || P < 0 || G < 0 || N < 0) return SSM_ERR_SHAPE;
    if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (dtype != SSM_BF16 || !ssm::ssd_supported(P, N)) return SSM_ERR_UNSUPPORTED;
    if (H > 0 && (G < 1 || H % G != 0)) return SSM_ERR_SHAPE;
    // 64 tokens of x and of Bt, Ct must span less than 4 GiB (32-bit offsets)
    if (H > ((int64_t)UINT32_MAX / (64 * 2 * 64)) || G * N > ((int64_t)UINT32_MAX / (2 * 64)))
        return SSM_ERR_UNSUPPORTED;
    if (checked_mul3(batch, L, H) < 0 || checked_mul3(checked_mul(batch, L), H, P) < 0 ||
        checked_mul3(checked_mul(batch, L), G, N) < 0 || checked_mul3(checked_mul(batch, H), P, N) < 0)
        return SSM_ERR_SHAPE;
    if (batch == 0 || H == 0) return SSM_OK;
    hipStream_t s = (hipStream_t)stream;
    if (L == 0) {
        if (!state_out) return SSM_OK;
        if (!aligned16(state_out) || (state_in && !aligned16(state_in))) return SSM_ERR_ALIGN;
        if (state_in == state_out) return SSM_OK;
        return ssm::launch_state_copy(state_in, state_out, batch * H * P * N, s) == hipSuccess ? SSM_OK
                                                                                              : SSM_ERR_HIP;
    }
    if (!x || !delta || !A || !Bt || !Ct || !y) return SSM_ERR_NULL;
    const void *ptrs[] = {x, delta, A, Bt, Ct, Dskip, state_in, state_out, y};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return SSM_ERR_ALIGN;
    ssm::SsdArgs a{};
    a.batch = batch;
    a.L = L;
    a.H = H;
    a.G = G;
    a.x = x;
    a.delta = delta;
    a.Bt = Bt;
    a.Ct = Ct;
    a.A = A;
    a.Dskip = Dskip;
    a.state_in = state_in;
    a.state_out = state_out;
    a.y = y;
    return ssm::launch_ssd(a, (int)N, s) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"

namespace ssm {

int scan_fwd_euler(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype, const void *x, const void *delta,
                   const float *A, const void *Bt, const void *Ct, const float *Dskip, const void *z,
                   const float *state_in, float *state_out, void *y, void *workspace, size_t workspace_bytes,
                   void *stream, bool launch) {
    return scan_fwd(batch, L, D, N, dtype, x, delta, nullptr, 0, A, Bt, Ct, Dskip, z, state_in, state_out, y,
                    workspace, workspace_bytes, stream, TrapIn{}, launch);
}

}  // namespace ssm
