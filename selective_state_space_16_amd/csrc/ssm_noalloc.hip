// ssm_scan_fwd_noalloc: the selective scan with its workspace in a static
// device array of this library instead of a buffer the caller brings, for
// callers that cannot allocate device memory at all.
//
// The scan's workspace holds the unit counters, the tag of the last finished
// call and, when sequences are cut into stripes, each stripe's records. Its
// size is bounded for every shape the stripe scan takes: the planner cuts at
// most 64 stripe-columns per unit list, so there are at most 8 x 64 x 4
// records of 64 lanes x (2 NL + 1) 8-byte words (NL <= 4), 9.0 MiB with the
// header. The array below holds that with room for small chunked-scan
// workspaces; a shape that needs more is refused with SSM_ERR_WORKSPACE.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/ssm.h"
#include "ssm_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)12 << 20;

// One copy per device, kept until the process ends. In host code this name
// only stands for the symbol: the device address comes from
// hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

__global__ void zero_fill(uint4 *p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's copy of the array, found (and cleared, on `s`) the
// first time a call runs on that device.
hipError_t scratch_for_current_device(hipStream_t s, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [&] {
        void *p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (g_err[dev] != hipSuccess) return;
        // the workspace must start at zero; a fill kernel rather than a
        // memset, so that the clearing may also be recorded into a graph
        hipLaunchKernelGGL(zero_fill, dim3(256), dim3(256), 0, s, (uint4 *)p, kScratchBytes / sizeof(uint4));
        g_err[dev] = hipGetLastError();
        if (g_err[dev] == hipSuccess) g_ptr[dev] = p;
    });
    if (g_err[dev] != hipSuccess) return g_err[dev];
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int ssm_scan_fwd_noalloc(int64_t batch, int64_t L, int64_t D, int64_t N, int dtype,
                                    const void *x, const void *delta, const float *A,
                                    const void *Bt, const void *Ct, const float *Dskip,
                                    const void *z, const float *state_in, float *state_out,
                                    void *y, void *stream) {
    // Every check first, against the array's size (an aligned stand-in
    // address: nothing is launched), then the array itself.
    const int st = ssm::scan_fwd_euler(batch, L, D, N, dtype, x, delta, A, Bt, Ct, Dskip, z, state_in, state_out,
                                       y, (void *)(uintptr_t)256, kScratchBytes, stream, false);
    if (st != SSM_OK) return st;
    void *ws = nullptr;
    if (ssm_scan_workspace_bytes(batch, L, D, N, dtype) > 0 &&
        scratch_for_current_device((hipStream_t)stream, &ws) != hipSuccess)
        return SSM_ERR_HIP;
    return ssm::scan_fwd_euler(batch, L, D, N, dtype, x, delta, A, Bt, Ct, Dskip, z, state_in, state_out, y, ws,
                               ws ? kScratchBytes : 0, stream, true);
}
