// Issue-rate calibration for the VALU roofline the scan kernels are measured
// against (libssm_calib.so; a measuring aid, not part of the libssm ABI).
//
// Every thread runs 8 independent dependency chains for `iters` steps, so that
// a wave always has independent work to issue, at an occupancy set by the
// launch. One chain step is
//   op 0: y = exp2(-y)                  (one v_exp_f32; converges to ~0.641)
//   op 1: y = fma(y, a, c)              (one v_fmac_f32)
//   op 2: four fmas then one exp2       (the mix of the scan's state update:
//                                        per element one exponential and four
//                                        multiplies / multiply-adds)
// The host times the launch with events and divides the lane instructions by
// the time. The last value of every chain is written out, so nothing is
// optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int OP>
__global__ __launch_bounds__(256) void valu_rate_kernel(float *out, int iters, float a, float c) {
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = 0.25f + 0.01f * (float)(threadIdx.x & 7) + 0.003f * (float)k;
#pragma unroll 4
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if constexpr (OP == 0) {
                y[k] = __builtin_amdgcn_exp2f(-y[k]);
            } else if constexpr (OP == 1) {
                y[k] = __builtin_fmaf(y[k], a, c);
            } else {
                y[k] = __builtin_fmaf(y[k], a, c);
                y[k] = __builtin_fmaf(y[k], a, c);
                y[k] = __builtin_fmaf(y[k], a, c);
                y[k] = __builtin_fmaf(y[k], a, c);
                y[k] = __builtin_amdgcn_exp2f(-y[k]);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += y[k];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// Launch `blocks` workgroups of 256 threads of chain kind `op` (0, 1, 2) for
// `iters` steps on `stream`; `out` holds blocks * 256 floats. Returns 0, or -1
// for a bad argument, -7 for a failed launch.
extern "C" int ssm_calib_valu_rate(int op, int blocks, int iters, float *out, void *stream) {
    if (blocks < 1 || iters < 1 || !out || op < 0 || op > 2) return -1;
    hipStream_t s = (hipStream_t)stream;
    const float a = 0.999f, c = 0.001f;
    if (op == 0) hipLaunchKernelGGL(valu_rate_kernel<0>, dim3(blocks), dim3(256), 0, s, out, iters, a, c);
    else if (op == 1) hipLaunchKernelGGL(valu_rate_kernel<1>, dim3(blocks), dim3(256), 0, s, out, iters, a, c);
    else hipLaunchKernelGGL(valu_rate_kernel<2>, dim3(blocks), dim3(256), 0, s, out, iters, a, c);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}
