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
    float *state_out;
    void *y;
    float *ws_state;   // (batch, K, D, N) chunk end states, then carried-in states
    float *ws_dsum;    // (batch, K, D)    summed delta per chunk
    int64_t K;         // number of sequence chunks
    int64_t Lc;        // tokens per chunk (the last chunk may be shorter)
};

struct StepArgs {
    int64_t batch, D;
    const void *x, *delta, *Bt, *Ct, *z;
    const float *A, *Dskip;
    float *state;
    void *y;
};

// Sequence split used for a scan of these sizes (deterministic).
void scan_plan(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t *K, int64_t *Lc);

// Launchers; return hipSuccess or the launch error.
hipError_t launch_scan(const ScanArgs &a, int N, int dtype, hipStream_t s);
hipError_t launch_state_copy(const float *src, float *dst, int64_t n, hipStream_t s);
hipError_t launch_step(const StepArgs &a, int N, int dtype, hipStream_t s);

}  // namespace ssm
