// Device building blocks of the gfx950 scan kernels: DPP broadcasts within a
// 16-lane row, permlane swaps, global-to-LDS loads the compiler does not
// track, LDS-only barriers, and epoch-tagged words for hand-offs between
// workgroups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ssm {

constexpr long kSpinLimit = 1L << 22;  // polls before a cross-workgroup wait gives up (a few seconds)

template <int SRC>
__device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + SRC, 0xF, 0xF, true));
}

// acc = sum over j < NL of (lane S0+j of the row's `c`) * h[j]: one
// v_mul_f32 and NL-1 v_fmac_f32, all with DPP sources, behind one pair of wait
// states (only `c` is read through DPP, so the NL instructions share them;
// h[j] are plain operands).
template <int NL, int S0>
__device__ __forceinline__ void dot_row(float &acc, float c, const float (&h)[NL]) {
    if constexpr (NL == 4) {
        asm volatile("s_nop 1"
                     "\n\tv_mul_f32_dpp %0, %1, %2 row_newbcast:%6 row_mask:0xf bank_mask:0xf"
                     "\n\tv_fmac_f32_dpp %0, %1, %3 row_newbcast:%7 row_mask:0xf bank_mask:0xf"
                     "\n\tv_fmac_f32_dpp %0, %1, %4 row_newbcast:%8 row_mask:0xf bank_mask:0xf"
                     "\n\tv_fmac_f32_dpp %0, %1, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf"
                     : "=&v"(acc)
                     : "v"(c), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "i"(S0), "i"(S0 + 1), "i"(S0 + 2),
                       "i"(S0 + 3));
    } else if constexpr (NL == 2) {
        asm volatile("s_nop 1"
                     "\n\tv_mul_f32_dpp %0, %1, %2 row_newbcast:%4 row_mask:0xf bank_mask:0xf"
                     "\n\tv_fmac_f32_dpp %0, %1, %3 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
                     : "=&v"(acc)
                     : "v"(c), "v"(h[0]), "v"(h[1]), "i"(S0), "i"(S0 + 1));
    } else {
        static_assert(NL == 1, "1, 2 or 4 states per lane");
        asm volatile("s_nop 1\n\tv_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                     : "=&v"(acc)
                     : "v"(c), "v"(h[0]), "i"(S0));
    }
}

// v_permlane32_swap: lanes 32-63 of a trade places with lanes 0-31 of b, so
// a = [a.lo, b.lo] and b = [a.hi, b.hi]. v_permlane16_swap: the odd rows of a
// trade places with the even rows of b. Written as inline assembly (with the
// two wait states a VALU-written source needs) because the compiler builtin
// returns both results in one register when they feed the same add.
__device__ __forceinline__ void swap_halves(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_odd_even_rows(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

template <int I, int END, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < END) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, END>(f);
    }
}

__device__ __forceinline__ uint32_t ld_flag(const uint32_t *p) {
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged(uint64_t *p, float v, uint32_t epoch) {
    __hip_atomic_store(p, ((uint64_t)epoch << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A tagged word loaded earlier: if it is not yet this call's, load it again
// until it is (its writer has already published the first word of the same
// record, so this is short) or the spin limit is reached.
__device__ __forceinline__ uint64_t recheck(uint64_t v, const uint64_t *p, uint32_t epoch) {
    for (long sp = 0; (uint32_t)(v >> 32) != epoch && sp < kSpinLimit; ++sp) v = ld_tagged(p);
    return v;
}
__device__ __forceinline__ uint64_t ld_valid(const uint64_t *p, uint32_t epoch) {
    return recheck(ld_tagged(p), p, epoch);
}

// LDS address of a __shared__ location, made wave-uniform. A generic
// pointer into the LDS aperture carries the LDS address in its low 32 bits.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// One 16-byte piece per lane from global memory straight into LDS at
// lds + lane*16 (global_load_lds_dwordx4; lds is wave-uniform). Written as
// inline assembly so that the compiler does not count these loads: it would
// otherwise wait for all of them before LDS reads and barriers that have
// nothing to do with them, which serialises the prefetch of the next tile
// with the scan of the current one. No registers receive data; the caller
// waits with vm_wait() before the data is read.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory");
}
// The same with a wave-uniform base address (SGPRs) and a per-lane 32-bit
// byte offset: no per-lane address arithmetic.
__device__ __forceinline__ void dma16_s(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                 : "memory");
}
// Wait until this wave's vector memory accesses (including the loads above)
// have completed.
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier that orders LDS accesses only. __syncthreads() would also
// wait for every global access the wave has in flight, which includes the
// next tile's loads into LDS; those are meant to stay in flight across the
// barriers of the current tile.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace ssm
