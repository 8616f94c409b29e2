// lds_dma.hpp -- copy helpers shared by the GEMM kernels on gfx950: DMA
// copies global -> LDS (global_load_lds), an explicit vector-memory wait, and
// the 16-byte piece swizzle of 128-byte LDS rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oproj {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// LDS byte offset of a __shared__ address, made wave-uniform (an SGPR).
__device__ __forceinline__ uint32_t lds_offset(const uint8_t* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u8*)p);
}

// DMA copies global -> LDS (global_load_lds): lane i's 16 (or 4) bytes land
// at lds + 16*i (4*i); `lds` is made wave-uniform and goes to M0.  Written as
// asm: the compiler cannot tell these LDS writes from the ring slots being
// read and would otherwise wait for every copy before each LDS read; all
// waits for the copies are explicit (wait_vmcnt).  Nothing else in the
// kernels that use them keeps a value in M0.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most min(ahead, N) pipeline steps of this wave's copies are
// still in flight, PER copy instructions per step (ahead < 0 counts as 0):
// the step being waited for is followed by `ahead` issued steps.
template <int N, int PER>
__device__ __forceinline__ void wait_ahead(int64_t ahead) {
    if constexpr (N <= 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= N)
            wait_vmcnt<PER * N>();
        else
            wait_ahead<N - 1, PER>(ahead);
    }
}

// 16-byte piece swizzle of a 128-byte LDS row.  A fragment read (ds_read_b128)
// has the lanes of 16 consecutive rows fetch the same piece; XOR with
// (row & 7) ^ ((row >> 3) & 1) puts any 8 consecutive rows on 8 different
// pieces and any 16 consecutive rows on 16 different (row parity, piece)
// bank groups, so the reads are conflict-free whether the LDS serves 8 lanes
// over 32 banks or 16 lanes over 64 banks per cycle.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// DMA copy with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (no per-copy vector address arithmetic).  The base is passed
// through readfirstlane so it always lands in scalar registers.
__device__ __forceinline__ uint64_t uniform64(const void* p) {
    const uint64_t v = reinterpret_cast<uintptr_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(uniform64(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}
// Same copy with the non-temporal hint, for data read exactly once (the
// weight stream of the decode kernel).
__device__ __forceinline__ void dma16s_nt(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(uniform64(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(uniform64(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

}  // namespace oproj
