// Direct global-to-LDS loads on gfx950 and the waits around them, shared by
// the warp-specialised product kernels: producer waves stream a kernel's
// operands into an LDS ring, math waves read them from LDS.
//
// global_load_lds_dwordx4 writes 16 bytes per lane to LDS at M0 + 16 lane
// (64 lanes fill 1 KB), counts on the wave's vector-memory counter, and does
// not pass through registers, so it does not compete with the math waves'
// LDS reads the way ds_write stores do.  A producer wave publishes a stage by
// waiting on its own counter and then reaching the block barrier; the barrier
// it uses carries no memory fence (a fence would make the wave drain every
// load still in flight).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// s_waitcnt operand: at most v vector-memory operations outstanding, the
// other counters left free.
constexpr unsigned dl_vmcnt(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr unsigned DL_LGKM0 = 15 | (3 << 14) | (7 << 4);   // lgkmcnt(0) only

typedef __attribute__((address_space(3))) void dl_lds_void_t;

// 16 bytes per lane from src into LDS at dst + 16 * lane (dst the same for
// the whole wave).
__device__ inline void dl_load16(const void *src, uint8_t *dst)
{
    __builtin_amdgcn_global_load_lds(src, (dl_lds_void_t *)dst, 16, 0, 0);
}

// Block barrier without a fence; the compiler may not move memory accesses
// across it.
__device__ inline void dl_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace bl
