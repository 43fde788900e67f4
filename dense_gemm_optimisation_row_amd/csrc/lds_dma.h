// Device helpers shared by the kernels that move tiles straight from global
// memory into LDS with buffer_load ... lds (gfx950).  Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgor {

typedef int intx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Buffer descriptor over [base, base + bytes): loads past the end read as
// zero, stores past it are dropped (bytes <= 0 gives an empty range).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, long long bytes)
{
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// The four words of the same raw buffer descriptor, for use as an
// inline-assembly operand (word 2 is the range in bytes).
__device__ __forceinline__ intx4 rsrc_words(const void *base, long long bytes)
{
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
    intx4 d;
    d.x = (int)(uint32_t)p;
    d.y = (int)((uint32_t)(p >> 32) & 0xffffu);
    d.z = n;
    d.w = 0x00020000;
    return d;
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void *p)
{
    return (uint32_t)(uintptr_t)(lds_void *)p;
}

// LDS poison (debug builds compiled with -DDGOR_LDS_POISON only): right
// before a global->LDS load is issued into a region, this wavefront fills the
// bytes the load will write with all-ones (a NaN in FP32, FP16, BF16 and both
// FP8 formats; -1 in INT8) and waits for those writes.  The load is issued
// only once the barrier that retires the region's last reads has passed, so
// a correct kernel never reads the poison: a read that runs ahead of that
// barrier, or of the wait for the load, returns the poison and corrupts C.
#ifdef DGOR_LDS_POISON
__device__ __forceinline__ void poison_lds(uint32_t lds, uint32_t bytes_per_lane)
{
    typedef __attribute__((address_space(3))) uint32_t lds_u32;
    lds_u32 *p = (lds_u32 *)(uintptr_t)(lds + bytes_per_lane * (threadIdx.x & 63));
    for (uint32_t i = 0; i < bytes_per_lane / 4; ++i)
        p[i] = 0xffffffffu;
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the writes have landed
}
#endif

// One global->LDS load of 64 x 16 bytes: lane p reads 16 bytes at byte offset
// voff of the descriptor's range (zeros when out of range) and writes them to
// LDS address lds + 16 p.  M0 carries the LDS address; one wait state
// separates its write from the load that reads it.  A kernel that uses this
// must keep nothing of its own in M0 (the compiler emits no M0 access in
// such a kernel, which a test checks on the generated code), so M0 is not
// restored.  The load is not tracked by the compiler's wait counters: the
// caller waits for it with vmcnt.
__device__ __forceinline__ void load_to_lds(intx4 rsrc, uint32_t lds, uint32_t voff)
{
#ifdef DGOR_LDS_POISON
    poison_lds(lds, 16);
#endif
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory");
}

// The same with 4 bytes per lane: lane p reads the dword at byte offset voff
// and writes it to LDS address lds + 4 p (a 256-byte run per load).
__device__ __forceinline__ void load_dword_to_lds(intx4 rsrc, uint32_t lds, uint32_t voff)
{
#ifdef DGOR_LDS_POISON
    poison_lds(lds, 4);
#endif
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory");
}

// s_waitcnt immediate (gfx9 encoding) for vmcnt(n) alone: vmcnt bits 3:0 and
// 15:14, expcnt (6:4) and lgkmcnt (11:8) left at their maximum.
constexpr int wait_vmcnt(int n)
{
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}
// The same with lgkmcnt(0): this wavefront's LDS reads have also returned.
constexpr int wait_vmcnt_lgkm0(int n)
{
    return (n & 15) | ((n >> 4) << 14) | (7 << 4);
}

static_assert(wait_vmcnt_lgkm0(16) == 0x4070, "vmcnt/lgkmcnt encoding");
static_assert(wait_vmcnt(0) == 0x0f70 && wait_vmcnt(8) == 0x0f78 && wait_vmcnt(24) == 0x4f78,
              "vmcnt encoding");

}  // namespace dgor
