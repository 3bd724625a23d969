// lds_dma.h -- direct global->LDS loads (global_load_lds_dword[x4]) and the
// vector-memory wait that tracks them, shared by every kernel that stages tiles
// this way (attention, GLA, projection).
//
// Each load moves 16 (or 4) bytes per active lane from global memory straight
// into LDS at base + 16 * lane (4 * lane), with base wave-uniform (held in m0).
// The loads are written as asm so that the compiler does not serialise them
// against LDS reads of another buffer (it cannot tell the buffers apart); they
// have no register outputs, and completion is tracked by wait_vmcnt.
#pragma once

#include "device_common.h"

namespace hta {

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima). Vector
// memory operations of a wave complete in issue order for this counter, so
// N > 0 waits for everything but the newest N.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 0x3) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    typedef __attribute__((address_space(3))) const char lds_char;
    return (uint32_t)(uintptr_t)(lds_char*)p;
}

// 16 bytes from sbase + voff (sbase wave-uniform, voff per lane) into LDS at
// lds + 16 * lane (lds wave-uniform).
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
    // readfirstlane pins the uniform bases to SGPRs for the asm operands
    // (it returns int: widen each half as uint32_t, never sign-extended)
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
    const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(ls), "v"(voff), "s"(sb)
                 : "m0");
}

// The same with 4 bytes per lane: LDS at lds + 4 * lane.
__device__ __forceinline__ void dma4(uint32_t voff, const void* sbase, uint32_t lds) {
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
    const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(ls), "v"(voff), "s"(sb)
                 : "m0");
}

// Per-lane global address forms: 16 (4) bytes from gptr into LDS at
// lds_base + 16 * lane (4 * lane); lds_base wave-uniform.
__device__ __forceinline__ void dma16p(const void* gptr, const void* lds_base) {
    const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_u32(lds_base));
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds), "v"(gptr) : "m0");
}
__device__ __forceinline__ void dma4p(const void* gptr, const void* lds_base) {
    const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_u32(lds_base));
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" : : "s"(lds), "v"(gptr) : "m0");
}

}  // namespace hta
