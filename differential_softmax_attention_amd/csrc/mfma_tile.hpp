// Tile staging and lane-exchange helpers shared by the MFMA forward kernels (gfx950).
//
// LDS tiles are unpadded rows of 16-byte chunks, XOR-swizzled per row so that the MFMA operand
// reads hit distinct banks, and are filled by global_load_lds (16 bytes per lane, lane i of a
// wave writing base + 16 i): each lane fetches the global chunk that belongs in its LDS slot, so
// no registers stage the tile.
//  K, d = 64  (8 chunks per row):  phys = c ^ ((row & 7) ^ ((row >> 3) & 1))
//  K, d = 128 (16 chunks per row): phys = c ^ (row & 15)
//  V, 128 wide (16 chunks per row): phys = c ^ ((row & 3) << 1) ^ ((c & 2) << 2)
#pragma once
#include "common.hpp"

namespace diffattn {

typedef __attribute__((address_space(3))) unsigned char lds_u8_t;

template <int D>
__device__ __forceinline__ int k_swz(int row) {
    return D == 64 ? ((row & 7) ^ ((row >> 3) & 1)) : (row & 15);
}
__device__ __forceinline__ int v_phys(int row, int c) { return c ^ ((row & 3) << 1) ^ ((c & 2) << 2); }
__device__ __forceinline__ int v_logical(int row, int p) {
    const int y = p ^ ((row & 3) << 1);
    return y ^ ((y & 2) << 2);
}

// s_waitcnt immediates for vmcnt(n), n < 16, with the other counters left unconstrained
constexpr unsigned kVmcnt[16] = {0x0F70, 0x0F71, 0x0F72, 0x0F73, 0x0F74, 0x0F75, 0x0F76, 0x0F77,
                                 0x0F78, 0x0F79, 0x0F7A, 0x0F7B, 0x0F7C, 0x0F7D, 0x0F7E, 0x0F7F};

// 16-byte global -> LDS DMA for one wave: lane i reads sbase + voff (voff per lane) and the
// chunk lands at LDS address lds_wave_base + 16 i. Issued from inline asm so that the compiler
// does not track it as an LDS store: its generic tracking would otherwise wait for the next
// tile's prefetch before every read of the current tile. Completion is ordered explicitly:
// s_waitcnt vmcnt and a barrier before a stage is read. The LDS base travels in M0, which the
// asm takes as an input operand so that the compiler knows the register is written. The compiler
// does not see the memory instruction inside the asm either, so it does not insert the five wait
// states that a vector memory read of an SGPR needs after a VALU instruction (such as the
// v_readfirstlane below) wrote it: the asm carries them itself (s_nop 4). Without them a schedule
// that puts the readfirstlane right before the load reads a stale base address.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_wave_base) {
    // the tile base is wave-uniform: pin it to SGPRs (readfirstlane returns int, so each word is
    // widened through uint32_t and the low word is not sign-extended)
    const uint64_t p = (uint64_t)(uintptr_t)sbase;
    const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                 : : "v"(voff), "s"((const void*)(uintptr_t)u), "{m0}"(lds_wave_base) : "memory");
}

// 4-byte variant: lane i reads sbase + voff and the word lands at lds_wave_base + 4 i
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_wave_base) {
    const uint64_t p = (uint64_t)(uintptr_t)sbase;
    const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1"
                 : : "v"(voff), "s"((const void*)(uintptr_t)u), "{m0}"(lds_wave_base) : "memory");
}

// maximum that ignores NaN-quieting (v_maximum3 / v_max without canonicalisation)
__device__ __forceinline__ float fmax_nc(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ bf16x8 lds16(const unsigned char* p) { return *(const bf16x8*)p; }
__device__ __forceinline__ bf16x8 ld_global_bf16x8(const bf16* p) { return *(const bf16x8*)p; }

// x combined with the value of x held by lane l ^ 32: both halves of the wave get the result
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmax_nc(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace diffattn
