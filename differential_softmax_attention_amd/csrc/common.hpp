// Device-side helpers shared by the libdiffattn kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Value held by lane (lane ^ mask), through the LDS crossbar. `addr` = (lane ^ mask) * 4.
__device__ __forceinline__ float lane_xor(float x, int addr) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(x)));
}

// x of a partner lane inside the lane's 16-lane row, by DPP (CTRL: 0xB1 lane ^ 1, 0x4E lane ^ 2,
// 0x141 lane 7 - i within 8, 0x140 lane 15 - i within 16)
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// x combined with x of lane ^ 16 and with x of lane ^ 32 (the gfx950 row swaps)
template <class F>
__device__ __forceinline__ float combine_rows(float x, F op) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Reductions over all 64 lanes of a wave: pairs, quads, the mirrored halves of 8 and of 16 lanes
// by DPP, then across rows. Each step combines two lanes that are also combined with each other
// (the operation commutes), so every lane ends with the same value.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_partner<0xB1>(x));
    x = fmaxf(x, dpp_partner<0x4E>(x));
    x = fmaxf(x, dpp_partner<0x141>(x));
    x = fmaxf(x, dpp_partner<0x140>(x));
    return combine_rows(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_partner<0xB1>(x);
    x += dpp_partner<0x4E>(x);
    x += dpp_partner<0x141>(x);
    x += dpp_partner<0x140>(x);
    return combine_rows(x, [](float a, float b) { return a + b; });
}

// 1 / (1 + e^-z): DIFF V2's per-token lambda from its projected logit. Saturates to 0 and 1 for
// large |z| (e^-z overflowing to +inf gives 0).
__device__ __forceinline__ float sigmoid_f32(float z) { return 1.f / (1.f + __expf(-z)); }

// 2^x on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// gfx950 transposing LDS read: within each group of 16 lanes, lane L supplies the address of
// four consecutive 16-bit elements (row L of a 16x4 block M); lane i receives
// M[4j + i/4][i%4] for j = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const bf16* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

}  // namespace diffattn
