// LDS layouts and MFMA helpers shared by the backward kernels (gfx950).
//
// Backward tiles are 32 rows of 64 or 128 bf16 and are read two ways: by rows (16-byte reads, the
// MFMA A rows or B columns of S = Q K^T and dP = go V^T) and transposed (ds_read_b64_tr_b16, the
// X^T operands of dK = dS^T Q, dQ = dS K and dV = P^T go). Their 16-byte chunk swizzles put both
// read patterns on distinct banks:
//   64 wide  (8 chunks per row):  chunk c of row r at c ^ (4 ((r >> 1) & 1) | ((r >> 2) & 3))
//   128 wide (16 chunks per row): chunk c of row r at c ^ (4 (r & 3) | ((r >> 2) & 3))
// A row read has 16 lanes reading one chunk of 16 consecutive rows; a transposing read has 32
// lanes reading 4 chunks (64 or 128 B apart in the 64 and 128 wide cases) of 4 consecutive rows.
#pragma once
#include "common.hpp"
#include "mfma_tile.hpp"
#include <utility>

namespace diffattn {

// Sum over the 32 lanes of the lane's half of the wave (lanes 0-31 or 32-63), for the row passes
// that take two rows per wave: the DPP steps of wave_sum within each 16-lane row, then the row
// swap with lane ^ 16. Every lane of a half ends with the same value.
__device__ __forceinline__ float half_sum(float x) {
    x += dpp_partner<0xB1>(x);
    x += dpp_partner<0x4E>(x);
    x += dpp_partner<0x141>(x);
    x += dpp_partner<0x140>(x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
}

namespace bwdt {

constexpr int kBN = 32;   // rows per tile

template <int W> __device__ __forceinline__ int swz(int row) {
    return W == 64 ? ((((row >> 1) & 1) << 2) | ((row >> 2) & 3)) : (((row & 3) << 2) | ((row >> 2) & 3));
}
// Row operand: row `row`, 16-byte logical chunk 2kk + h2.
template <int W> __device__ __forceinline__ int rowop(int row, int kk, int h2) {
    return row * (W * 2) + (((2 * kk + h2) ^ swz<W>(row)) * 16);
}
// Transposing read (A operand X^T of a row-major tile X whose rows are the MFMA k index): 16-lane
// group G covers columns 32 mt + 16 (G & 1) .. +15 and rows 16 kb + 4 (G >> 1) + 0..3 (lo) and
// +8 (hi); lane L supplies row + L/4 and columns + 4 (L % 4) .. +3.
template <int W> __device__ __forceinline__ int trop(int lane, int kb, int mt, int hi) {
    const int G = lane >> 4, L = lane & 15;
    const int row = 16 * kb + 4 * (G >> 1) + (L >> 2) + 8 * hi;
    const int c = mt * 4 + (G & 1) * 2 + ((L >> 1) & 1);
    return row * (W * 2) + ((c ^ swz<W>(row)) * 16) + (L & 1) * 8;
}
// Logical chunk held by LDS slot s of a W-wide tile (slot = row * (W / 8) + physical chunk), for
// the DMA that fills the tile slot by slot.
template <int W> __device__ __forceinline__ int slot_row(int s) { return s / (W / 8); }
template <int W> __device__ __forceinline__ int slot_chunk(int s) { return (s % (W / 8)) ^ swz<W>(s / (W / 8)); }

__device__ __forceinline__ bf16x8 tr_pair(const unsigned char* base, int lo, int hi) {
    const i16x4 a = lds_read_tr16((const bf16*)(base + lo));
    const i16x4 b = lds_read_tr16((const bf16*)(base + hi));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
// C registers kb*8 .. kb*8+7 of a 32x32 tile as the bf16 B operand of the next MFMA whose k index
// is the tile's row index (the k order matches the transposing read)
__device__ __forceinline__ bf16x8 c_to_b(const f32x16& x, int kb) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (bf16)x[kb * 8 + j];
    return r;
}

// acc += a b with the accumulator held in AGPRs. The gradient accumulators stay live across the
// whole tile loop while each tile's products are worked on by VALU code in VGPRs; issuing these
// accumulations by hand pins the accumulators to the AGPR file, where the compiler would otherwise
// copy them back and forth. The compiler does not look into the asm, so it also carries the two
// wait states that a VALU write of an operand needs before an MFMA reads it.
__device__ __forceinline__ void mfma_agpr(f32x16& acc, bf16x8 a, bf16x8 b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// The same without the two wait states, for the fixed-order pair loops, where each B operand is
// packed by the vector work of an earlier step, many instructions ahead of its first MFMA; the
// wait-state check of the product's gfx950 assembly covers every such site (and fails the build's
// CPU tests if a schedule ever puts the writing instruction closer).
__device__ __forceinline__ void mfma_agpr_ready(f32x16& acc, bf16x8 a, bf16x8 b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last such MFMA and VALU reads of its accumulator (more than the 18 the
// longest MFMA needs).
__device__ __forceinline__ void agpr_drain(f32x16& x0, f32x16& x1, f32x16& x2, f32x16& x3) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3));
}

// The end of a loop iteration whose asm MFMAs accumulate into these eight tiles: the compiler may
// copy or move accumulators at the top of the next iteration (out of sight of the asm, so with no
// wait states of its own), so the iteration ends with the 18 wait states an MFMA result needs
// before any other instruction touches it (8 + 8 + 4 here).
__device__ __forceinline__ void agpr_fence(f32x16& x0, f32x16& x1, f32x16& x2, f32x16& x3, f32x16& x4, f32x16& x5,
                                           f32x16& x6, f32x16& x7) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3), "+a"(x4), "+a"(x5), "+a"(x6), "+a"(x7));
}

template <int V> struct IC { static constexpr int value = V; };

// f(IC<0>), f(IC<1>), ..., f(IC<N - 1>): a loop whose index is a compile-time constant
template <int... I, class F> __device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
    (f(IC<I>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

}  // namespace bwdt
}  // namespace diffattn
