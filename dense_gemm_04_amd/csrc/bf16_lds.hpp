// LDS tile layouts and fragment reads shared by the bf16 kernels that stage
// 64-deep K slabs (gemm_bf16_tiled.hip, gemm_bf16_few.hip).
#pragma once

#include "common.hpp"

namespace dg {
namespace bf16lds {

constexpr int kBK = 64;

// A k-contiguous tile [rows][64]: chunk c (8 bf16) of row `row`. XOR with row mod 8 keeps
// the eight 16-byte reads of 8 consecutive rows on distinct banks, and keeps
// every address affine in the 16-row block index (one address register).
__device__ __forceinline__ int a_off(int row, int c) {
    return row * kBK + ((c ^ (row & 7)) << 3);
}

// B tile [64][BN]: chunk c (8 bf16) of row k. The XOR term is even, so a
// 16-lane group's two neighbouring chunks stay neighbours, and depends on
// k mod 4 (the rows within a 16-lane group of a transposing read) and on k / 8
// (the rows of the other groups). 256-wide rows (32 chunks, 512 bytes, twice
// the LDS banks) take k / 8 mod 4; 128-wide rows (16 chunks, 256 bytes, once
// the banks) take k / 8 mod 2, so the term stays below 16 and every chunk in
// its own row, and puts the odd groups of 8 rows on the other half of the banks.
// 64-wide rows (8 chunks, 128 bytes, half the banks) alternate bank halves by
// themselves, so the term separates the rows of each parity that a 32-lane
// read phase touches (k0 .. k0 + 3 and k0 + 8 .. k0 + 11): (k / 2 mod 2) and
// (k / 8 mod 2), values 0 .. 6, and rows 2m and 2m + 1 share it.
template <int BN>
__device__ __forceinline__ int b_swz(int k) {
    if constexpr (BN == 256) return ((k & 3) | (((k >> 3) & 3) << 2)) << 1;
    if constexpr (BN == 64) return (((k >> 1) & 1) << 1) | (((k >> 3) & 1) << 2);
    return ((k & 3) << 1) | (((k >> 3) & 1) << 3);
}
template <int BN>
__device__ __forceinline__ int b_off(int k, int c) {
    return k * BN + ((c ^ b_swz<BN>(k)) << 3);
}


template <int BN>
__device__ __forceinline__ bf16x8 read_b_frag(const uint16_t* Bs, int k0, int col) {
    // Lane 4r + q of each 16-lane group addresses row k0 + r (+4), columns col .. col+3.
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(Bs + b_off<BN>(k0, col >> 3) + (col & 7)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(Bs + b_off<BN>(k0 + 4, col >> 3) + (col & 7)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The lane index, computed afresh (mbcnt) from an operand the compiler cannot
// see through, so that it is not kept live in a register across the main loop.
__device__ __forceinline__ int opaque_lane() {
    unsigned m = ~0u;
    asm volatile("" : "+s"(m));
    return (int)__builtin_amdgcn_mbcnt_hi(m, __builtin_amdgcn_mbcnt_lo(m, 0u));
}

}  // namespace bf16lds
}  // namespace dg
