// bf16 GEMM for products with few output tiles:
// C = alpha * op(A) * op(B) + beta * C, fp32 accumulation, one rounding to bf16.
//
// With at most a few hundred 64 x 64 tiles each CU holds one workgroup of the
// tiled kernel, whose 4 waves (each a quarter of the tile) meet at a barrier
// after every 64-deep slab with 8 MFMAs each in between; 1024^2 x 4096 runs
// there at about 11% of the matrix cores, and neither more waves nor a deeper
// copy ring changed that. Here each of the 4 waves computes the whole 64 x 64
// tile over its own quarter of K (the RTX 3090 SGEMM article, section 7.2,
// cuts K so that more units work on one tile; here the units are the waves of
// one workgroup):
//   * every wave stages its slabs in two LDS stages of its own, in the tiled
//     kernel's layouts (A [64][64] k-contiguous, row-major B [64][64] as it
//     lies; a transposed operand the other way round), 32 KB per wave, copied
//     with LDS-destined 128-bit buffer loads and waited for with the wave's
//     own vmcnt: the K loop has no workgroup barrier;
//   * 32 MFMAs per wave and slab, fragments of the next k step read while
//     the current step's MFMAs run;
//   * after the loop each wave writes its fp32 partial tile to LDS, and wave
//     w adds the four partials of rows 16 w .. 16 w + 15 in wave order (the
//     same bits on every call; they differ from the tiled kernel's, which
//     adds the slabs in one sequence), then applies the epilogue to those rows.
//
// Edges as in the tiled kernel: descriptors end where the matrices end (rows
// past M, N and K arrive as zeros), k >= K inside a k-contiguous slab is
// zeroed in LDS, columns past N are never stored.
//
// Rows aligned to 4 bytes only (DW) fill the same LDS layouts with 4-byte
// copies, four times as many instructions for the same bytes; the arithmetic,
// and so every bit of the result, is that of 16-byte rows.

#include <type_traits>

#include "bf16_lds.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace dg {
namespace {

using namespace bf16lds;

constexpr int kT = 64;                       // tile edge
constexpr int kW = 4;                        // waves, one K range each
constexpr int kSlab = kT * kBK;              // bf16 elements of one operand slab
constexpr int kCopies = kSlab * 2 / 1024;    // 1 KB copies per operand slab
constexpr int kGroupM = 4;

template <bool EPI, bool TA, bool TB, bool DW>
__global__ __launch_bounds__(kW * 64, 1)
void gemm_bf16_few_kernel(GemmArgs<uint16_t> p, int tiles_m, int tiles_n) {
    // [wave][stage][A slab | B slab]: 32 KB per wave.
    __shared__ __attribute__((aligned(16))) uint16_t lds[kW * 2 * 2 * kSlab];
    static_assert(kW * 2 * 2 * kSlab * 2 >= kW * 16 * 64 * 16, "partial tiles fit the stages");

    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, kGroupM, tm, tn);
    const int64_t m0 = (int64_t)tm * kT, n0 = (int64_t)tn * kT;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int pl = lane & 15, g = lane >> 4;
    const int tr_row = pl >> 2, tr_col = (pl & 3) * 4;   // transposing-read role of this lane

    // This wave's K slabs: kb .. ke - 1 (empty for the last waves when K is short).
    const int64_t nk = (K + kBK - 1) / kBK;
    const int64_t per = (nk + kW - 1) / kW;
    const int64_t kb = (int64_t)wave * per;
    const int64_t ke = kb + per < nk ? kb + per : nk;
    uint16_t* const mine = lds + wave * (2 * 2 * kSlab);
    auto a_stage = [&](int st) { return mine + st * 2 * kSlab; };
    auto b_stage = [&](int st) { return mine + st * 2 * kSlab + kSlab; };

    // Descriptors of the k-contiguous operands (row-major A, transposed B):
    // rows m0 .. (or n0 ..) of the tile, ending after element K of the last
    // one, rounded up to the copy width (16 bytes, or 4 with DW).
    constexpr int64_t kRnd = DW ? 3 : 15;
    constexpr int kSlabCopies = (DW ? 4 : 1) * 2 * kCopies;   // copy instructions per slab
    const int64_t rows_a = M - m0 < kT ? M - m0 : kT;
    const rsrc_t a_desc = make_rsrc(p.A + m0 * lda, (uint32_t)((((rows_a - 1) * lda + K) * 2 + kRnd) & ~kRnd));
    const int64_t rows_bt = N - n0 < kT ? N - n0 : kT;
    const rsrc_t bt_desc = make_rsrc(p.B + n0 * ldb, (uint32_t)((((rows_bt - 1) * ldb + K) * 2 + kRnd) & ~kRnd));

    // One slab of both operands into stage `st`: 8 copies of 1 KB each, lane l
    // of copy I filling bytes 16 l .. of rows 8 I + l / 8 at physical chunk
    // l mod 8, so it fetches the logical chunk the layout puts there.
    const int lrow = lane >> 3, pos = lane & 7;
    auto copy_kc = [&](rsrc_t desc, int64_t ld, int64_t k0, uint32_t dst) {
#pragma unroll
        for (int I = 0; I < kCopies; ++I)
            dma16(desc, (uint32_t)(lrow * ld * 2 + ((pos ^ lrow) << 4)),
                  (uint32_t)(((8 * I) * ld + k0) * 2), dst + I * 1024);
    };
    auto copy_mn = [&](const uint16_t* base, int64_t ld, int64_t k0, int64_t extent, uint32_t dst) {
        // Rows k0 .. K - 1 of the storage, ending after its column `extent`.
        const int64_t rem = (((K - k0 - 1) * ld + extent) * 2 + 15) & ~(int64_t)15;
        const rsrc_t desc = make_rsrc(base + k0 * ld, rem < ((int64_t)1 << 31) ? (uint32_t)rem : 0x80000000u);
#pragma unroll
        for (int I = 0; I < kCopies; ++I) {
            const int row = 8 * I + lrow;
            dma16(desc, (uint32_t)(lrow * ld * 2 + ((pos ^ b_swz<kT>(row)) << 4)),
                  (uint32_t)((8 * I) * ld * 2), dst + I * 1024);
        }
    };
    // 4-byte copies: sub-copy s (0 .. 3) of 1 KB copy I fills LDS bytes
    // 1024 I + 256 s .. + 255, lane l the 4 bytes at 4 l of them, which lie
    // in rows 8 I + 2 s + h (h = l / 32) at in-row byte (4 l) mod 128 of the
    // layout. A k-contiguous row r keeps its logical chunk c at physical
    // chunk c ^ (r mod 8), here (l / 4) mod 8 ^ (2 s + h): the lane reads
    // in-row byte (4 l) mod 128 ^ 16 h ^ 32 s. An m/n-contiguous row r uses
    // the chunk swizzle b_swz(r), the same for both rows of a sub-copy: in-row
    // byte (4 l) mod 128 ^ 16 b_swz(8 I + 2 s).
    // The row stride and the LDS base pass through an empty asm statement, so
    // that the 32 per-copy scalar offsets of an operand are formed at each
    // slab instead of being hoisted out of the K loop, where they would not
    // fit in scalar registers.
    auto dw_kc = [&](rsrc_t desc, int64_t ld, int64_t k0, uint32_t dst) __attribute__((always_inline)) {
        const int ln = opaque_lane(), h = ln >> 5;
        uint32_t ld2 = (uint32_t)(ld * 2), base = dst;
        asm volatile("" : "+s"(ld2), "+s"(base));
        const uint32_t rowb = (uint32_t)h * ld2;
        const uint32_t in0 = (uint32_t)(((4 * ln) & 127) ^ (h << 4));
#pragma unroll
        for (int I = 0; I < kCopies; ++I)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                dma4(desc, rowb + (in0 ^ (uint32_t)(32 * s)),
                     (uint32_t)(8 * I + 2 * s) * ld2 + (uint32_t)(k0 * 2), base + 1024 * I + 256 * s);
    };
    auto dw_mn = [&](const uint16_t* bp, int64_t ld, int64_t k0, int64_t extent, uint32_t dst) __attribute__((always_inline)) {
        const int64_t rem = (((K - k0 - 1) * ld + extent) * 2 + 3) & ~(int64_t)3;
        const rsrc_t desc = make_rsrc(bp + k0 * ld, rem < ((int64_t)1 << 31) ? (uint32_t)rem : 0x80000000u);
        const int ln = opaque_lane(), h = ln >> 5;
        uint32_t ld2 = (uint32_t)(ld * 2), base = dst;
        asm volatile("" : "+s"(ld2), "+s"(base));
        const uint32_t rowb = (uint32_t)h * ld2;
        const uint32_t in0 = (uint32_t)((4 * ln) & 127);
#pragma unroll
        for (int I = 0; I < kCopies; ++I)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = 8 * I + 2 * s;
                dma4(desc, rowb + (in0 ^ (uint32_t)(b_swz<kT>(row) << 4)), (uint32_t)row * ld2,
                     base + 1024 * I + 256 * s);
            }
    };
    auto issue = [&](int64_t kt, int st) __attribute__((always_inline)) {
        const int64_t k0 = kt * kBK;
        const uint32_t As = lds_addr(a_stage(st)), Bs = lds_addr(b_stage(st));
        if constexpr (DW) {
            if constexpr (TA) dw_mn(p.A + m0, lda, k0, M - m0, As);
            else dw_kc(a_desc, lda, k0, As);
            if constexpr (TB) dw_kc(bt_desc, ldb, k0, Bs);
            else dw_mn(p.B + n0, ldb, k0, N - n0, Bs);
        } else {
            if constexpr (TA) copy_mn(p.A + m0, lda, k0, M - m0, As);
            else copy_kc(a_desc, lda, k0, As);
            if constexpr (TB) copy_kc(bt_desc, ldb, k0, Bs);
            else copy_mn(p.B + n0, ldb, k0, N - n0, Bs);
        }
        // Synchronous-copy build: the copies complete before anything else.
        if constexpr (kLdsCheck == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    };
    // Poison build: a stage is filled with NaN by its wave once the wave has
    // read it, before the next slab's copies (LDS operations of one wave run
    // in order, and the wait keeps the fill ahead of the copies).
    auto poison = [&](int st) {
        if constexpr (kLdsCheck == 1) {
            u32x4* q = reinterpret_cast<u32x4*>(a_stage(st));
            for (int i = lane; i < 2 * kSlab / 8; i += 64) q[i] = u32x4{~0u, ~0u, ~0u, ~0u};
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        }
    };

    // In the last slab of a ragged K, a k-contiguous slab holds the next
    // row's values at k >= K: zero them (lane r takes row r).
    const int k_tail = (int)(K - (nk - 1) * kBK);
    const bool tail_here = (!TA || TB) && ke == nk && kb < ke && k_tail < kBK;
    auto zero_tail = [&](int st) {
        auto zero_rows = [&](uint16_t* S) {
#pragma unroll
            for (int c = 0; c < kBK / 8; ++c) {
                if (8 * c + 8 <= k_tail) continue;
                u32x4* q = reinterpret_cast<u32x4*>(S + a_off(lane, c));
                *q = mask_tail(*q, k_tail - 8 * c);
            }
        };
        if constexpr (!TA) zero_rows(a_stage(st));
        if constexpr (TB) zero_rows(b_stage(st));
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fa[2][4], fb[2][4];
    auto read_frags = [&](int st, int ks, int buf) {
        const uint16_t* As = a_stage(st);
        const uint16_t* Bs = b_stage(st);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (TA) fa[buf][i] = read_b_frag<kT>(As, 32 * ks + 8 * g + tr_row, 16 * i + tr_col);
            else fa[buf][i] = *reinterpret_cast<const bf16x8*>(As + a_off(16 * i + pl, 4 * ks + g));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (TB) fb[buf][j] = *reinterpret_cast<const bf16x8*>(Bs + a_off(16 * j + pl, 4 * ks + g));
            else fb[buf][j] = read_b_frag<kT>(Bs, 32 * ks + 8 * g + tr_row, 16 * j + tr_col);
        }
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[buf][j], fa[buf][i], acc[j][i], 0, 0, 0);
    };

    // Two stages per wave: slab t + 1 is in flight while slab t is multiplied;
    // slab t + 2 goes into slab t's stage once its fragments are in registers.
    if (kb < ke) {
        if constexpr (kLdsCheck == 1) { poison(0); poison(1); }
        issue(kb, 0);
        if (kb + 1 < ke) issue(kb + 1, 1);
        // Wait for slab kb with slab kb + 1 still in flight (with 4-byte
        // copies 64 instructions, one more than vmcnt counts: one of them is
        // waited for too).
        if (kb + 1 < ke) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kSlabCopies < 63 ? kSlabCopies : 63));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        if (tail_here && kb + 1 == ke) zero_tail(0);
        read_frags(0, 0, 0);
        auto slab = [&](int64_t kt, int cur) {
            const int nxt = cur ^ 1;
            read_frags(cur, 1, 1);
            mfmas(0);
            if (kt + 1 < ke) {
                // Slab kt + 1 has landed (no later slab is in flight yet).
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                if (tail_here && kt + 2 == ke) zero_tail(nxt);
                read_frags(nxt, 0, 0);
            }
            mfmas(1);
            if (kt + 2 < ke) {
                // Both fragments of slab kt are in registers (the MFMAs above
                // waited for them): the stage takes slab kt + 2.
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                poison(cur);
                issue(kt + 2, cur);
            }
        };
        for (int64_t kt = kb; kt < ke; kt += 2) {
            slab(kt, 0);
            if (kt + 1 < ke) slab(kt + 1, 1);
        }
    }

    // Partial tiles: value (j, i) of lane l of wave w at f32x4 index
    // (16 w + 4 j + i) 64 + l, in the stages every wave has finished with.
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(16 * wave + 4 * j + i) * 64 + lane] = acc[j][i];
    __syncthreads();
    // Wave w finishes row block i = w: the four partials added in wave order.
    f32x4 sum[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        sum[j] = red[(4 * j + wave) * 64 + lane];
#pragma unroll
        for (int q = 1; q < kW; ++q) sum[j] += red[(16 * q + 4 * j + wave) * 64 + lane];
    }

    // Epilogue: sum[j] register r holds C(m0 + 16 w + pl, n0 + 16 j + 4 g + r).
    // With EPI, the product is also scaled by the row's and the column's
    // quantisation scale (row_factor folds the row scale into alpha).
    const float alpha = p.alpha, beta = p.beta;
    const int64_t row = m0 + 16 * wave + pl;
    if (row >= M) return;
    uint16_t* crow = p.C + row * p.ldc;
    const float fr = EPI ? row_factor(p, row) : alpha;
    // With DW, C's rows too may be aligned to 4 bytes only.
    using cvec = std::conditional_t<DW, u32x2_a4, u32x2>;
    u32x2 c0[4];
    if (beta != 0.f) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + 16 * j + 4 * g;
            c0[j] = col + 4 <= N ? (u32x2)*reinterpret_cast<const cvec*>(crow + col) : u32x2{0u, 0u};
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + 16 * j + 4 * g;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v[r] = fr * sum[j][r];
            if constexpr (EPI) v[r] = activate(v[r] * col_factor(p, col + r) + bias_at(p, col + r), p.act);
        }
        if (col + 4 <= N) {
            if (beta != 0.f) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[r] += beta * bf16_to_f32((uint16_t)(c0[j][r >> 1] >> (16 * (r & 1))));
            }
            *reinterpret_cast<cvec*>(crow + col) = cvec{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (col + r < N) {
                    float x = v[r];
                    if (beta != 0.f) x += beta * bf16_to_f32(crow[col + r]);
                    crow[col + r] = f32_to_bf16(x);
                }
            }
        }
    }
}

template <bool EPI, bool DW>
const void* pick_few(bool ta, bool tb) {
    return ta ? (tb ? (const void*)&gemm_bf16_few_kernel<EPI, true, true, DW>
                    : (const void*)&gemm_bf16_few_kernel<EPI, true, false, DW>)
              : (tb ? (const void*)&gemm_bf16_few_kernel<EPI, false, true, DW>
                    : (const void*)&gemm_bf16_few_kernel<EPI, false, false, DW>);
}

}  // namespace

hipError_t launch_bf16_few(const GemmArgs<uint16_t>& a, bool dw, hipStream_t s) {
    const int64_t tiles_m = (a.M + kT - 1) / kT, tiles_n = (a.N + kT - 1) / kT;
    int tm = (int)tiles_m, tn = (int)tiles_n;
    GemmArgs<uint16_t> args = a;
    void* kargs[] = {&args, &tm, &tn};
    const bool epi = has_epilogue(a);
    const void* fn = dw ? (epi ? pick_few<true, true>(a.ta, a.tb) : pick_few<false, true>(a.ta, a.tb))
                        : (epi ? pick_few<true, false>(a.ta, a.tb) : pick_few<false, false>(a.ta, a.tb));
    if (tiles_m * tiles_n > kMaxGrid) return hipErrorInvalidConfiguration;
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n)), dim3(kW * 64), kargs, 0, s);
}

}  // namespace dg
