// bf16 GEMM on gfx950 matrix cores: C = alpha * A * B + beta * C, row-major,
// fp32 accumulation, one rounding to bf16 at the end.
//
// Structure (the tiling recipe of the RTX 3090 SGEMM article, sections 3-5,
// and the pipelining of the Blackwell BF16 GEMM notes, section 2.3, rebuilt
// for CDNA4):
//   * one workgroup per BM x BN tile of C, tiles renumbered per XCD;
//   * K walked in slabs of BK = 64: A slab (BM x 64) and B slab (64 x BN) are
//     fetched with 128-bit loads into registers while the previous slab is
//     being multiplied, then written to the other half of a double-buffered
//     LDS (one barrier per slab);
//   * both slabs are stored k-contiguous in LDS ([row][k] for A, [col][k] for
//     B), so every MFMA operand fragment is one 128-bit LDS read. Row-major B
//     is transposed in registers (8 x 8 blocks of bf16) on its way to LDS;
//   * each LDS row is 8 chunks of 16 bytes whose position is XOR-swizzled with
//     the row index, so the 128-bit reads and writes of a wave hit distinct
//     banks (the padding idea of the article's section 4.3, without the
//     wasted bytes);
//   * each wave owns a (BM / WAVES_M) x (BN / WAVES_N) block of C held as
//     16x16 fp32 accumulators of v_mfma_f32_16x16x32_bf16;
//   * the epilogue forms alpha * acc + beta * C0 in fp32 (with EPI, bias and
//     activation before the beta term) and rounds to bf16 (notes, section
//     1.2 and 6.3), storing 16 bytes per lane.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 used here: lane l = p + 16 g
// (p in 0..15, g in 0..3) supplies A(row p, k = 8g .. 8g+7) and B(k = 8g ..
// 8g+7, col p), and receives D(row 4g + i, col p) in accumulator register i.
// Which k the hardware pairs is irrelevant to the result as long as A and B
// use the same assignment, which they do.
//
// The n index inside a wave is interleaved: MFMA block tn covers the columns
// wn0 + FN * p + tn (p = 0..15), so after the loop each lane holds FN
// consecutive columns of one row and can store them as one vector.
//
// Edges (Z-Turbo CUDA tuning page, section 3.1; Blackwell notes, section
// 4.3): rows of A past M, columns of B past N and k past K are loaded as zero,
// and the epilogue stores only in-range elements. Rows that are not 16-byte
// aligned (VEC = false) use the same 128-bit accesses at 2-byte alignment and
// element-wise ones only at the edges.
//
// Transposed operands (TA: A stored K x M; TB: B stored N x K) only change the
// global loads: an operand whose memory rows run along k (row-major A,
// transposed B) is loaded in 8-element chunks of a row, one whose rows run
// along m or n (row-major B, transposed A) in 8 x 8 blocks that are transposed
// in registers. Both land k-contiguous in LDS, so the MFMA loop is the same.

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dg {
namespace {

constexpr int kBK = 64;            // k per slab (8 chunks of 8 bf16)
constexpr int kGroupM = 4;         // tile rows per raster group

// Element offset of chunk `c` (8 bf16) of row `row` in a [rows][64] LDS tile,
// with an XOR-swizzled chunk position per tile. For the A tile, (row ^ row / 4
// ^ row / 32) mod 8 measures conflict-free on gfx950 (SQ_LDS_BANK_CONFLICT on
// probes of each pattern) for its fragment reads (16 consecutive rows), its
// chunk stores and its transposed block stores (rows 8 apart); the B tile's
// fragment reads take rows 8 apart, which cost one extra cycle per 16 lanes
// under every chunk XOR tried, and it keeps (row ^ row / 8) mod 8, under
// which its stores are conflict-free.
template <bool ATILE>
__device__ __forceinline__ int lds_off(int row, int c) {
    const int x = ATILE ? (row ^ (row >> 2) ^ (row >> 5)) : (row ^ (row >> 3));
    return row * kBK + ((c ^ (x & 7)) << 3);
}

// 8 consecutive bf16 from p, of which the first `valid` are in range.
__device__ __forceinline__ u32x4 load8_elems(const uint16_t* p, int valid) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t lo = (2 * e < valid) ? (uint32_t)p[2 * e] : 0u;
        uint32_t hi = (2 * e + 1 < valid) ? (uint32_t)p[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

template <bool VEC>
__device__ __forceinline__ u32x4 load8(const uint16_t* p, int valid) {
    if (valid >= 8)
        return VEC ? *reinterpret_cast<const u32x4*>(p) : (u32x4)*reinterpret_cast<const u32x4_a2*>(p);
    if (valid <= 0) return u32x4{0u, 0u, 0u, 0u};
    return load8_elems(p, valid);
}

// 8 x 8 transpose of bf16: x[r] holds row r (8 columns, two per dword);
// y[j] receives column j (8 rows, two per dword).
__device__ __forceinline__ void transpose8x8(const u32x4 (&x)[8], u32x4 (&y)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lo = x[2 * q][j >> 1], hi = x[2 * q + 1][j >> 1];
            y[j][q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                              : ((lo & 0xffffu) | (hi << 16));
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool VEC, bool EPI, bool TA, bool TB>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64)
void gemm_bf16_mfma_kernel(GemmArgs<uint16_t> p, int tiles_m, int tiles_n) {
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int A_CHUNKS = BM * (kBK / 8) / NT;          // 16-byte A chunks per thread
    constexpr int B_BLOCKS = (kBK / 8) * (BN / 8) / NT;    // 8x8 B blocks per thread
    constexpr int STAGE = (BM + BN) * kBK;                 // bf16 elements per LDS stage
    static_assert(A_CHUNKS * NT == BM * (kBK / 8), "A slab must split evenly");
    static_assert(B_BLOCKS * NT == (kBK / 8) * (BN / 8), "B slab must split evenly");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be 16-aligned");
    // A transposed A uses the block loader and a transposed B the chunk
    // loader; with BM == BN both take 8 registers of 16 bytes per thread.
    static_assert(BM == BN && A_CHUNKS == 8 * B_BLOCKS, "loaders share register shapes");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, kGroupM, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

    u32x4 ra[A_CHUNKS];
    u32x4 rb[B_BLOCKS][8];

    // 8 consecutive bf16; FULL: known to be in range, loaded with no test.
    auto ld8 = [&](auto full_tag, const uint16_t* base, int64_t off, int valid) -> u32x4 {
        if constexpr (decltype(full_tag)::value)
            return VEC ? *reinterpret_cast<const u32x4*>(base + off)
                       : (u32x4)*reinterpret_cast<const u32x4_a2*>(base + off);
        else
            return load8<VEC>(base + (valid > 0 ? off : 0), valid);
    };
    // Chunk loader (memory rows along k): thread t's chunk i is tile row
    // t / 8 + i * NT / 8 (of `extent` rows from r0), k chunk t % 8.
    auto load_chunks = [&](auto full_tag, const uint16_t* base, int64_t ld, int64_t extent,
                           int64_t r0, int64_t k0, u32x4* regs) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int r = t / 8 + i * (NT / 8), c = t % 8;
            const int64_t gm = r0 + r, gk = k0 + 8 * c;
            int valid = (gm < extent) ? (int)(K - gk < 8 ? K - gk : 8) : 0;
            regs[i] = ld8(full_tag, base, gm * ld + gk, valid);
        }
    };
    // Block loader (memory rows along m or n): thread t's block bi is the 8 x 8
    // block (kb, nb) of the 64 x BN slab; register r holds its row k = 8 kb + r.
    auto load_blocks = [&](auto full_tag, const uint16_t* base, int64_t ld, int64_t extent,
                           int64_t c0, int64_t k0, u32x4 (*regs)[8]) {
#pragma unroll
        for (int bi = 0; bi < B_BLOCKS; ++bi) {
            const int blk = t + bi * NT;
            const int kb = blk / (BN / 8), nb = blk % (BN / 8);
            const int64_t gn = c0 + 8 * nb;
            const int nvalid = (int)(extent - gn < 8 ? (extent - gn < 0 ? 0 : extent - gn) : 8);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int64_t gk = k0 + 8 * kb + r;
                const int valid = gk < K ? nvalid : 0;
                regs[bi][r] = ld8(full_tag, base, gk * ld + gn, valid);
            }
        }
    };
    auto store_chunks = [&](auto a_tile, uint16_t* S, const u32x4* regs) {
        constexpr bool AT = decltype(a_tile)::value;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int r = t / 8 + i * (NT / 8), c = t % 8;
            *reinterpret_cast<u32x4*>(S + lds_off<AT>(r, c)) = regs[i];
        }
    };
    auto store_blocks = [&](auto a_tile, uint16_t* S, const u32x4 (*regs)[8]) {
        constexpr bool AT = decltype(a_tile)::value;
#pragma unroll
        for (int bi = 0; bi < B_BLOCKS; ++bi) {
            const int blk = t + bi * NT;
            const int kb = blk / (BN / 8), nb = blk % (BN / 8);
            u32x4 y[8];
            transpose8x8(regs[bi], y);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<u32x4*>(S + lds_off<AT>(8 * nb + j, kb)) = y[j];
        }
    };
    // With TA the A registers hold blocks and with TB the B registers hold
    // chunks (same register count, viewed through the other shape).
    u32x4 (*ra_blocks)[8] = reinterpret_cast<u32x4 (*)[8]>(ra);
    u32x4* rb_chunks = &rb[0][0];

    // Interior slabs (tile inside M and N, slab inside K) load every chunk
    // whole with no range test; the edge path's per-lane tests would
    // otherwise sit in every slab, with waits for all outstanding loads.
    auto gload_slab = [&](auto full_tag, int64_t k0) {
        if constexpr (TA) load_blocks(full_tag, p.A, p.lda, M, m0, k0, ra_blocks);
        else load_chunks(full_tag, p.A, p.lda, M, m0, k0, ra);
        if constexpr (TB) load_chunks(full_tag, p.B, p.ldb, N, n0, k0, rb_chunks);
        else load_blocks(full_tag, p.B, p.ldb, N, n0, k0, rb);
    };
    const bool full_tile = m0 + BM <= M && n0 + BN <= N;
    auto gload = [&](int64_t k0) {
        if (full_tile && k0 + kBK <= K) gload_slab(std::true_type{}, k0);
        else gload_slab(std::false_type{}, k0);
    };

    auto sstore = [&](int stage) {
        uint16_t* As = smem + stage * STAGE;
        uint16_t* Bs = As + BM * kBK;
        if constexpr (TA) store_blocks(std::true_type{}, As, ra_blocks);
        else store_chunks(std::true_type{}, As, ra);
        if constexpr (TB) store_chunks(std::false_type{}, Bs, rb_chunks);
        else store_blocks(std::false_type{}, Bs, rb);
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wm0 = (wave / WAVES_N) * WTM, wn0 = (wave % WAVES_N) * WTN;
    const int pl = lane & 15, g = lane >> 4;

    auto compute = [&](int stage) {
        const uint16_t* As = smem + stage * STAGE;
        const uint16_t* Bs = As + BM * kBK;
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            bf16x8 a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(As + lds_off<true>(wm0 + 16 * i + pl, 4 * ks + g));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                b[j] = *reinterpret_cast<const bf16x8*>(Bs + lds_off<false>(wn0 + FN * pl + j, 4 * ks + g));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    const int64_t nk = (K + kBK - 1) / kBK;
    // Poison build: stage 0 starts as NaN; the other stage is refilled with
    // NaN at the top of each slab, after the barrier that retired it.
    if constexpr (kLdsCheck == 1) lds_retire(smem, STAGE * 2, threadIdx.x, blockDim.x);
    gload(0);
    sstore(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kLdsCheck == 1 && kt + 1 < nk)
            lds_retire(smem + (cur ^ 1) * STAGE, STAGE * 2, threadIdx.x, blockDim.x);
        if (kt + 1 < nk) gload((kt + 1) * kBK);
        compute(cur);
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: lane (pl, g) holds rows 4g + i of each 16-row block and the FN
    // consecutive columns wn0 + FN * pl .. + FN - 1.
    // With EPI, the product is also scaled by the row's and the column's
    // quantisation scale (row_factor folds the row scale into alpha).
    const float alpha = p.alpha, beta = p.beta;
    float bv[FN], cv[FN];
    if constexpr (EPI) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            bv[j] = bias_at(p, n0 + wn0 + FN * pl + j);
            cv[j] = col_factor(p, n0 + wn0 + FN * pl + j);
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm0 + 16 * i + 4 * g + r;
            const int64_t col = n0 + wn0 + FN * pl;
            if (row >= M) continue;
            const float fr = EPI ? row_factor(p, row) : alpha;
            float v[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) v[j] = fr * acc[i][j][r];
            if constexpr (EPI) {
#pragma unroll
                for (int j = 0; j < FN; ++j) v[j] = activate(v[j] * cv[j] + bv[j], p.act);
            }
            uint16_t* dst = p.C + row * p.ldc + col;
            if (FN == 8 && col + 8 <= N) {
                if (beta != 0.f) {
                    const u32x4 c0 = VEC ? *reinterpret_cast<const u32x4*>(dst)
                                         : (u32x4)*reinterpret_cast<const u32x4_a2*>(dst);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        v[j] += beta * bf16_to_f32((uint16_t)(c0[j >> 1] >> (16 * (j & 1))));
                }
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
                if (VEC) *reinterpret_cast<u32x4*>(dst) = o;
                else *reinterpret_cast<u32x4_a2*>(dst) = (u32x4_a2)o;
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if (col + j < N) {
                        float x = v[j];
                        if (beta != 0.f) x += beta * bf16_to_f32(dst[j]);
                        dst[j] = f32_to_bf16(x);
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool VEC, bool EPI>
const void* pick_general(bool ta, bool tb) {
    return ta ? (tb ? (const void*)&gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, VEC, EPI, true, true>
                    : (const void*)&gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, VEC, EPI, true, false>)
              : (tb ? (const void*)&gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, VEC, EPI, false, true>
                    : (const void*)&gemm_bf16_mfma_kernel<BM, BN, WAVES_M, WAVES_N, VEC, EPI, false, false>);
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_tiles(const GemmArgs<uint16_t>& a, bool vec, hipStream_t s) {
    const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm = (int)tiles_m, tn = (int)tiles_n;
    GemmArgs<uint16_t> args = a;
    void* kargs[] = {&args, &tm, &tn};
    const bool epi = has_epilogue(a);
    const void* fn =
        vec ? (epi ? pick_general<BM, BN, WAVES_M, WAVES_N, true, true>(a.ta, a.tb)
                   : pick_general<BM, BN, WAVES_M, WAVES_N, true, false>(a.ta, a.tb))
            : (epi ? pick_general<BM, BN, WAVES_M, WAVES_N, false, true>(a.ta, a.tb)
                   : pick_general<BM, BN, WAVES_M, WAVES_N, false, false>(a.ta, a.tb));
    if (tiles_m * tiles_n > kMaxGrid) return hipErrorInvalidConfiguration;
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n)), dim3(WAVES_M * WAVES_N * 64),
                           kargs, 0, s);
}

}  // namespace

hipError_t launch_bf16_general(const GemmArgs<uint16_t>& a, bool vec, hipStream_t s) {
    return launch_tiles<256, 256, 2, 2>(a, vec, s);
}

// Rows (and bases) of A, B and C aligned to 4 bytes: even leading dimensions.
static bool rows_4byte(const GemmArgs<uint16_t>& a) {
    auto al = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 3) == 0; };
    return al(a.A) && al(a.B) && al(a.C) && a.lda % 2 == 0 && a.ldb % 2 == 0 && a.ldc % 2 == 0;
}

hipError_t launch_bf16_mfma(const GemmArgs<uint16_t>& a, bool vec, void* ws, size_t ws_bytes,
                            int cus, hipStream_t s) {
    // 16-byte rows take the tiled kernel's 1 KB copies, 4-byte rows its
    // 4-byte ones; other rows, and offsets past its 31-bit range, the
    // element-wise kernel.
    if (bf16_tiled_fits(a) && (vec || rows_4byte(a)))
        return launch_bf16_tiled(a, !vec, ws, ws_bytes, cus, s);
    return launch_bf16_general(a, vec, s);
}

}  // namespace dg
