// fp32 GEMM (SGEMM) on gfx950 matrix cores: C = alpha * op(A) * op(B) + beta * C,
// fp32 products and fp32 accumulation (v_mfma_f32_16x16x4_f32).
//
// The RTX 3090 SGEMM article builds its 10.23 TFLOPS kernel from shared-memory
// tiles (section 3), float4 loads (section 4), register accumulators and
// double buffering (section 5). The same ideas are kept here, but the inner
// product runs on the fp32 matrix cores instead of per-thread FMAs:
//   * BM x BN tiles of C, renumbered per XCD; on the copy path without
//     split-K the grid is as many workgroups as can be resident (two per CU)
//     and each walks its tiles in turn, so no workgroup is launched between
//     rounds of tiles;
//   * K in slabs of BK = 32 in a double-buffered LDS (one barrier per slab);
//   * operands with 16-byte rows are copied from global memory straight into
//     LDS (buffer_load_dwordx4 ... lds) one slab ahead, each in its stored
//     layout: a k-contiguous operand (row-major A, transposed B) as [row][k]
//     with an XOR-swizzled chunk position, an m/n-contiguous one (row-major B,
//     transposed A) as [k][col] in plain rows;
//   * a k-contiguous tile gives each lane 4 consecutive k of one row per
//     128-bit LDS read, used in 4 successive MFMAs (blocks of 16 consecutive
//     rows); an m/n-contiguous tile gives each lane 4 consecutive rows at one
//     k, one per MFMA block (blocks interleaved 4 ways);
//   * every LDS access pattern measures bank-conflict free
//     (SQ_LDS_BANK_CONFLICT on probes of each pattern);
//   * the fused alpha/beta epilogue (with EPI, bias and activation before the
//     beta term) follows the block layout: 128-bit loads and stores when a
//     lane holds 4 consecutive columns, element-wise ones otherwise.
//
// Rows aligned only to 4 bytes (VEC = false, DW = true) take the same copy
// path with 4-byte LDS-destined loads, four per 1 KB copy, into the same
// layouts. Past the copies' 31-bit offset range operands are register-staged:
// 128-bit global accesses at 4-byte alignment (element-wise only at the
// edges), then LDS stores; transposed operands on that path are loaded as
// 4 x 4 blocks and transposed in registers, so the LDS layout is that of
// row-major operands.
//
// Operand layout of v_mfma_f32_16x16x4_f32: lane l = p + 16 g supplies A(row p,
// k_g) and B(k_g, col p) for one k per lane group g, and receives D(row 4g + i,
// col p) in accumulator register i. A and B use the same k for each g.

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dg {
namespace {

constexpr int kBK = 32;       // k per slab
// Tile rows per raster group. Each XCD owns a contiguous run of tiles and runs
// 64 workgroups at once (32 CUs x 2), so groups of 8 tile rows make each XCD's
// round an 8 x 8 block of tiles, the fewest A rows and B columns per round
// (L2 fetch at 4096^3: 752 MB per call against 779 MB with groups of 4; the
// time is the same).
constexpr int kGroupM = 8;

// Float offset of chunk `c` (4 floats) of row `row` in a [rows][32] tile. The
// chunk XOR (row ^ row / 4) mod 8 measures conflict-free on gfx950 for the
// fragment reads (16 consecutive rows x 4 chunks), the row-major stores (8
// rows x 8 chunks) and the transposed stores (32 rows 4 apart x 2 chunks);
// (row ^ row / 8) mod 8 cost the fragment reads 4 extra cycles each.
__device__ __forceinline__ int a_off(int row, int c) {
    return row * kBK + ((c ^ ((row ^ (row >> 2)) & 7)) << 2);
}

// Float offset of column `col` (a multiple of 4) of row `kr` in a [32][BN]
// tile. With a transposed B (SWZ) chunk positions are XORed with (kr / 4)
// mod 8: a row's 128-bit reads (consecutive chunks) stay conflict-free, and
// so do the transposed stores, which write 2 chunks of 8 rows 4 apart per
// 16 lanes (unswizzled they cost 53 extra cycles per store, an XOR with
// 2 * ((kr / 4) mod 8) still 7.5). Row-major B is stored in plain rows, whose
// stores and reads are conflict-free as they are.
template <int BN, bool SWZ>
__device__ __forceinline__ int b_off(int kr, int col) {
    if constexpr (SWZ) return kr * BN + ((((col >> 2) ^ ((kr >> 2) & 7))) << 2);
    return kr * BN + col;
}

__device__ __forceinline__ f32x4 load4_elems(const float* p, int valid) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (e < valid) ? p[e] : 0.f;
    return v;
}

template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float* p, int valid) {
    if (valid >= 4)
        return VEC ? *reinterpret_cast<const f32x4*>(p)
                   : (f32x4)*reinterpret_cast<const f32x4_a4*>(p);
    if (valid <= 0) return f32x4{0.f, 0.f, 0.f, 0.f};
    return load4_elems(p, valid);
}

// ws (only with SPLIT and ts.tail > 0): [counters: one int per split tile,
// padded to 256 bytes][slots: tail x parts partial tiles of BM x BN fp32,
// element e of thread t at e * NT + t].
// 4 x 4 transpose: y[j][i] = x[i][j].
__device__ __forceinline__ void transpose4x4(const f32x4 (&x)[4], f32x4 (&y)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = f32x4{x[0][j], x[1][j], x[2][j], x[3][j]};
}

// Whether a workgroup walks several tiles: on the copy paths without split-K,
// workgroup w takes tiles w, w + gridDim.x, ... (the same XCD slot each time).
// The register-staged path keeps one tile per workgroup: in a tile loop its
// registers no longer fit two waves per SIMD. With split-K every workgroup is
// one work item.
constexpr bool walks_tiles(bool copies, bool split) { return copies && !split; }

// One tile (or, with SPLIT, one K range of a tile) for work item bidx of nbid.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool VEC, bool DW, bool SPLIT, bool EPI,
          bool TA, bool TB>
__device__ __forceinline__ void f32_tile(GemmArgs<float> p, int tiles_m, int tiles_n, TailSplit ts,
                                         unsigned char* ws, const int bidx, const int nbid) {
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    constexpr int FM = WTM / 16;          // 16-row blocks per wave
    constexpr int NG = WTN / 64;          // 64-column groups per wave (4 MFMA blocks each)
    constexpr int A_CHUNKS = BM * (kBK / 4) / NT;
    constexpr int B_CHUNKS = kBK * (BN / 4) / NT;
    constexpr int STAGE = BM * kBK + kBK * BN;   // floats per LDS stage
    static_assert(A_CHUNKS * NT == BM * (kBK / 4), "A slab must split evenly");
    static_assert(B_CHUNKS * NT == kBK * (BN / 4), "B slab must split evenly");
    static_assert(WTM % 16 == 0 && WTN % 64 == 0, "wave tile shape");
    // The transposed loaders give each thread one 4 x 4 block of the slab.
    static_assert(!TA || (kBK / 4) * (BM / 4) == NT, "transposed A: one block per thread");
    static_assert(!TB || (kBK / 4) * (BN / 4) == NT, "transposed B: one block per thread");
    static_assert(A_CHUNKS == 4 && B_CHUNKS == 4, "block loaders reuse the chunk registers");
    // LDS-destined copies for operands with 16-byte rows. Each operand is
    // staged as it is stored: a row-major A as [m][k] and a transposed B as
    // [n][k] (k-contiguous, swizzled by a_off, read 4 consecutive k per lane),
    // a row-major B as [k][n] and a transposed A as [k][m] (plain rows, read
    // 4 consecutive n or m per lane). A k-contiguous operand's MFMA blocks
    // cover 16 consecutive rows (columns); an m/n-contiguous operand's blocks
    // are 4-way interleaved.
    // DW: rows aligned to 4 bytes only, copied by 4-byte LDS-destined loads
    // into the same layouts (256 bytes per wave instruction, four per 1 KB
    // copy of the 16-byte schedule).
    static_assert(!(VEC && DW), "one copy width");
    constexpr bool DMA = VEC || DW;
    constexpr bool AMC = DMA && TA;      // A^T staged [k][m]
    constexpr bool BKC = DMA && TB;      // B^T staged [n][k]
    static_assert(!DMA || (BM == 128 && BN == 128 && NT == 256 && NG == 1),
                  "the copy schedule covers 128 x 32 and 32 x 128 slabs with 4 waves");

    __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t nk = (K + kBK - 1) / kBK;
    int tm, tn, ti = 0, part = 0;
    int64_t kb = 0, ke = nk;                        // k slabs of this workgroup
    bool split_tile = false;
    if (!SPLIT || bidx < ts.full) {
        tile_coords(bidx, SPLIT ? ts.full : nbid, tiles_m, tiles_n, kGroupM, tm, tn);
    } else {
        // Split tail: consecutive workgroups take the K ranges of one tile.
        const int u = bidx - ts.full;
        ti = __builtin_amdgcn_readfirstlane(u / ts.parts);
        part = __builtin_amdgcn_readfirstlane(u - ti * ts.parts);
        raster_tile(ts.full + ti, tiles_m, tiles_n, kGroupM, tm, tn);
        kb = (int64_t)part * ts.cps;
        ke = kb + ts.cps < nk ? kb + ts.cps : nk;
        split_tile = true;
    }
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

    f32x4 ra[A_CHUNKS], rb[B_CHUNKS];

    // Transposed A (K x M storage): thread t loads rows k0 + 4 (t / (BM / 4)) + r,
    // r = 0..3, at columns m0 + 4 (t % (BM / 4)) .. + 3.
    // Transposed B (N x K storage): thread t loads rows n0 + 4 (t / 8) + r at
    // columns k0 + 4 (t % 8) .. + 3.
    const int ta_kb = t / (BM / 4), ta_mb = t % (BM / 4);
    const int tb_nb = t / (kBK / 4), tb_kb = t % (kBK / 4);

    // Global -> register loads of one slab. FULL: the tile lies inside M and
    // N and the slab inside K, so every chunk is loaded whole with no range
    // test. The edge path's per-lane tests would otherwise be compiled into
    // every slab, with a wait for all outstanding loads in the middle.
    auto gload_slab = [&](auto full_tag, int64_t k0) {
        constexpr bool FULL = decltype(full_tag)::value;
        auto ld = [&](const float* base, int64_t off, int valid) -> f32x4 {
            if constexpr (FULL)
                return VEC ? *reinterpret_cast<const f32x4*>(base + off)
                           : (f32x4)*reinterpret_cast<const f32x4_a4*>(base + off);
            else
                return load4<VEC>(base + (valid > 0 ? off : 0), valid);
        };
        if constexpr (TA) {
            const int64_t gm = m0 + 4 * ta_mb;
            const int mvalid = (int)(M - gm < 4 ? (M - gm < 0 ? 0 : M - gm) : 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t gk = k0 + 4 * ta_kb + r;
                const int valid = gk < K ? mvalid : 0;
                ra[r] = ld(p.A, gk * p.lda + gm, valid);
            }
        } else {
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i) {
                const int r = t / 8 + i * (NT / 8), c = t % 8;
                const int64_t gm = m0 + r, gk = k0 + 4 * c;
                const int valid = (gm < M) ? (int)(K - gk < 4 ? K - gk : 4) : 0;
                ra[i] = ld(p.A, gm * p.lda + gk, valid);
            }
        }
        if constexpr (TB) {
            const int64_t gk = k0 + 4 * tb_kb;
            const int kvalid = (int)(K - gk < 4 ? (K - gk < 0 ? 0 : K - gk) : 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t gn = n0 + 4 * tb_nb + r;
                const int valid = gn < N ? kvalid : 0;
                rb[r] = ld(p.B, gn * p.ldb + gk, valid);
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int idx = t + i * NT;
                const int kr = idx / (BN / 4), c = idx % (BN / 4);
                const int64_t gk = k0 + kr, gn = n0 + 4 * c;
                const int valid = (gk < K) ? (int)(N - gn < 4 ? N - gn : 4) : 0;
                rb[i] = ld(p.B, gk * p.ldb + gn, valid);
            }
        }
    };
    const bool full_tile = m0 + BM <= M && n0 + BN <= N;
    auto gload = [&](int64_t k0) {
        if (full_tile && k0 + kBK <= K) gload_slab(std::true_type{}, k0);
        else gload_slab(std::false_type{}, k0);
    };

    auto sstore = [&](int stage) {
        float* As = smem + stage * STAGE;
        float* Bs = As + BM * kBK;
        if constexpr (TA) {
            f32x4 y[4];
            transpose4x4(ra, y);     // y[j] = A(m0 + 4 ta_mb + j, 4 ta_kb .. + 3)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(As + a_off(4 * ta_mb + j, ta_kb)) = y[j];
        } else {
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i) {
                const int r = t / 8 + i * (NT / 8), c = t % 8;
                *reinterpret_cast<f32x4*>(As + a_off(r, c)) = ra[i];
            }
        }
        if constexpr (TB) {
            f32x4 y[4];
            transpose4x4(rb, y);     // y[j] = B(4 tb_kb + j, n0 + 4 tb_nb .. + 3)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(Bs + b_off<BN, TB>(4 * tb_kb + j, 4 * tb_nb)) = y[j];
        } else {
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const int idx = t + i * NT;
                const int kr = idx / (BN / 4), c = idx % (BN / 4);
                *reinterpret_cast<f32x4*>(Bs + b_off<BN, TB>(kr, 4 * c)) = rb[i];
            }
        }
    };

    f32x4 acc[FM][NG][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int gq = 0; gq < NG; ++gq)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][gq][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wm0 = (wave / WAVES_N) * WTM, wn0 = (wave % WAVES_N) * WTN;
    const int pl = lane & 15, g = lane >> 4;

    auto compute = [&](int stage) {
        const float* As = smem + stage * STAGE;
        const float* Bs = As + BM * kBK;
        if constexpr (AMC || BKC) {
            // k-contiguous tile: lane (pl, g) reads 4 consecutive k of row
            // (column) 16 x + pl once per 16 k and uses them in 4 successive
            // MFMAs. m/n-contiguous tile: one 128-bit read per k of 4
            // consecutive rows (columns) 4 pl .. 4 pl + 3, one per block.
#pragma unroll
            for (int q = 0; q < kBK / 16; ++q) {
                f32x4 a[FM], b[4];
                if constexpr (!AMC) {
#pragma unroll
                    for (int i = 0; i < FM; ++i)
                        a[i] = *reinterpret_cast<const f32x4*>(As + a_off(wm0 + 16 * i + pl, 4 * q + g));
                }
                if constexpr (BKC) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        b[j] = *reinterpret_cast<const f32x4*>(Bs + a_off(wn0 + 16 * j + pl, 4 * q + g));
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int kr = 16 * q + 4 * g + s;
                    f32x4 a4, b4;
                    if constexpr (AMC) a4 = *reinterpret_cast<const f32x4*>(As + kr * BM + wm0 + 4 * pl);
                    if constexpr (!BKC) b4 = *reinterpret_cast<const f32x4*>(Bs + kr * BN + wn0 + 4 * pl);
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[i][0][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                AMC ? a4[i] : a[i][s], BKC ? b[j][s] : b4[j], acc[i][0][j], 0, 0, 0);
                }
            }
            return;
        }
#pragma unroll
        for (int q = 0; q < kBK / 16; ++q) {
            f32x4 a[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = *reinterpret_cast<const f32x4*>(As + a_off(wm0 + 16 * i + pl, 4 * q + g));
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int kr = 16 * q + 4 * g + s;
                f32x4 b[NG];
#pragma unroll
                for (int gq = 0; gq < NG; ++gq)
                    b[gq] = *reinterpret_cast<const f32x4*>(Bs + b_off<BN, TB>(kr, wn0 + 64 * gq + 4 * pl));
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int gq = 0; gq < NG; ++gq)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[i][gq][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                a[i][s], b[gq][j], acc[i][gq][j], 0, 0, 0);
            }
        }
    };

    if constexpr (DMA) {
        // Operands with 16-byte rows: slabs go straight from global memory to
        // LDS (buffer_load_dwordx4 ... lds, 1 KB per wave instruction), with
        // no register staging and no LDS store instructions.
        //   k-contiguous tile ([128][32]: row-major A, transposed B): copy I
        //     fills tile rows 8 I .. 8 I + 7, lane l the 16 bytes at physical
        //     chunk l % 8 of row 8 I + l / 8, so it fetches the logical chunk
        //     that a_off puts there: l % 8 ^ ((row ^ row / 4) mod 8), which for
        //     row = 8 I + r is l % 8 ^ ((r ^ r / 4) mod 8) ^ 2 I mod 8.
        //   m/n-contiguous tile ([32][128]: row-major B, transposed A): copy I
        //     fills k rows 2 I and 2 I + 1 in plain order.
        // Each wave issues copies 4 wave .. 4 wave + 3 of each operand and
        // slab. Descriptors are re-based at every slab and end at the last
        // valid element, so rows (columns) past M, N and K arrive as zeros;
        // elements at k >= K inside the valid rows of a k-contiguous tile are
        // zeroed in LDS after they land.
        const int ar = lane >> 3, ap = lane & 7;
        const int s_ar = (ar ^ (ar >> 2)) & 7;
        const int wv = __builtin_amdgcn_readfirstlane(wave);   // scalar copy offsets
        uint32_t a_voff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a_voff[i] = (uint32_t)((ar * p.lda + 4 * (ap ^ s_ar ^ (2 * i))) * 4);
        const uint32_t b_voff = (uint32_t)(((lane >> 5) * p.ldb + 4 * (lane & 31)) * 4);
        const uint32_t at_voff = (uint32_t)(((lane >> 5) * p.lda + 4 * (lane & 31)) * 4);
        uint32_t bt_voff[4];     // transposed B: the A copy pattern over ldb
#pragma unroll
        for (int i = 0; i < 4; ++i)
            bt_voff[i] = (uint32_t)((ar * p.ldb + 4 * (ap ^ s_ar ^ (2 * i))) * 4);
        // 4-byte copies: sub-copy s (0..3) of copy I fills 256 bytes at
        // I * 1024 + s * 256. In a k-contiguous tile that is rows 8 I + 2 s
        // + h (h = lane / 32) at physical position lane % 32: chunk pc =
        // (lane % 32) / 4, element e = lane % 4. Its logical chunk is pc ^
        // ((r ^ r / 4) mod 8) ^ 2 I mod 8 with r = 2 s + h, and since the row
        // swizzle of 2 s + 1 is that of 2 s with bit 0 flipped, that is
        // (pc ^ h) ^ c(s, I) with c(s, I) = ((2 s) ^ (2 s) / 4 ^ 2 I) mod 8, a
        // compile-time value. dw_koff[c] holds the lane's byte offset for each
        // c (row h, logical chunk (pc ^ h) ^ c, element e); the row offset
        // 8 I + 2 s goes into the scalar offset. In an m/n-contiguous tile a
        // sub-copy is half of one k row: lane l takes element 64 (s & 1) + l
        // of row 2 I + s / 2.
        uint32_t dw_akoff[8], dw_bkoff[8];
        if constexpr (DW) {
            const int h = lane >> 5, pc = (lane & 31) >> 2, e = lane & 3;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                dw_akoff[c] = (uint32_t)((h * p.lda + 4 * ((pc ^ h) ^ c) + e) * 4);
                dw_bkoff[c] = (uint32_t)((h * p.ldb + 4 * ((pc ^ h) ^ c) + e) * 4);
            }
        }
        auto dw_c = [](int s, int I) { return ((2 * s) ^ ((2 * s) >> 2) ^ (2 * I)) & 7; };
        const int64_t rows_a = M - m0 < BM ? M - m0 : BM;
        const int64_t cols_b = N - n0 < BN ? N - n0 : BN;   // also B^T's valid rows
        auto dma = [&](int64_t kt, int stage) {
            const int64_t k0 = kt * kBK;
            const uint32_t As = lds_addr(smem + stage * STAGE);
            const uint32_t Bs = As + BM * kBK * 4;
            const int64_t rows_k = K - k0 < kBK ? K - k0 : kBK;
            if constexpr (AMC) {
                // A^T (K x M storage): copy I fills k rows 2 I, 2 I + 1 of
                // [32][128], plain, like a row-major B.
                const rsrc_t ad = make_rsrc(p.A + k0 * p.lda + m0,
                                            (uint32_t)(((rows_k - 1) * p.lda + rows_a) * 4));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int I = 4 * wv + i;
                    if constexpr (DW) {
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            dma4(ad, (uint32_t)(4 * lane),
                                 (uint32_t)(((2 * I + (s >> 1)) * p.lda + 64 * (s & 1)) * 4),
                                 As + I * 1024 + s * 256);
                    } else {
                        dma16(ad, at_voff, (uint32_t)(2 * I * p.lda * 4), As + I * 1024);
                    }
                }
            } else {
                const rsrc_t ad = make_rsrc(p.A + m0 * p.lda + k0,
                                            (uint32_t)(((rows_a - 1) * p.lda + (K - k0)) * 4));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int I = 4 * wv + i;
                    if constexpr (DW) {
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            dma4(ad, dw_akoff[dw_c(s, i)], (uint32_t)((8 * I + 2 * s) * p.lda * 4),
                                 As + I * 1024 + s * 256);
                    } else {
                        dma16(ad, a_voff[i], (uint32_t)(8 * I * p.lda * 4), As + I * 1024);
                    }
                }
            }
            if constexpr (BKC) {
                const rsrc_t bd = make_rsrc(p.B + n0 * p.ldb + k0,
                                            (uint32_t)(((cols_b - 1) * p.ldb + (K - k0)) * 4));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int J = 4 * wv + j;
                    if constexpr (DW) {
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            dma4(bd, dw_bkoff[dw_c(s, j)], (uint32_t)((8 * J + 2 * s) * p.ldb * 4),
                                 Bs + J * 1024 + s * 256);
                    } else {
                        dma16(bd, bt_voff[j], (uint32_t)(8 * J * p.ldb * 4), Bs + J * 1024);
                    }
                }
            } else {
                const rsrc_t bd = make_rsrc(p.B + k0 * p.ldb + n0,
                                            (uint32_t)(((rows_k - 1) * p.ldb + cols_b) * 4));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int J = 4 * wv + j;
                    if constexpr (DW) {
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            dma4(bd, (uint32_t)(4 * lane),
                                 (uint32_t)(((2 * J + (s >> 1)) * p.ldb + 64 * (s & 1)) * 4),
                                 Bs + J * 1024 + s * 256);
                    } else {
                        dma16(bd, b_voff, (uint32_t)(2 * J * p.ldb * 4), Bs + J * 1024);
                    }
                }
            }
        };
        // Zero the elements at k >= K (kr = K - k0 valid) of one stage's
        // k-contiguous tiles: A's rows 0 .. BM - 1 unless A is staged [k][m],
        // B^T's rows after them (a_off(BM + n, c) is B^T's a_off(n, c)) when B
        // is staged [n][k]. An m/n-contiguous tile has zero rows there already.
        constexpr int kZeroLo = AMC ? BM : 0, kZeroHi = BKC ? BM + BN : BM;
        auto zero_a_tail = [&](int stage, int kr) {
            float* As = smem + stage * STAGE;
            for (int row = kZeroLo + t; row < kZeroHi; row += NT) {
#pragma unroll
                for (int c = 0; c < kBK / 4; ++c) {
                    if (4 * c + 4 <= kr) continue;
                    f32x4* q = reinterpret_cast<f32x4*>(As + a_off(row, c));
                    f32x4 v = *q;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (4 * c + e < kr) ? v[e] : 0.f;
                    *q = v;
                }
            }
        };
        const int k_tail = (int)(K - (nk - 1) * kBK);   // 1 .. kBK
        const bool tail_here = kZeroLo < kZeroHi && ke == nk && k_tail < kBK;
        // Checking builds (no-ops otherwise): stage 0 starts as NaN and each
        // stage is refilled with NaN once retired (poison); copies are
        // bracketed by barriers (synchronous copies).
        if constexpr (kLdsCheck == 1) lds_retire(smem, STAGE * 4, t, NT);
        copy_begin();
        dma(kb, 0);
        copy_end();
        lds_barrier();
        if (tail_here && kb + 1 == ke) {
            zero_a_tail(0, k_tail);
            __syncthreads();
        }
        for (int64_t kt = kb; kt < ke; ++kt) {
            const int cur = (int)((kt - kb) & 1);
            // The other stage was last read in slab kt - 1, before the
            // barrier that ended it.
            if (kt + 1 < ke) {
                if constexpr (kLdsCheck == 1) lds_retire(smem + (cur ^ 1) * STAGE, STAGE * 4, t, NT);
                copy_begin();
                dma(kt + 1, cur ^ 1);
                copy_end();
            }
            compute(cur);
            if (kt + 1 < ke) {
                lds_barrier();
                if (tail_here && kt + 2 == ke) {
                    zero_a_tail(cur ^ 1, k_tail);
                    __syncthreads();
                }
            }
        }
    } else {
        // Poison build: stage 0 starts as NaN; the other stage is refilled
        // with NaN at the top of each slab, after the barrier that retired it.
        if constexpr (kLdsCheck == 1) lds_retire(smem, STAGE * 4, t, NT);
        gload(kb * kBK);
        sstore(0);
        __syncthreads();
        for (int64_t kt = kb; kt < ke; ++kt) {
            const int cur = (int)((kt - kb) & 1);
            if (kLdsCheck == 1 && kt + 1 < ke) lds_retire(smem + (cur ^ 1) * STAGE, STAGE * 4, t, NT);
            if (kt + 1 < ke) gload((kt + 1) * kBK);
            compute(cur);
            if (kt + 1 < ke) sstore(cur ^ 1);
            __syncthreads();
        }
    }

    if (SPLIT && split_tile) {
        // Store this K range's partial tile with device-coherent stores (sc1:
        // written through the per-XCD L2, as agent-scope atomics are), count
        // in once they have completed, and let the tile's last arrival read
        // the ranges back the same way and add them in range order before the
        // epilogue. No cache write-back or invalidate is needed.
        constexpr int E4 = FM * NG * 4;                   // f32x4 values per thread
        constexpr int kSc1 = 16;                          // cache-policy bit sc1
        int* counters = reinterpret_cast<int*>(ws);
        const unsigned char* slots = ws + (((int64_t)ts.tail * 4 + 255) & ~(int64_t)255);
        const rsrc_t sd = make_rsrc(slots + (int64_t)ti * ts.parts * (BM * BN * 4),
                                    (uint32_t)(ts.parts * BM * BN * 4));
        // Value c of thread t of range q sits at byte ((q * E4 + c) * NT + t) * 16.
        auto voff = [&](int q, int c) { return (uint32_t)(((q * E4 + c) * NT + t) * 16); };
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int gq = 0; gq < NG; ++gq)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][gq][j]), sd,
                                                           voff(part, (i * NG + gq) * 4 + j), 0, kSc1);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        __shared__ int last_flag;
        if (t == 0)
            last_flag = __hip_atomic_fetch_add(counters + ti, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) == ts.parts - 1;
        __syncthreads();
        if (!last_flag) return;
        // The last arrival reads every range back, its own included (its
        // stores have completed), so no accumulator stays live meanwhile.
        f32x4 sum[E4];
#pragma unroll
        for (int c = 0; c < E4; ++c) sum[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < ts.parts; ++q) {
            f32x4 v[E4];
#pragma unroll
            for (int c = 0; c < E4; ++c)
                v[c] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(sd, voff(q, c), 0, kSc1));
#pragma unroll
            for (int c = 0; c < E4; ++c) sum[c] += v[c];
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int gq = 0; gq < NG; ++gq)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][gq][j] = sum[(i * NG + gq) * 4 + j];
        // Leave the counter at zero for the next call that uses this workspace.
        if (t == 0) __hip_atomic_store(counters + ti, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    const float alpha = p.alpha, beta = p.beta;
    if constexpr (BKC) {
        // Block j of row block i: lane (pl, g) holds rows 16 i + 4 g + r (or
        // 16 g + 4 r + i with A staged [k][m]) of column wn0 + 16 j + pl; 16
        // lanes store 64 consecutive bytes.
        // With EPI, the product is also scaled by the row's and the column's
        // quantisation scale (row_factor folds the row scale into alpha).
        float bvk[4], cvk[4];
        if constexpr (EPI) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bvk[j] = bias_at(p, n0 + wn0 + 16 * j + pl);
                cvk[j] = col_factor(p, n0 + wn0 + 16 * j + pl);
            }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm0 + (AMC ? 16 * g + 4 * r + i : 16 * i + 4 * g + r);
                if (row >= M) continue;
                const float fr = EPI ? row_factor(p, row) : alpha;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t col = n0 + wn0 + 16 * j + pl;
                    if (col >= N) continue;
                    float x = fr * acc[i][0][j][r];
                    if constexpr (EPI) x = activate(x * cvk[j] + bvk[j], p.act);
                    float* dst = p.C + row * p.ldc + col;
                    if (beta != 0.f) x += beta * *dst;
                    *dst = x;
                }
            }
        }
        return;
    }
    float bv[NG][4], cv[NG][4];
    if constexpr (EPI) {
#pragma unroll
        for (int gq = 0; gq < NG; ++gq)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bv[gq][j] = bias_at(p, n0 + wn0 + 64 * gq + 4 * pl + j);
                cv[gq][j] = col_factor(p, n0 + wn0 + 64 * gq + 4 * pl + j);
            }
    }
    // With beta != 0, a workgroup that computes one tile loads all of its C
    // values before the first store (the stores could alias later loads, so
    // the compiler would otherwise wait for each load in turn). A workgroup
    // that walks tiles skips this: the extra registers would leave room for
    // only one wave per SIMD.
    constexpr bool kPreloadC = !walks_tiles(DMA, SPLIT);
    f32x4 cpre[kPreloadC ? FM : 1][4][NG];
    if (kPreloadC && beta != 0.f) {
#pragma unroll
        for (int i = 0; i < (kPreloadC ? FM : 1); ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm0 + (AMC ? 16 * g + 4 * r + i : 16 * i + 4 * g + r);
#pragma unroll
                for (int gq = 0; gq < NG; ++gq) {
                    const int64_t col = n0 + wn0 + 64 * gq + 4 * pl;
                    const float* src = p.C + row * p.ldc + col;
                    cpre[i][r][gq] = (row < M && col + 4 <= N)
                                         ? (VEC ? *reinterpret_cast<const f32x4*>(src)
                                                : (f32x4)*reinterpret_cast<const f32x4_a4*>(src))
                                         : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // Block i of an m-contiguous A covers rows 4 x + i.
            const int64_t row = m0 + wm0 + (AMC ? 16 * g + 4 * r + i : 16 * i + 4 * g + r);
            if (row >= M) continue;
            const float fr = EPI ? row_factor(p, row) : alpha;
#pragma unroll
            for (int gq = 0; gq < NG; ++gq) {
                const int64_t col = n0 + wn0 + 64 * gq + 4 * pl;
                float* dst = p.C + row * p.ldc + col;
                f32x4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = fr * acc[i][gq][j][r];
                if constexpr (EPI) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = activate(v[j] * cv[gq][j] + bv[gq][j], p.act);
                }
                if (col + 4 <= N) {
                    if (beta != 0.f) {
                        f32x4 c0;
                        if constexpr (kPreloadC) c0 = cpre[i][r][gq];
                        else c0 = VEC ? *reinterpret_cast<const f32x4*>(dst)
                                      : (f32x4)*reinterpret_cast<const f32x4_a4*>(dst);
#pragma unroll
                        for (int j = 0; j < 4; ++j) v[j] += beta * c0[j];
                    }
                    if (VEC) *reinterpret_cast<f32x4*>(dst) = v;
                    else *reinterpret_cast<f32x4_a4*>(dst) = (f32x4_a4)v;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (col + j < N) {
                            float x = v[j];
                            if (beta != 0.f) x += beta * dst[j];
                            dst[j] = x;
                        }
                    }
                }
            }
        }
    }
}

constexpr int kSlotsPerCu = 2;   // resident workgroups per compute unit (64 KB LDS each)

template <int BM, int BN, int WAVES_M, int WAVES_N, bool VEC, bool DW, bool SPLIT, bool EPI,
          bool TA, bool TB>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64)
void gemm_f32_mfma_kernel(GemmArgs<float> p, int tiles_m, int tiles_n, TailSplit ts,
                          unsigned char* ws) {
    if constexpr (!walks_tiles(VEC || DW, SPLIT)) {
        f32_tile<BM, BN, WAVES_M, WAVES_N, VEC, DW, SPLIT, EPI, TA, TB>(p, tiles_m, tiles_n, ts, ws,
                                                                      (int)blockIdx.x, (int)gridDim.x);
    } else {
        const int64_t total = (int64_t)tiles_m * tiles_n;
        for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
            // The previous tile's last slab may have been read from stage 0.
            if (b != (int64_t)blockIdx.x) __syncthreads();
            f32_tile<BM, BN, WAVES_M, WAVES_N, VEC, DW, SPLIT, EPI, TA, TB>(p, tiles_m, tiles_n, ts,
                                                                          ws, (int)b, (int)total);
        }
    }
}

// Reading one range's 64 KB partial tile back costs the last range about a
// quarter of a slab's time (32 k of a 128 x 128 tile, two workgroups per CU).
// Splitting a last round more than half full measured (one MI355X, with and
// without a workspace): 2304^2 x 2048 237 -> 204 us, 2048 x 2560 x 4096 467
// -> 408, 1664 x 2560 x 8192 921 -> 646, 2300 x 2290 x 2050 (unaligned) 332
// -> 227; 3072 x 2048 x 1024 in ranges of 8 slabs lost (123 -> 144), hence
// ranges of at least 16 slabs there.
constexpr double kF32FixupSlabs = 0.25;

TailSplit plan_tail(int64_t tiles, int64_t nk, int cus) {
    return plan_tail_split(tiles, nk, (int64_t)cus * kSlotsPerCu, 1, kF32FixupSlabs);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool VEC, bool DW, bool SPLIT, bool EPI>
const void* pick_layout(bool ta, bool tb) {
#define DG_F32_KERNEL(TA, TB) \
    (const void*)&gemm_f32_mfma_kernel<BM, BN, WAVES_M, WAVES_N, VEC, DW, SPLIT, EPI, TA, TB>
    return ta ? (tb ? DG_F32_KERNEL(true, true) : DG_F32_KERNEL(true, false))
              : (tb ? DG_F32_KERNEL(false, true) : DG_F32_KERNEL(false, false));
#undef DG_F32_KERNEL
}

// Copy mode: 0 register-staged, 1 16-byte copies (VEC), 2 4-byte copies (DW).
template <int BM, int BN, int WAVES_M, int WAVES_N, bool EPI, bool SPLIT>
const void* pick_mode(int mode, bool ta, bool tb) {
    return mode == 1 ? pick_layout<BM, BN, WAVES_M, WAVES_N, true, false, SPLIT, EPI>(ta, tb)
         : mode == 2 ? pick_layout<BM, BN, WAVES_M, WAVES_N, false, true, SPLIT, EPI>(ta, tb)
                     : pick_layout<BM, BN, WAVES_M, WAVES_N, false, false, SPLIT, EPI>(ta, tb);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool EPI>
const void* pick_kernel(int mode, bool split, bool ta, bool tb) {
    return split ? pick_mode<BM, BN, WAVES_M, WAVES_N, EPI, true>(mode, ta, tb)
                 : pick_mode<BM, BN, WAVES_M, WAVES_N, EPI, false>(mode, ta, tb);
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_tiles(const GemmArgs<float>& a, int mode, void* ws, size_t ws_bytes, int cus,
                        hipStream_t s) {
    const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm = (int)tiles_m, tn = (int)tiles_n;
    GemmArgs<float> args = a;
    TailSplit ts = plan_tail(tiles_m * tiles_n, (a.K + kBK - 1) / kBK, cus);
    const bool split = ws != nullptr && ts.tail > 0 && ws_bytes >= tail_workspace(ts, BM, BN);
    if (!split) ts = TailSplit{(int)(tiles_m * tiles_n), 0, 1, 0};
    unsigned char* wsp = split ? static_cast<unsigned char*>(ws) : nullptr;
    void* kargs[] = {&args, &tm, &tn, &ts, &wsp};
    const void* fn = has_epilogue(a)
                         ? pick_kernel<BM, BN, WAVES_M, WAVES_N, true>(mode, split, a.ta, a.tb)
                         : pick_kernel<BM, BN, WAVES_M, WAVES_N, false>(mode, split, a.ta, a.tb);
    const int64_t items = split ? (int64_t)ts.full + (int64_t)ts.tail * ts.parts : tiles_m * tiles_n;
    if (items > kMaxGrid) return hipErrorInvalidConfiguration;
    const int64_t slots = (int64_t)kSlotsPerCu * cus;
    const int64_t grid = walks_tiles(mode != 0, split) && items > slots ? slots : items;
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(WAVES_M * WAVES_N * 64), kargs, 0, s);
}

}  // namespace

// True when every offset the LDS-destined copies form (within one slab, from
// descriptors re-based per slab) fits in 31 bits: 128 rows of a k-contiguous
// operand (row-major A, transposed B), 32 rows of the other kind.
static bool f32_copies_fit(const GemmArgs<float>& a) {
    const int64_t lim = (int64_t)1 << 31;
    return (a.ta ? 32 * a.lda + 128 : 128 * a.lda + 32) * 4 < lim &&
           (a.tb ? 128 * a.ldb + 32 : 32 * a.ldb + 128) * 4 < lim;
}

hipError_t launch_f32_mfma(const GemmArgs<float>& a, bool vec, void* ws, size_t ws_bytes, int cus,
                           hipStream_t s) {
    // Operands with 16-byte rows take the 16-byte copy path, others the
    // 4-byte one; past the copies' offset range both take the register-staged
    // path at element alignment.
    const int mode = !f32_copies_fit(a) ? 0 : (vec ? 1 : 2);
    return launch_tiles<128, 128, 2, 2>(a, mode, ws, ws_bytes, cus, s);
}

size_t f32_mfma_workspace(int64_t M, int64_t N, int64_t K, int cus) {
    if (M < 1 || N < 1 || K < 1) return 0;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    return tail_workspace(plan_tail(tiles, (K + kBK - 1) / kBK, cus), 128, 128);
}

}  // namespace dg
