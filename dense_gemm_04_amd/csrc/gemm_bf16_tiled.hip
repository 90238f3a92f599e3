// bf16 GEMM on gfx950 matrix cores, vector path: C = alpha * A * B + beta * C,
// row-major, fp32 accumulation, one rounding to bf16 at the end.
//
// Used when A, B and C rows are 4-byte aligned: with 16-byte rows (the
// common case, and every workload shape of interest) slabs move in 1 KB
// copies, with rows aligned to 4 bytes only (DW: even leading dimensions) in
// 256-byte ones, into the same LDS layouts. The element-wise kernel in
// gemm_bf16_mfma.hip covers everything else.
//
// Tiling (the shared-memory tiling, float4 loads, register blocking and
// double buffering of the RTX 3090 SGEMM article, sections 3-5, and the
// asynchronous load/compute pipelining of the Blackwell BF16 GEMM notes,
// section 2.3, re-planned for CDNA4):
//   * one workgroup of 8 waves (2 x 4, each a 128 x 64 block of C) per
//     256 x 256 tile (or of 8 waves of 64 x 32 per 128 x 128 tile, for
//     products with few large tiles), tiles renumbered per XCD and rastered
//     in groups of 4 tile rows for L2 reuse;
//   * K in slabs of 64 held in two LDS stages. Slabs move from global memory
//     straight into LDS with LDS-destined 128-bit buffer loads (no register
//     round trip), two slabs ahead of the MFMAs; one barrier per slab
//     publishes slab t + 1 and retires every read of slab t;
//   * A is stored [m][k] (128-byte rows) and B [k][n] exactly as it lies in
//     memory (512-byte rows); each 16-byte chunk is placed at an XOR-swizzled
//     position within its row so that the 128-bit A reads and the
//     transposing B reads of a wave spread over all LDS banks;
//   * MFMA fragments: A(m, k..k+7) is one ds_read_b128; B(k..k+7, n) is two
//     ds_read_b64_tr_b16, which hand lane i of each 16-lane group column i of
//     a 4 x 16 block of row-major B. The next k step's fragments are read
//     while the current step's MFMAs run;
//   * v_mfma_f32_16x16x32_bf16 is issued with B as the first operand, so each
//     16 x 16 accumulator is a block of C transposed and every lane ends up
//     holding 4 consecutive columns of one row of C: the fused epilogue
//     (alpha * acc + beta * C0, then RNE to bf16; with EPI, bias and
//     activation before the beta term) uses 8-byte loads/stores;
//   * edges: the descriptors end where the matrices end, so rows of A past M
//     and rows of B past K read as zero; columns of B past N only feed output
//     columns that are never stored; k past K in the last slab is zeroed in
//     the LDS copy of A (Z-Turbo CUDA tuning page, section 3.1: zero-filled
//     tile edges; Blackwell notes, section 4.3: predicate the tail).
//   * split K (SPLIT, with a caller workspace): when the tiles leave the last
//     round of resident workgroups at most half full, as shapes with fewer
//     tiles than compute units do, each tile of that round is cut into K
//     ranges (the RTX 3090 SGEMM article, section 7.2: more multiprocessors
//     at work on the same tile); their fp32 partial tiles meet in the
//     workspace and the last range to finish adds them in range order;
//   * transposed operands (TA: A stored K x M; TB: B stored N x K) change only
//     where a slab's contiguous dimension lies. An operand whose rows run
//     along k (row-major A, transposed B) is copied and read the way A is
//     above: [row][k] in LDS, 128-bit fragment reads, the K tail zeroed in
//     LDS. An operand whose rows run along m or n (row-major B, transposed A)
//     is copied and read the way B is: [k][row] in LDS, transposing reads,
//     rows past K cut off by its descriptor.
//
// Operand layout of v_mfma_f32_16x16x32_bf16: lane l = p + 16 g supplies
// X(row p, k = 8g .. 8g+7) as its first operand and Y(k = 8g .. 8g+7, col p)
// as its second, and receives D(row 4g + r, col p) in register r. A and B use
// the same k assignment, so the hardware's internal pairing does not matter.

#include <type_traits>

#include "bf16_lds.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace dg {
namespace {

constexpr int kGroupM = 4;
using namespace bf16lds;

// ws (only with SPLIT and ts.tail > 0): [counters: one int per split tile,
// padded to 256 bytes][slots: tail x parts partial tiles of BM x BN fp32,
// value c of thread t at byte (c * threads + t) * 16 of its slot].
// DW: A, B and C rows (and bases) are aligned to 4 bytes, not 16.
// The second bound is waves per SIMD: 128 x 128 tiles run two workgroups of
// 8 waves per CU (at most 128 VGPRs) unless split over a workspace, which
// only happens when the split workgroups fit one per CU; 64 x 64 tiles (4
// waves) run up to four.
// KS = 2: two groups of WAVES_M x WAVES_N waves in one workgroup share each
// tile, each over its own half of K with its own LDS stages (the host
// launches it only with an even number of K slabs and no split); group 1
// hands its accumulators to group 0 through LDS after the loop. Both groups
// take every barrier in the same order: the loop's barriers depend only on
// the number of slabs, which the groups share.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool EPI, bool TA, bool TB, bool SPLIT, bool DW,
          int KS = 1>
__global__ __launch_bounds__(KS * WAVES_M * WAVES_N * 64, (BM == 128 && !SPLIT) || BM == 64 ? 4 : 2)
void gemm_bf16_tiled_kernel(GemmArgs<uint16_t> p, int tiles_m, int tiles_n, TailSplit ts,
                            unsigned char* ws) {
    static_assert(KS == 1 || (KS == 2 && !SPLIT && BM == 128 && BN == 128), "K split in the workgroup");
    constexpr int kNT = WAVES_M * WAVES_N * 64;                // threads of one group
    constexpr int kWaves = WAVES_M * WAVES_N;
    constexpr int kBM = BM, kBN = BN;
    constexpr int kWTM = BM / WAVES_M, kWTN = BN / WAVES_N;   // wave tile
    constexpr int kFM = kWTM / 16, kFN = kWTN / 16;
    constexpr int kAStage = BM * kBK;                         // bf16 elements
    constexpr int kBStage = kBK * BN;
    // Only the first wave of each SIMD (waves 0 .. kWaves / 2 - 1 with two
    // waves per SIMD) issues the 1 KB slab copies: a burst of copies fills
    // the texture unit's queue and stalls the issuing wave, and the other wave
    // on the SIMD keeps the matrix core busy meanwhile. The 4-byte copies are
    // four times as many instructions, and every wave shares them (4096^3
    // with 4100-element rows: 140 against 130 us; 512 x 8192 x 8192: 190
    // against 131 us).
    constexpr int kDmaWaves = DW ? kWaves : kWaves / 2;
    constexpr int kACopies = kAStage * 2 / 1024 / kDmaWaves;  // 1 KB LDS copies per issuing wave
    constexpr int kBCopies = kBStage * 2 / 1024 / kDmaWaves;
    constexpr int kBRowsPerCopy = 1024 / (BN * 2);            // rows of a [64][BN] slab per copy
    static_assert(kACopies * kDmaWaves * 1024 == kAStage * 2, "A slab must split evenly");
    static_assert(kBCopies * kDmaWaves * 1024 == kBStage * 2, "B slab must split evenly");
    static_assert(BN == 256 || BN == 128 || BN == 64, "B row length");
    static_assert((BM == 256 || BM == 128 || BM == 64) && (!TA || BM == BN), "operand tile sizes");
    static_assert(kWTM % 16 == 0 && kWTN % 16 == 0, "wave tile");
    // One array per operand and pipeline stage, so the compiler can tell which
    // stage an LDS-destined load writes and does not make reads of the other
    // stage wait for it. Laid out [A0 | A1 | B0 | B1]: stage 1 is 32 KB past
    // stage 0, within reach of the LDS instructions' immediate offset.
    // With KS = 2 each array holds both groups' stages, group g at g x stage.
    __shared__ __attribute__((aligned(16))) uint16_t a_st0[KS * kAStage];
    __shared__ __attribute__((aligned(16))) uint16_t a_st1[KS * kAStage];
    __shared__ __attribute__((aligned(16))) uint16_t b_st0[KS * kBStage];
    __shared__ __attribute__((aligned(16))) uint16_t b_st1[KS * kBStage];

    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int64_t nk = (K + kBK - 1) / kBK;
    int tm, tn, ti = 0, part = 0;
    int64_t kb = 0, ke = nk;                        // K slabs of this workgroup
    bool split_tile = false;
    if (!SPLIT || (int)blockIdx.x < ts.full) {
        tile_coords(blockIdx.x, SPLIT ? ts.full : gridDim.x, tiles_m, tiles_n, kGroupM, tm, tn);
    } else {
        // Split tail: consecutive workgroups take the K ranges of one tile.
        const int u = (int)blockIdx.x - ts.full;
        ti = __builtin_amdgcn_readfirstlane(u / ts.parts);
        part = __builtin_amdgcn_readfirstlane(u - ti * ts.parts);
        raster_tile(ts.full + ti, tiles_m, tiles_n, kGroupM, tm, tn);
        kb = (int64_t)part * ts.cps;
        ke = kb + ts.cps < nk ? kb + ts.cps : nk;
        split_tile = true;
    }
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    // wave / t: index within this thread's group (the whole workgroup when
    // KS = 1); grp: the group, which owns slabs grp x nk / 2 .. with KS = 2.
    const int grp = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) / kWaves;
    const int t = (int)threadIdx.x - grp * kNT, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    if constexpr (KS == 2) {
        kb = grp * (nk / 2);
        ke = kb + nk / 2;
    }
    auto a_stage = [&](int stage) -> uint16_t* { return (stage == 0 ? a_st0 : a_st1) + grp * kAStage; };
    auto b_stage = [&](int stage) -> uint16_t* { return (stage == 0 ? b_st0 : b_st1) + grp * kBStage; };

    // A descriptor (row-major A): rows m0 .. min(M, m0 + 256) - 1, ending
    // after element K of the last row (rounded up to its 16-byte chunk, which
    // stays in its page). Rows past M therefore arrive in LDS as zeros. The
    // same for a transposed B (rows n0 .. of the N x K storage). Each is dead
    // code when its operand is not k-contiguous.
    // With 4-byte copies the end is rounded up to a 4-byte word instead
    // (the base is only 4-byte aligned).
    constexpr int64_t kRnd = DW ? 3 : 15;
    const int64_t rows_a = (M - m0 < kBM) ? M - m0 : kBM;
    (void)kNT;
    const uint32_t a_bytes = (uint32_t)((((rows_a - 1) * lda + K) * 2 + kRnd) & ~kRnd);
    const rsrc_t a_desc = make_rsrc(p.A + m0 * lda, a_bytes);
    const int64_t rows_bt = (N - n0 < kBN) ? N - n0 : kBN;
    const uint32_t bt_bytes = (uint32_t)((((rows_bt - 1) * ldb + K) * 2 + kRnd) & ~kRnd);
    const rsrc_t bt_desc = make_rsrc(p.B + n0 * ldb, bt_bytes);

    // Global -> LDS copies. One buffer_load_dwordx4 ... lds moves 1 KB: lane l
    // fills bytes [16 l, 16 l + 16) of the destination, so each lane fetches
    // the global chunk that the swizzle puts at its LDS position.
    //   k-contiguous tile ([256][64], row-major A or transposed B): copy I
    //      fills rows 8 I .. 8 I + 7; lane -> row 8 I + l / 8.
    //   m/n-contiguous slab ([64][R], row-major B or transposed A): copy I
    //      fills rows Q I .. Q I + Q - 1 (Q = 1024 / row bytes); lane -> row
    //      Q I + l / (64 / Q).
    //
    // 4-byte copies (DW): sub-copy s (0 .. 3) of 1 KB copy I fills LDS bytes
    // 1024 I + 256 s .. + 255, lane l the 4 bytes at 4 l of them, in the same
    // swizzled layouts.
    //   k-contiguous tile: rows 8 I + 2 s + h (h = l / 32), physical chunk
    //      (l / 4) mod 8, which holds logical chunk (l / 4) mod 8 ^ (2 s + h)
    //      of the row (its row mod 8 is 2 s + h): in-row byte
    //      ((4 l) mod 128 ^ 16 h) ^ 32 s.
    //   m/n-contiguous slab (rows of BN elements; a transposed A has BM == BN):
    //      slab byte b = 1024 I + 256 s lies in row b / 2BN at in-row byte
    //      b mod 2BN + 4 l, whose chunk index is XOR-ed with the row's swizzle:
    //      in-row byte 4 l ^ x with x = b mod 2BN ^ 16 b_swz(row), the same
    //      for every lane.
    // The lane offsets come from an opaque copy of the lane index (see the
    // transposed copies below), and the row stride and LDS base pass through
    // an empty asm statement, so that the per-copy scalar offsets are formed
    // at each slab instead of being hoisted out of the K loop, where they
    // would not fit in scalar registers.
    auto dw_kc = [&](int ln, rsrc_t desc, int64_t ld, int I, int64_t k0, uint32_t dst) __attribute__((always_inline)) {
        const int h = ln >> 5;
        uint32_t ld2 = (uint32_t)(ld * 2), base = dst + I * 1024;
        asm volatile("" : "+s"(ld2), "+s"(base));
        const uint32_t rowb = (uint32_t)h * ld2;
        const uint32_t in0 = (uint32_t)(((4 * ln) & 127) ^ (h << 4));
#pragma unroll
        for (int s = 0; s < 4; ++s)
            dma4(desc, rowb + (in0 ^ (uint32_t)(32 * s)),
                 (uint32_t)(8 * I + 2 * s) * ld2 + (uint32_t)(k0 * 2), base + s * 256);
    };
    auto dw_mn = [&](int ln, rsrc_t desc, int64_t ld, int I, uint32_t dst) __attribute__((always_inline)) {
        uint32_t ld2 = (uint32_t)(ld * 2), base = dst;
        asm volatile("" : "+s"(ld2), "+s"(base));
        if constexpr (2 * kBN >= 256) {
            const uint32_t l4 = (uint32_t)(4 * ln);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int b = 1024 * I + 256 * s;
                const int row = b / (2 * kBN);
                const uint32_t x = (uint32_t)((b % (2 * kBN)) ^ (b_swz<kBN>(row) << 4));
                dma4(desc, l4 ^ x, (uint32_t)row * ld2, base + b);
            }
        } else {
            // 128-byte rows: sub-copy s holds rows 8 I + 2 s + h (h = l / 32),
            // which share one swizzle.
            const int h = ln >> 5;
            const uint32_t rowb = (uint32_t)h * ld2;
            const uint32_t in0 = (uint32_t)((4 * ln) & 127);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = 8 * I + 2 * s;
                const uint32_t x = (uint32_t)(b_swz<kBN>(row) << 4);
                dma4(desc, rowb + (in0 ^ x), (uint32_t)row * ld2, base + 1024 * I + 256 * s);
            }
        }
    };
    const int a_lrow = lane >> 3, a_pos = lane & 7;
    const int b_lrow = lane / (64 / kBRowsPerCopy), b_pos = lane % (64 / kBRowsPerCopy);
    // Inlined at each call site: an out-of-line copy routine would read its
    // captured descriptors and offsets back from per-lane stack memory.
    auto dma = [&](int64_t kt, int stage) __attribute__((always_inline)) {
        if (wave >= kDmaWaves) return;
        const int64_t k0 = kt * kBK;
        const uint32_t As = lds_addr(a_stage(stage));
        const uint32_t Bs = lds_addr(b_stage(stage));
        if constexpr (DW) {
            const int ln = opaque_lane();
            if constexpr (!TA) {
#pragma unroll
                for (int i = 0; i < kACopies; ++i) dw_kc(ln, a_desc, lda, wave * kACopies + i, k0, As);
            } else {
                const int64_t rem = (((K - k0 - 1) * lda + (M - m0)) * 2 + kRnd) & ~kRnd;
                const uint32_t bytes = rem < ((int64_t)1 << 31) ? (uint32_t)rem : 0x80000000u;
                const rsrc_t desc = make_rsrc(p.A + k0 * lda + m0, bytes);
#pragma unroll
                for (int i = 0; i < kACopies; ++i) dw_mn(ln, desc, lda, wave * kACopies + i, As);
            }
            if constexpr (!TB) {
                const int64_t rem = (((K - k0 - 1) * ldb + (N - n0)) * 2 + kRnd) & ~kRnd;
                const uint32_t bytes = rem < ((int64_t)1 << 31) ? (uint32_t)rem : 0x80000000u;
                const rsrc_t desc = make_rsrc(p.B + k0 * ldb + n0, bytes);
#pragma unroll
                for (int i = 0; i < kBCopies; ++i) dw_mn(ln, desc, ldb, wave * kBCopies + i, Bs);
            } else {
#pragma unroll
                for (int i = 0; i < kBCopies; ++i) dw_kc(ln, bt_desc, ldb, wave * kBCopies + i, k0, Bs);
            }
            return;
        }
        if constexpr (!TA) {
#pragma unroll
            for (int i = 0; i < kACopies; ++i) {
                const int I = wave * kACopies + i;
                const int c = a_pos ^ a_lrow;       // (8 I + a_lrow) mod 8 == a_lrow
                dma16(a_desc, (uint32_t)(a_lrow * lda * 2 + c * 16),
                      (uint32_t)(((8 * I) * lda + k0) * 2), As + I * 1024);
            }
        } else {
            // Transposed A, slab rows k0 .. K - 1 of the K x M storage. The
            // per-copy lane offsets are recomputed here from an opaque copy
            // of the lane index rather than kept live across the loop: with
            // both operands copied this way they would not fit in registers,
            // and a spilled offset's reload waits for every copy in flight.
            const int64_t rem = (((K - k0 - 1) * lda + (M - m0)) * 2 + 15) & ~(int64_t)15;
            const uint32_t bytes = rem < ((int64_t)1 << 31) ? (uint32_t)rem : 0x80000000u;
            const rsrc_t desc = make_rsrc(p.A + k0 * lda + m0, bytes);
            const int ln = opaque_lane();
            const int lrow = ln / (64 / kBRowsPerCopy), pos = ln % (64 / kBRowsPerCopy);
#pragma unroll
            for (int i = 0; i < kACopies; ++i) {
                const int I = wave * kACopies + i;
                const int row = kBRowsPerCopy * I + lrow;
                const int c = pos ^ b_swz<BM>(row);
                dma16(desc, (uint32_t)(lrow * lda * 2 + c * 16),
                      (uint32_t)((kBRowsPerCopy * I) * lda * 2), As + I * 1024);
            }
        }
        if constexpr (!TB) {
            // B descriptor for this slab: rows k0 .. K - 1, ending after column N of
            // row K - 1, so rows past K arrive as zeros.
            const int64_t rem = (((K - k0 - 1) * ldb + (N - n0)) * 2 + 15) & ~(int64_t)15;
            const uint32_t b_bytes = rem < ((int64_t)1 << 31) ? (uint32_t)rem : 0x80000000u;
            const rsrc_t b_desc = make_rsrc(p.B + k0 * ldb + n0, b_bytes);
            if constexpr (TA) {
                // Both operands copied as m/n-contiguous slabs: recompute the
                // lane offsets here too (see the transposed A copies).
                const int ln = opaque_lane();
                const int lrow = ln / (64 / kBRowsPerCopy), pos = ln % (64 / kBRowsPerCopy);
#pragma unroll
                for (int i = 0; i < kBCopies; ++i) {
                    const int I = wave * kBCopies + i;
                    const int row = kBRowsPerCopy * I + lrow;
                    const int c = pos ^ b_swz<BN>(row);
                    dma16(b_desc, (uint32_t)(lrow * ldb * 2 + c * 16),
                          (uint32_t)((kBRowsPerCopy * I) * ldb * 2), Bs + I * 1024);
                }
            } else {
#pragma unroll
                for (int i = 0; i < kBCopies; ++i) {
                    const int I = wave * kBCopies + i;
                    const int row = kBRowsPerCopy * I + b_lrow;
                    const int c = b_pos ^ b_swz<BN>(row);
                    dma16(b_desc, (uint32_t)(b_lrow * ldb * 2 + c * 16),
                          (uint32_t)((kBRowsPerCopy * I) * ldb * 2), Bs + I * 1024);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kBCopies; ++i) {
                const int I = wave * kBCopies + i;
                const int c = a_pos ^ a_lrow;
                dma16(bt_desc, (uint32_t)(a_lrow * ldb * 2 + c * 16),
                      (uint32_t)(((8 * I) * ldb + k0) * 2), Bs + I * 1024);
            }
        }
    };

    // In the last slab of a ragged K, a k-contiguous tile (row-major A,
    // transposed B) would hold the next row's values at k >= K: zero them in
    // LDS (threads stride over the rows). An m/n-contiguous slab is already
    // zero there.
    constexpr bool kZeroTail = !TA || TB;
    auto zero_a_tail = [&](int stage, int kr) {
        if constexpr (!TA) {
            uint16_t* As = a_stage(stage);
            for (int row = t; row < kBM; row += kNT) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    if (8 * c + 8 <= kr) continue;
                    u32x4* q = reinterpret_cast<u32x4*>(As + a_off(row, c));
                    *q = mask_tail(*q, kr - 8 * c);
                }
            }
        }
        if constexpr (TB) {
            uint16_t* Bs = b_stage(stage);
            for (int row = t; row < kBN; row += kNT) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    if (8 * c + 8 <= kr) continue;
                    u32x4* q = reinterpret_cast<u32x4*>(Bs + a_off(row, c));
                    *q = mask_tail(*q, kr - 8 * c);
                }
            }
        }
    };

    f32x4 acc[kFN][kFM];
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int i = 0; i < kFM; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int wm0 = (wave / WAVES_N) * kWTM, wn0 = (wave % WAVES_N) * kWTN;
    const int pl = lane & 15, g = lane >> 4;
    const int tr_row = pl >> 2, tr_col = (pl & 3) * 4;   // transposing-read role of this lane

    bf16x8 fa[2][kFM], fb[2][kFN];
    auto read_frags = [&](int stage, int ks, int buf) {
        const uint16_t* As = a_stage(stage);
        const uint16_t* Bs = b_stage(stage);
#pragma unroll
        for (int i = 0; i < kFM; ++i) {
            if constexpr (TA)
                fa[buf][i] = read_b_frag<BM>(As, 32 * ks + 8 * g + tr_row, wm0 + 16 * i + tr_col);
            else
                fa[buf][i] = *reinterpret_cast<const bf16x8*>(As + a_off(wm0 + 16 * i + pl, 4 * ks + g));
        }
#pragma unroll
        for (int j = 0; j < kFN; ++j) {
            if constexpr (TB)
                fb[buf][j] = *reinterpret_cast<const bf16x8*>(Bs + a_off(wn0 + 16 * j + pl, 4 * ks + g));
            else
                fb[buf][j] = read_b_frag<BN>(Bs, 32 * ks + 8 * g + tr_row, wn0 + 16 * j + tr_col);
        }
    };
    // The MFMA runs go at raised wave priority, so that a wave with matrix
    // work to issue wins the SIMD's issue slot over one that is issuing
    // copies or LDS reads.
    auto mfmas = [&](int buf) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < kFM; ++i)
#pragma unroll
            for (int j = 0; j < kFN; ++j)
                acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[buf][j], fa[buf][i],
                                                                    acc[j][i], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
    };

    // Pipeline (two LDS stages): while slab t is multiplied, slab t + 1 is in
    // flight to the other stage. The barrier in the middle of each slab both
    // publishes slab t + 1 and retires every read of slab t, after which slab
    // t + 2 may overwrite it. Fragments of the next k step are always read one
    // step ahead of the MFMAs that use them.
    // Slabs kb .. ke - 1 (all of K unless the tile is split); only the range
    // that ends at nk holds the ragged K tail.
    const int k_tail = (int)(K - (nk - 1) * kBK);   // 1 .. 64
    const bool tail_here = kZeroTail && ke == nk && k_tail < kBK;
    // The barrier after the zeroing: taken by both groups of a KS = 2
    // workgroup at the same slab index (their ranges have equal lengths).
    const bool tail_bar = kZeroTail && k_tail < kBK && (KS == 2 || ke == nk);
    // Checking builds: both stages start as NaN (poison) and every batch of
    // copies is bracketed by barriers (synchronous copies); no-ops otherwise.
    auto retire = [&](int stage) {
        if constexpr (kLdsCheck == 1) {
            lds_retire(a_stage(stage), kAStage * 2, t, kNT);
            lds_retire(b_stage(stage), kBStage * 2, t, kNT);
        }
    };
    retire(0);
    retire(1);
    copy_begin();
    dma(kb, 0);
    copy_end();
    lds_barrier();
    if (tail_bar && kb + 1 == ke) {
        if (tail_here) zero_a_tail(0, k_tail);
        lds_barrier();
    }
    if (kb + 1 < ke) {
        copy_begin();
        dma(kb + 1, 1);
        copy_end();
    }
    read_frags(0, 0, 0);
    // One slab; `cur` is a literal at both call sites (the loop is unrolled by
    // two), so every LDS access names its stage array statically.
    auto slab = [&](int64_t kt, int cur) {
        read_frags(cur, 1, 1);
        mfmas(0);
        if (kt + 1 < ke) {
            lds_barrier();
            // Every read of stage `cur` (slab kt) is retired here.
            retire(cur);
            if (tail_bar && kt + 2 == ke) {
                if (tail_here) zero_a_tail(cur ^ 1, k_tail);
                lds_barrier();
            }
            if (kt + 2 < ke) {
                copy_begin();
                dma(kt + 2, cur);
                copy_end();
            }
            read_frags(cur ^ 1, 0, 0);
        }
        mfmas(1);
    };
    for (int64_t kt = kb; kt < ke; kt += 2) {
        slab(kt, 0);
        if (kt + 1 < ke) slab(kt + 1, 1);
    }

    if constexpr (KS == 2) {
        // Group 1 hands its partial tile to group 0 through LDS (value c of
        // lane l of wave w at f32x4 (c x waves + w) x 64 + l, across a_st0 and
        // a_st1), and group 0 adds it to its own: acc = first half of K +
        // second half, the same bits on every call.
        constexpr int E4 = kFN * kFM;
        constexpr int kPerArr = KS * kAStage * 2 / 16;                // f32x4 per A array
        static_assert(E4 * kWaves * 64 <= 2 * kPerArr, "partial tile fits the A stages");
        auto slot = [&](int c) -> f32x4* {
            const int q = (c * kWaves + wave) * 64 + lane;
            return reinterpret_cast<f32x4*>(q < kPerArr ? a_st0 : a_st1) + (q < kPerArr ? q : q - kPerArr);
        };
        lds_only_barrier();                            // every stage read is done
        if (grp == 1) {
#pragma unroll
            for (int j = 0; j < kFN; ++j)
#pragma unroll
                for (int i = 0; i < kFM; ++i) *slot(j * kFM + i) = acc[j][i];
        }
        lds_only_barrier();
        if (grp == 1) {
            // The epilogue below takes one barrier for whole tiles (before
            // its scratch use) and none otherwise: match it, then leave.
            if ((kWTN == 64 || kWTN == 32) && m0 + kBM <= M && n0 + kBN <= N) lds_only_barrier();
            return;
        }
#pragma unroll
        for (int j = 0; j < kFN; ++j)
#pragma unroll
            for (int i = 0; i < kFM; ++i) acc[j][i] += *slot(j * kFM + i);
    }

    if constexpr (SPLIT) {
        if (split_tile) {
            // Store this K range's partial tile with device-coherent stores
            // (sc1: written through the per-XCD L2), count in once they have
            // completed, and let the tile's last arrival read the ranges back
            // the same way and add them in range order before the epilogue.
            // No cache write-back or invalidate is needed.
            constexpr int E4 = kFN * kFM;                     // f32x4 values per thread
            constexpr int kSc1 = 16;                          // cache-policy bit sc1
            int* counters = reinterpret_cast<int*>(ws);
            const unsigned char* slots = ws + (((int64_t)ts.tail * 4 + 255) & ~(int64_t)255);
            const rsrc_t sd = make_rsrc(slots + (int64_t)ti * ts.parts * (kBM * kBN * 4),
                                        (uint32_t)(ts.parts * kBM * kBN * 4));
            auto voff = [&](int q, int c) { return (uint32_t)(((q * E4 + c) * kNT + t) * 16); };
#pragma unroll
            for (int j = 0; j < kFN; ++j)
#pragma unroll
                for (int i = 0; i < kFM; ++i)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[j][i]), sd,
                                                           voff(part, j * kFM + i), 0, kSc1);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __syncthreads();
            __shared__ int last_flag;
            if (t == 0)
                last_flag = __hip_atomic_fetch_add(counters + ti, 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) == ts.parts - 1;
            __syncthreads();
            if (!last_flag) return;
            // The last arrival reads every range back, its own included (its
            // stores have completed): one value of all eight possible ranges
            // at a time (loads past the tile's `parts` ranges fall outside the
            // descriptor and read as zeros), added in range order.
#pragma unroll
            for (int j = 0; j < kFN; ++j) {
#pragma unroll
                for (int i = 0; i < kFM; ++i) {
                    f32x4 v[kMaxSplitParts];
#pragma unroll
                    for (int q = 0; q < kMaxSplitParts; ++q)
                        v[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                             sd, voff(q, j * kFM + i), 0, kSc1));
                    f32x4 sum = v[0];
#pragma unroll
                    for (int q = 1; q < kMaxSplitParts; ++q) sum += v[q];
                    acc[j][i] = sum;
                }
            }
            // Leave the counter at zero for the next call that uses this workspace.
            if (t == 0) __hip_atomic_store(counters + ti, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // Epilogue: acc[j][i] register r holds C(m0 + wm0 + 16 i + pl, n0 + wn0 + 16 j + 4 g + r).
    // With EPI, the product is also scaled by the row's and the column's
    // quantisation scale (row_factor folds the row scale into alpha).
    const float alpha = p.alpha, beta = p.beta;
    if constexpr (kWTN == 64 || kWTN == 32) {
    if (m0 + kBM <= M && n0 + kBN <= N) {
        // Whole tiles: C is read and written 16 bytes (8 columns) per lane
        // and instruction, 8 rows of 128 bytes (64-column wave tiles) or 16
        // rows of 64 bytes (32-column ones) per wave instruction, instead of
        // the 4 columns a lane holds after the MFMAs (16 rows of 32 bytes
        // per instruction): the projection with beta = 1 ran 685 against
        // 646 us in a copy with this access pattern, 2560^3 with beta = 1 on
        // 128 x 128 tiles 40.8 against 36.4 us. Each 16-row block of a wave's
        // results goes through a wave-private LDS scratch into row order.
        // Lane l takes columns
        // 8 (l mod kLpr) .. + 7 of rows l / kLpr + kRpp h of each block. The
        // arithmetic is the same as below.
        constexpr int kLpr = kWTN / 8;             // lanes per row (8 columns each)
        constexpr int kRpp = 64 / kLpr;            // rows per pass
        constexpr int kPasses = 16 / kRpp;
        const int cc = lane % kLpr, rr = lane / kLpr;
        const int64_t gcol = n0 + wn0 + 8 * cc;
        float cf8[8], bv8[8];
        if constexpr (EPI) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                cf8[e] = col_factor(p, gcol + e);
                bv8[e] = bias_at(p, gcol + e);
            }
        }
        // C rows aligned to 4 bytes only (DW): the same 128-bit accesses at
        // 4-byte alignment.
        using cvec = std::conditional_t<DW, u32x4_a4, u32x4>;
        u32x4 c0q[kFM][kPasses];
        if (beta != 0.f) {
#pragma unroll
            for (int i = 0; i < kFM; ++i)
#pragma unroll
                for (int h = 0; h < kPasses; ++h)
                    c0q[i][h] = *reinterpret_cast<const cvec*>(
                        p.C + (m0 + wm0 + 16 * i + rr + kRpp * h) * p.ldc + gcol);
        }
        // Every wave has read its last fragments: the stages are free.
        lds_only_barrier();
        // Scratch rows: 64 floats with 16-byte chunk c of row r at chunk
        // c ^ (r mod 16) for 64-column wave tiles (measured conflict-free);
        // kWTN + 4 floats, unswizzled, for 32-column ones (about 2 conflict
        // cycles per access measured; two XOR layouts measured 4).
        constexpr int kScrLd = kWTN == 64 ? 64 : kWTN + 4, kScrPerStage = kWaves / 2;
        auto scr_at = [](int r, int c) { return r * kScrLd + 4 * (kWTN == 64 ? (c ^ (r & 15)) : c); };
        static_assert(kScrPerStage * 16 * kScrLd * 4 <= kAStage * 2, "half the wave scratches per A stage");
        float* scr = reinterpret_cast<float*>(wave < kScrPerStage ? a_st0 : a_st1) +
                     (wave % kScrPerStage) * 16 * kScrLd;
#pragma unroll
        for (int i = 0; i < kFM; ++i) {
#pragma unroll
            for (int j = 0; j < kFN; ++j)
                *reinterpret_cast<f32x4*>(scr + scr_at(pl, 4 * j + g)) = acc[j][i];
#pragma unroll
            for (int h = 0; h < kPasses; ++h) {
                const int row = rr + kRpp * h;
                const f32x4 lo = *reinterpret_cast<const f32x4*>(scr + scr_at(row, 2 * cc));
                const f32x4 hi = *reinterpret_cast<const f32x4*>(scr + scr_at(row, 2 * cc + 1));
                const int64_t grow = m0 + wm0 + 16 * i + row;
                const float fr = EPI ? row_factor(p, grow) : alpha;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[e] = fr * (e < 4 ? lo[e] : hi[e - 4]);
                    if constexpr (EPI) v[e] = activate(v[e] * cf8[e] + bv8[e], p.act);
                }
                if (beta != 0.f) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[e] += beta * bf16_to_f32((uint16_t)(c0q[i][h][e >> 1] >> (16 * (e & 1))));
                }
                *reinterpret_cast<cvec*>(p.C + grow * p.ldc + gcol) =
                    u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7])};
            }
        }
        return;
    }
    }
    float bv[kFN][4], cv[kFN][4];
    if constexpr (EPI) {
#pragma unroll
        for (int j = 0; j < kFN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bv[j][r] = bias_at(p, n0 + wn0 + 16 * j + 4 * g + r);
                cv[j][r] = col_factor(p, n0 + wn0 + 16 * j + 4 * g + r);
            }
    }
    // With beta != 0 each lane loads all of its C values before its first
    // store. The stores could alias later loads, so the compiler would
    // otherwise wait out one memory round trip per 4 columns of a row. The
    // fragment registers are dead here, which leaves room for the 64 values.
    using cvec2 = std::conditional_t<DW, u32x2_a4, u32x2>;
    u32x2 cpre[kFM][kFN];
    if (beta != 0.f) {
#pragma unroll
        for (int i = 0; i < kFM; ++i) {
            const int64_t row = m0 + wm0 + 16 * i + pl;
#pragma unroll
            for (int j = 0; j < kFN; ++j) {
                const int64_t col = n0 + wn0 + 16 * j + 4 * g;
                cpre[i][j] = (row < M && col + 4 <= N)
                                 ? *reinterpret_cast<const cvec2*>(p.C + row * p.ldc + col)
                                 : u32x2{0u, 0u};
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
        const int64_t row = m0 + wm0 + 16 * i + pl;
        if (row >= M) continue;
        uint16_t* crow = p.C + row * p.ldc;
        const float fr = EPI ? row_factor(p, row) : alpha;
#pragma unroll
        for (int j = 0; j < kFN; ++j) {
            const int64_t col = n0 + wn0 + 16 * j + 4 * g;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = fr * acc[j][i][r];
            if constexpr (EPI) {
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = activate(v[r] * cv[j][r] + bv[j][r], p.act);
            }
            if (col + 4 <= N) {
                cvec2* dst = reinterpret_cast<cvec2*>(crow + col);
                if (beta != 0.f) {
                    const u32x2 c0 = cpre[i][j];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] += beta * bf16_to_f32((uint16_t)(c0[r >> 1] >> (16 * (r & 1))));
                }
                *dst = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
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
}

}  // namespace

// True when every buffer offset the tiled kernel forms fits in 31 bits: a
// k-contiguous tile spans 256 rows plus K elements, an m/n-contiguous slab 64
// rows plus its tile width (at least 256 elements).
bool bf16_tiled_fits(const GemmArgs<uint16_t>& a) {
    const int64_t lim = (int64_t)1 << 31;
    auto kc = [&](int64_t ld) { return (256 * ld + a.K) * 2 < lim; };
    auto mc = [&](int64_t ld, int64_t extent) { return (kBK * ld + 256 + extent) * 2 < lim; };
    return (a.ta ? mc(a.lda, a.M) : kc(a.lda)) && (a.tb ? kc(a.ldb) : mc(a.ldb, a.N));
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool EPI, bool SPLIT, bool DW, int KS = 1>
const void* pick_layout(bool ta, bool tb) {
#define DG_TILED(TA, TB) \
    (const void*)&gemm_bf16_tiled_kernel<BM, BN, WAVES_M, WAVES_N, EPI, TA, TB, SPLIT, DW, KS>
    return ta ? (tb ? DG_TILED(true, true) : DG_TILED(true, false))
              : (tb ? DG_TILED(false, true) : DG_TILED(false, false));
#undef DG_TILED
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool EPI, bool SPLIT, int KS = 1>
const void* pick_tiled(bool ta, bool tb, bool dw) {
    return dw ? pick_layout<BM, BN, WAVES_M, WAVES_N, EPI, SPLIT, true, KS>(ta, tb)
              : pick_layout<BM, BN, WAVES_M, WAVES_N, EPI, SPLIT, false, KS>(ta, tb);
}

// Three tile sizes: 256 x 256 (8 waves of 128 x 64, 128 KB of LDS, one
// workgroup per CU), 128 x 128 (8 waves of 64 x 32, 64 KB, two per CU; or,
// one per CU, 16 waves in two groups that split K, 128 KB: ks_preferred) and
// 64 x 64 (4 waves of 32 x 32, 32 KB, up to four per CU).
// The smaller tile multiplies less per byte it stages (4096^3: 127.5 against
// 103.3 us) but gives four times the workgroups, which products with few
// 256 x 256 tiles need (512 x 8192 x 8192: 64 such tiles, 162.2 us; 256 of
// 128 x 128, 79.7 us). Its 8 waves read 50% more LDS per MFMA than 4 waves of
// 64 x 64 would, but keep two waves on every SIMD even when a tile has its CU
// to itself: 512 x 8192 x 8192 ran 87.5 us with 4 waves, 2560^3 42.1 us
// against 40.1.
//
// The model, in units of one 256 x 256 tile's K loop on a CU: 256 x 256 tiles
// cost ceil(tiles / 256); a round of 128 x 128 tiles costs 0.61 with two per
// CU and 0.49 with at most one (the measured ratios above), so 4096^3 costs
// 1 against 1.22, 4352 x 4096 x 4096 (272 large tiles, two rounds) 2 against
// 1.71 (182.2 against 152.5 us), 3072^3 1 against 1.10 (67.3 against 76.5).
// 128 x 128 tiles run when they cost under 0.95 of the larger ones. Planned
// for a full MI355X (256 CUs) whatever the device, so the choice, and the
// rounding that follows from it, does not depend on partitioning.
//
// Among products that take 128 x 128 tiles, those with at most 160 of them
// (and no split over a workspace) run 64 x 64 tiles instead, unless the
// few-tile kernel takes them (below): four times the
// workgroups for four times the LDS reads per MFMA. Measured against 128 x
// 128 tiles: 1024^2 x 4096 (64 small tiles) 32.2 against 41.0 us, 1280^2 x
// 4096 (100) 33.1 against 44.1, 1536^2 x 4096 (144) 41.1 against 43.2,
// 1536 x 2048 x 4096 (192) 43.5 against 42.7, 2048^3 (256) 29.9 against 25.7.
// A round of 64 x 64 tiles costs about 0.385 + 0.07 (q - 1) at q tiles per CU,
// under the 0.49 of a lone round of 128 x 128 ones while q < 2.5.
constexpr int64_t kTilePlanCus = 256;

int tiled_tile(int64_t M, int64_t N) {
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    const double cost256 = (double)((t256 + kTilePlanCus - 1) / kTilePlanCus);
    const int64_t full = t128 / (2 * kTilePlanCus), rem = t128 % (2 * kTilePlanCus);
    const double cost128 = 0.61 * (double)full + (rem == 0 ? 0.0 : rem > kTilePlanCus ? 0.61 : 0.49);
    return cost128 < 0.95 * cost256 ? 128 : 256;
}

// Split K (with a workspace) for 128 x 128 tiles only, when they leave most
// CUs idle (fewer than half as many tiles as CUs, planned at one workgroup per
// CU: a second workgroup on a CU only shares its matrix cores). The model
// gives 256 x 256 tiles only to products with more than 128 of them, whose
// last round is more than half full, where a split measured slower (3072^2 x
// 8192's 144 tiles cut into 5 K ranges: 168 -> 231 us).
// Each K range spans at least 16 slabs (1024 k): every range stores an fp32
// partial tile and the tile's last range reads them all back, which only
// ranges with that much MFMA work to save pay for.
constexpr int kTiledMinSlabs = 16;
constexpr double kTiledFixupSlabs = -1.0;

TailSplit plan_tiled128(int64_t M, int64_t N, int64_t K, int cus) {
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    return plan_tail_split(tiles, (K + kBK - 1) / kBK, (int64_t)cus, kTiledMinSlabs, kTiledFixupSlabs);
}

// The few-tile kernel (gemm_bf16_few.hip: one 64 x 64 tile per workgroup, K
// split over its 4 waves, one workgroup per CU):
//   * without a split over a workspace, for up to two rounds of its tiles
//     (512 on a full MI355X), where the tiled kernel's 64 x 64 or 128 x 128
//     tiles would run (1024^2 x 4096: 18 against 32 us; 1280^2 x 4096, 400
//     tiles: 31.8 against 33.3; 1536^2 x 4096, 576 tiles: 45.8 against 40.5);
//     with 4-byte copies (dw) for one round only, as its four times as many
//     copy instructions make a second round cost more than the tiled
//     kernel's (1024^2 x 4096: 27.7 against 44.8 us; 1024 x 1536 x 4096,
//     384 tiles: 52.0 against 49.0);
//   * with one, when its tiles fit one round and are at least as many as the
//     split's workgroups (1024^2 x 4096: 256 tiles against 64 x 4 ranges,
//     18.3 against 24.1 us; 129 x 1000 x 8200: 48 against 16 x 8, 33.1
//     against 23.2 us; 384 x 1024 x 8192: 96 against 24 x 8, 27.5 against 24.0;
//     with 4-byte copies 1024^2 x 2048: 15.9 against 25.0 us, 1024^2 x 4096:
//     28.6 against 29.4, 1024^2 x 8192: 49.6 against 41.3); with K up to 4096
//     also when they are at least half as many (64 x 8192 x 4096: 128 tiles
//     against 64 x 4 ranges, 20.7 against 25.4 us; 48 x 8192 x 4096 20.0
//     against 25.0), where the split's ranges are short.
static bool few_preferred(int64_t M, int64_t N, int64_t K, const TailSplit* split, bool dw) {
    const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
    if (split != nullptr) {
        const int64_t wgs = (int64_t)split->tail * split->parts;
        return t64 <= kTilePlanCus && (t64 >= wgs || (K <= 4096 && 2 * t64 >= wgs));
    }
    return t64 <= (dw ? 1 : 2) * kTilePlanCus;
}

// 128 x 128 tiles with K split between two groups of 8 waves in each
// workgroup (KS = 2, 16 waves and 128 KB of LDS per CU): for products with at
// most one such tile per CU and an even number of at least 32 K slabs. A CU
// holding one tile of the plain kernel runs 8 waves, 2 per SIMD; two groups
// give it 4 per SIMD, as two workgroups per CU would, and the tile finishes in
// about half the slab steps. Measured (one MI355X, medians of 7): 512 x 8192 x
// 8192 87.0 -> 72.5 us, 2048^2 x 8192 86.7 -> 77.4, 1024 x 4096 x 4096 43.5
// -> 37.6, 1792 x 2048 x 8192 77.9 -> 66.7, 2048^2 x 2048 24.9 -> 23.2, but
// 2048^2 x 1024 (16 slabs) 12.5 -> 13.6. It also replaces 64 x 64 tiles for
// 129 .. 160 tiles of 128 x 128 (1536^2 x 4096 41.8 -> 36.6 us, 1536^2 x 8192
// 77.2 -> 64.0, with 4-byte rows 66.5 -> 53.2), not for fewer (with 4-byte
// rows 1280^2 x 4096, 100 tiles: 49.8 -> 53.1).
static bool ks_preferred(int64_t tiles128, int64_t K) {
    const int64_t nk = (K + kBK - 1) / kBK;
    return tiles128 <= kTilePlanCus && nk % 2 == 0 && nk >= 32;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool EPI>
hipError_t launch_cfg(const GemmArgs<uint16_t>& a, bool dw, void* ws, size_t ws_bytes, int cus,
                      hipStream_t s) {
    const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm = (int)tiles_m, tn = (int)tiles_n;
    GemmArgs<uint16_t> args = a;
    TailSplit ts = TailSplit{(int)(tiles_m * tiles_n), 0, 1, 0};
    bool split = false;
    if constexpr (BM == 128) {
        const TailSplit plan = plan_tiled128(a.M, a.N, a.K, cus);
        split = ws != nullptr && plan.tail > 0 && ws_bytes >= tail_workspace(plan, BM, BN);
        if (split) ts = plan;
    }
    unsigned char* wsp = split ? static_cast<unsigned char*>(ws) : nullptr;
    void* kargs[] = {&args, &tm, &tn, &ts, &wsp};
    // At most one 128 x 128 tile per CU and no split: two groups of 8 waves
    // share each tile's K (ks_preferred).
    int ks = 1;
    if constexpr (BM == 128)
        if (!split && ks_preferred(tiles_m * tiles_n, a.K)) ks = 2;
    const void* fn;
    if constexpr (BM == 128)
        fn = split ? pick_tiled<BM, BN, WAVES_M, WAVES_N, EPI, true>(a.ta, a.tb, dw)
             : ks == 2 ? pick_tiled<BM, BN, WAVES_M, WAVES_N, EPI, false, 2>(a.ta, a.tb, dw)
                       : pick_tiled<BM, BN, WAVES_M, WAVES_N, EPI, false>(a.ta, a.tb, dw);
    else
        fn = pick_tiled<BM, BN, WAVES_M, WAVES_N, EPI, false>(a.ta, a.tb, dw);
    const int64_t grid = split ? (int64_t)ts.full + (int64_t)ts.tail * ts.parts : tiles_m * tiles_n;
    if (grid > kMaxGrid) return hipErrorInvalidConfiguration;
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(ks * WAVES_M * WAVES_N * 64), kargs, 0, s);
}

// Modelled time of what launch_tiles (below) runs for an M x N product
// without a split, in rounds of 256 x 256 tiles at equal K: the few-tile
// kernel about 0.17 of such a round per round of its tiles (0.28 with 4-byte
// copies; 1024^2 x 4096: 17-18 and 27.7 us against about 100 for a round of
// 256 x 256 tiles), 64 x 64 tiles 0.385 + 0.07 (q - 1) at q per CU, 128 x 128
// tiles as in tiled_tile.
static double tiled_cost(int64_t M, int64_t N, bool dw) {
    const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
    if (tiled_tile(M, N) == 128) {
        if (few_preferred(M, N, 0, nullptr, dw))
            return (dw ? 0.28 : 0.17) * (double)((t64 + kTilePlanCus - 1) / kTilePlanCus);
        const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
        if (8 * t128 <= 5 * kTilePlanCus)
            return 0.385 + 0.07 * (double)((t64 + kTilePlanCus - 1) / kTilePlanCus - 1);
        const int64_t full = t128 / (2 * kTilePlanCus), rem = t128 % (2 * kTilePlanCus);
        return 0.61 * (double)full + (rem == 0 ? 0.0 : rem > kTilePlanCus ? 0.61 : 0.49);
    }
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    return (double)((t256 + kTilePlanCus - 1) / kTilePlanCus);
}

struct Bf16Partition {
    int by;            // 0: none; 1: columns [split, N) of C; 2: rows [split, M)
    int64_t split;
};

// Products with at least one whole round of 256 x 256 tiles and a partly full
// last one: the fewest trailing tile columns (or rows) that hold the last
// round's tiles run as a separate product (on the few-tile kernel when it is
// thin), leaving the tiled kernel whole rounds of 256 x 256 tiles, when the
// model puts the pair below 0.95 of the whole product as planned. Measured
// (one MI355X, medians of 7; model ratio in brackets): 4352 x 4096 x 4096
// 159.2 -> 128.6 us (0.68, a 256-row strip on the few-tile kernel),
// 4224 x 4096 x 4096 159.4 -> 119.2 (0.68), 4096 x 4608 x 4096 149.6 -> 131.8
// (0.78), 4500 x 4100 x 4096 218.3 -> 191.3 (0.87), 8448 x 8192 x 4096
// 469.1 -> 441.9 (0.87), 8192 x 12544 x 4096 671.5 -> 649.1 (0.91); with
// 4-byte rows 4352 x 4096 x 4096 219.5 -> 158.1 (0.75); but 5120^2 x 4096
// 186.0 -> 183.7 and 6144 x 4352 x 4096 185.2 -> 187.1 (both 1.0).
static Bf16Partition plan_bf16_partition(int64_t M, int64_t N, bool dw) {
    const Bf16Partition none{0, 0};
    const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256, tiles = tm * tn;
    const int64_t left = tiles % kTilePlanCus;
    if (tiles <= kTilePlanCus || left == 0) return none;
    const int64_t rn = (left + tm - 1) / tm, rm = (left + tn - 1) / tn;
    auto rounds = [](int64_t t) { return (double)((t + kTilePlanCus - 1) / kTilePlanCus); };
    const double cost_n = rn < tn ? rounds(tm * (tn - rn)) + tiled_cost(M, N - (tn - rn) * 256, dw) : 1e300;
    const double cost_m = rm < tm ? rounds((tm - rm) * tn) + tiled_cost(M - (tm - rm) * 256, N, dw) : 1e300;
    const bool by_cols = cost_n <= cost_m;
    if ((by_cols ? cost_n : cost_m) >= 0.95 * tiled_cost(M, N, dw)) return none;
    return by_cols ? Bf16Partition{1, (tn - rn) * 256} : Bf16Partition{2, (tm - rm) * 256};
}

static hipError_t launch_tiles(const GemmArgs<uint16_t>& a, bool dw, void* ws, size_t ws_bytes,
                               int cus, hipStream_t s);

hipError_t launch_bf16_tiled(const GemmArgs<uint16_t>& a, bool dw, void* ws, size_t ws_bytes,
                             int cus, hipStream_t s) {
    const Bf16Partition pt = plan_bf16_partition(a.M, a.N, dw);
    if (pt.by == 0) return launch_tiles(a, dw, ws, ws_bytes, cus, s);
    GemmArgs<uint16_t> head = a, strip = a;
    const int64_t k0 = pt.split;
    if (pt.by == 1) {                      // columns [k0, N) of C
        head.N = k0;
        strip.N = a.N - k0;
        strip.B = a.tb ? a.B + k0 * a.ldb : a.B + k0;
        strip.C = a.C + k0;
        if (a.bias != nullptr) strip.bias = a.bias + k0;
        if (a.col_scale != nullptr) strip.col_scale = a.col_scale + k0;
    } else {                               // rows [k0, M) of C
        head.M = k0;
        strip.M = a.M - k0;
        strip.A = a.ta ? a.A + k0 : a.A + k0 * a.lda;
        strip.C = a.C + k0 * a.ldc;
        if (a.row_scale != nullptr) strip.row_scale = a.row_scale + k0;
    }
    // Whole rounds: the head takes 256 x 256 tiles (tiled_tile picks them for
    // any product of whole rounds) and no split.
    const hipError_t e = launch_tiles(head, dw, nullptr, 0, cus, s);
    if (e != hipSuccess) return e;
    return launch_tiles(strip, dw, nullptr, 0, cus, s);
}

// Products that take 256 x 256 tiles in a single partly full round (129 ..
// 256 tiles) may instead run 128 x 128 tiles, two per CU, when a workspace
// lets the last round of those be split over K: 3072^3 has 144 large tiles,
// or 512 small ones for one full round and 64 more cut into 3 K ranges.
// Modelled in rounds of 256 x 256 tiles as in tiled_tile, the split ranges of
// the last round at a lone 128 x 128 tile's rate divided by the ranges.
// Measured (one MI355X, medians of 7, 256 x 256 tiles against the split):
// 3072^2 x 8192 165.1 -> 141.3 us, 3072^2 x 4096 90.3 -> 79.4, 2048 x 4608 x
// 4096 87.1 -> 78.0, 3072 x 3328 x 4096 90.6 -> 85.6, 3072^3 73.5 -> 69.1
// (A stored K x M: 70.4 -> 66.0; 4-byte rows: 99.6 -> 88.2). With B stored
// N x K the split ran slower (3072^3: 64.8 -> 90.2 us), so the launcher keeps
// such products on 256 x 256 tiles; the workspace query, which does not know
// the layout, still sizes the split for them.
static bool split128_preferred(int64_t M, int64_t N, int64_t K, int cus) {
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    if (t256 > kTilePlanCus || 2 * t256 <= kTilePlanCus) return false;
    const TailSplit plan = plan_tiled128(M, N, K, cus);
    if (plan.tail == 0) return false;
    const int64_t full = plan.full / (2 * kTilePlanCus), rem = plan.full % (2 * kTilePlanCus);
    const double head = 0.61 * (double)full + (rem == 0 ? 0.0 : rem > kTilePlanCus ? 0.61 : 0.49);
    const double tail = 0.49 * (double)plan.cps / (double)((K + kBK - 1) / kBK);
    return head + tail < 0.9;
}

static hipError_t launch_tiles(const GemmArgs<uint16_t>& a, bool dw, void* ws, size_t ws_bytes,
                               int cus, hipStream_t s) {
    if (ws != nullptr && !a.tb && tiled_tile(a.M, a.N) == 256 && split128_preferred(a.M, a.N, a.K, cus) &&
        ws_bytes >= tail_workspace(plan_tiled128(a.M, a.N, a.K, cus), 128, 128)) {
        if (has_epilogue(a)) return launch_cfg<128, 128, 2, 4, true>(a, dw, ws, ws_bytes, cus, s);
        return launch_cfg<128, 128, 2, 4, false>(a, dw, ws, ws_bytes, cus, s);
    }
    if (tiled_tile(a.M, a.N) == 128) {
        // At most 160 small tiles (on a full MI355X) and no split over a
        // workspace: 64 x 64 tiles.
        const int64_t t128 = ((a.M + 127) / 128) * ((a.N + 127) / 128);
        const TailSplit plan = plan_tiled128(a.M, a.N, a.K, cus);
        const bool split = ws != nullptr && plan.tail > 0 && ws_bytes >= tail_workspace(plan, 128, 128);
        if (few_preferred(a.M, a.N, a.K, split ? &plan : nullptr, dw)) return launch_bf16_few(a, dw, s);
        if (8 * t128 <= 5 * kTilePlanCus && !split && !(2 * t128 > kTilePlanCus && ks_preferred(t128, a.K))) {
            if (has_epilogue(a)) return launch_cfg<64, 64, 2, 2, true>(a, dw, ws, ws_bytes, cus, s);
            return launch_cfg<64, 64, 2, 2, false>(a, dw, ws, ws_bytes, cus, s);
        }
        if (has_epilogue(a)) return launch_cfg<128, 128, 2, 4, true>(a, dw, ws, ws_bytes, cus, s);
        return launch_cfg<128, 128, 2, 4, false>(a, dw, ws, ws_bytes, cus, s);
    }
    if (has_epilogue(a)) return launch_cfg<256, 256, 2, 4, true>(a, dw, ws, ws_bytes, cus, s);
    return launch_cfg<256, 256, 2, 4, false>(a, dw, ws, ws_bytes, cus, s);
}

size_t bf16_tiled_workspace(int64_t M, int64_t N, int64_t K, int cus) {
    if (M < 1 || N < 1 || K < 1) return 0;
    if (tiled_tile(M, N) == 256)
        return split128_preferred(M, N, K, cus) ? tail_workspace(plan_tiled128(M, N, K, cus), 128, 128) : 0;
    // A partitioned product (16-byte rows) runs no split.
    if (plan_bf16_partition(M, N, false).by != 0) return 0;
    const TailSplit plan = plan_tiled128(M, N, K, cus);
    // Products the few-tile kernel takes in preference to the split need no
    // workspace.
    if (plan.tail > 0 && few_preferred(M, N, K, &plan, false)) return 0;
    return tail_workspace(plan, 128, 128);
}

}  // namespace dg
