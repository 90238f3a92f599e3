// Small-M bf16 GEMM (M <= 128): C = alpha * A * B + beta * C with fp32
// accumulation, for the inference shapes where a few rows of activations meet
// a large weight matrix. The Blackwell BF16 GEMM notes (section 5.2) point out
// that such GEMMs reuse almost nothing and are bound by reading B, so the aim
// is to stream B from HBM exactly once with enough of it in flight, while the
// matrix cores do the little arithmetic there is.
//
// Vector path (16-byte aligned rows): one workgroup (4 waves) per 64-column
// strip of C, or per strip and K segment when a workspace lets K be split.
// Chunks of 128 rows of B (and the matching 128 columns of A) are copied
// straight from global memory into a deep ring of LDS stages with
// LDS-destined buffer loads, several chunks ahead of their use. B stays
// row-major in LDS and its MFMA fragments come from transposing LDS reads
// (ds_read_b64_tr_b16); A's from 128-bit LDS reads. Rows past K and M arrive
// as zeros through the descriptor bounds; the ragged K tail of A is masked in
// registers.
//
// Transposed B (TB: B stored N x K, the layout of a weight matrix kept as
// [out][in]) takes the same vector kernel: a chunk is then 64 rows of B's
// storage (one per output column) times 128 k, copied and read the way A is.
//
// Element-wise path (any alignment): one workgroup per 32-column strip and
// all of K; 8 x 8 blocks of B are read with predicated loads, transposed in
// registers and written k-contiguous to a double-buffered LDS tile; A
// fragments are loaded from global memory. The four waves split each chunk's
// k range, and their fp32 partial tiles are summed in LDS in a fixed order
// before the epilogue.
//
// Both epilogues form alpha * acc + beta * C0 in fp32; with EPI the bias is
// added and the activation applied before the beta term.

#include "common.hpp"
#include "kernels.hpp"

namespace dg {
namespace {

constexpr int kNT = 256;         // 4 waves
constexpr int kBN = 32;          // columns per workgroup
constexpr int kKC = 512;         // k rows per chunk
constexpr int kKSteps = kKC / 32 / (kNT / 64);   // MFMA k-steps per wave per chunk

// Element offset of 16-byte chunk `c` (8 k values) of column `col` in a
// [kBN][kKC] LDS tile, XOR-swizzled within groups of 8 chunks.
__device__ __forceinline__ int bt_off(int col, int c) {
    return col * kKC + ((c ^ ((col ^ (col >> 3)) & 7)) << 3);
}

template <bool VEC>
__device__ __forceinline__ u32x4 load8(const uint16_t* p, int valid) {
    if (valid >= 8)
        return VEC ? *reinterpret_cast<const u32x4*>(p) : (u32x4)*reinterpret_cast<const u32x4_a2*>(p);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (e < valid) w[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
    return u32x4{w[0], w[1], w[2], w[3]};
}

template <int MB, bool VEC, bool EPI>
__global__ __launch_bounds__(kNT)
void gemm_bf16_skinny_kernel(GemmArgs<uint16_t> p, int strips) {
    __shared__ __attribute__((aligned(16))) uint16_t bt[2][kBN * kKC];
    __shared__ __attribute__((aligned(16))) float part[kNT / 64][MB * 16 * kBN];

    int tm, strip;
    tile_coords(blockIdx.x, gridDim.x, 1, strips, 1, tm, strip);
    const int64_t n0 = (int64_t)strip * kBN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int pl = lane & 15, g = lane >> 4;

    // This thread's 8 x 8 block of a chunk: rows 8 * kb .. + 7, columns 8 * cb .. + 7.
    const int kb = t / 4, cb = t % 4;
    const int64_t gn = n0 + 8 * cb;
    const int nvalid = (int)(N - gn >= 8 ? 8 : (N - gn > 0 ? N - gn : 0));

    u32x4 rb[2][8];
    bf16x8 ra[2][kKSteps][MB];

    auto gload = [&](int set, int64_t k0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t gk = k0 + 8 * kb + r;
            const int valid = gk < K ? nvalid : 0;
            rb[set][r] = load8<VEC>(p.B + (valid > 0 ? gk * p.ldb + gn : 0), valid);
        }
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int64_t row = 16 * mb + pl;
                const int64_t gk = k0 + 32 * (wave * kKSteps + s) + 8 * g;
                const int valid = row < M ? (int)(K - gk >= 8 ? 8 : (K - gk > 0 ? K - gk : 0)) : 0;
                const u32x4 v = load8<VEC>(p.A + (valid > 0 ? row * p.lda + gk : 0), valid);
                ra[set][s][mb] = __builtin_bit_cast(bf16x8, v);
            }
        }
    };

    auto sstore = [&](int set, int stage) {
        const u32x4 (&x)[8] = rb[set];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            u32x4 y;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = x[2 * q][j >> 1], hi = x[2 * q + 1][j >> 1];
                y[q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            *reinterpret_cast<u32x4*>(&bt[stage][bt_off(8 * cb + j, kb)]) = y;
        }
    };

    f32x4 acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb][0] = acc[mb][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int set, int stage) {
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
            const int c = 4 * (wave * kKSteps + s) + g;     // 16-byte chunk along k
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(&bt[stage][bt_off(16 * h + pl, c)]);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[set][s][mb], b, acc[mb][h], 0, 0, 0);
            }
        }
    };

    // Up to two chunks in flight: the loads of chunk c + 2 go out as soon as
    // chunk c has been consumed, while chunk c + 1 is still arriving. The loop
    // is unrolled by two so the register sets are fixed at compile time.
    // One barrier per chunk: stage s is rewritten two chunks after it was
    // read, and the barrier of the chunk in between separates the two.
    const int64_t nc = (K + kKC - 1) / kKC;
    // Poison build: both stages start as NaN, and each is refilled with NaN
    // after the barrier that retires it (a no-op in other builds).
    if constexpr (kLdsCheck == 1) {
        lds_retire(bt[0], kBN * kKC * 2, t, kNT);
        lds_retire(bt[1], kBN * kKC * 2, t, kNT);
    }
    gload(0, 0);
    if (nc > 1) gload(1, kKC);
    for (int64_t c = 0; c < nc; c += 2) {
        sstore(0, 0);
        __syncthreads();
        if (c > 0 && kLdsCheck == 1) lds_retire(bt[1], kBN * kKC * 2, t, kNT);
        compute(0, 0);
        if (c + 2 < nc) gload(0, (c + 2) * kKC);
        if (c + 1 < nc) {
            sstore(1, 1);
            __syncthreads();
            if (kLdsCheck == 1) lds_retire(bt[0], kBN * kKC * 2, t, kNT);
            compute(1, 1);
            if (c + 3 < nc) gload(1, (c + 3) * kKC);
        }
    }

    // Sum the four waves' partial tiles in a fixed order, then the epilogue.
    // Partial tile layout: part[wave][row * 32 + col].
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part[wave][(16 * mb + 4 * g + i) * kBN + 16 * h + pl] = acc[mb][h][i];
    __syncthreads();
    const float alpha = p.alpha, beta = p.beta;
    for (int e = t; e < MB * 16 * kBN; e += kNT) {
        const int row = e / kBN, col = e % kBN;
        const int64_t gc = n0 + col;
        if (row >= M || gc >= N) continue;
        float s = part[0][e];
#pragma unroll
        for (int w = 1; w < kNT / 64; ++w) s += part[w][e];
        float v = alpha * s;
        if constexpr (EPI)
            v = activate(row_factor(p, row) * col_factor(p, gc) * s + bias_at(p, gc), p.act);
        uint16_t* dst = p.C + row * p.ldc + gc;
        if (beta != 0.f) v += beta * bf16_to_f32(*dst);
        *dst = f32_to_bf16(v);
    }
}

// ---- vector path -------------------------------------------------------------
//
// Work is cut into units: a strip of 64 columns of C (one 128-byte line of
// every B row; a half line costs a whole line's worth of HBM bandwidth) times
// a segment of K made of whole 128-row chunks, one unit per workgroup.
// Without a workspace a unit is a whole strip. With one, K is cut into
// segments so that the units fill the chip; each workgroup stores its fp32
// partial tile in its unit's slot, and the last workgroup to finish a strip's
// segments (an atomic counter per strip) adds the slots in segment order and
// applies the epilogue.
//
// Wave w owns strip columns 16 w .. 16 w + 15 and all k of each chunk, so no
// partial sums cross waves.

constexpr int kVBN = 64;                 // strip width (columns)
constexpr int kVKC = 128;                // k rows per chunk
constexpr int kMaxWorkgroups = 256;      // one per compute unit
constexpr int kMaxSegments = 64;

// MB 16-row blocks of A (M <= 16 MB). The ring takes what LDS allows: 6, 5,
// 4 and 3 stages of 20, 24, 32 and 48 KB for MB = 1, 2, 4, 8.
template <int MB> struct SmallM {
    static constexpr int kBStage = kVKC * kVBN;           // bf16, [128][64] row-major
    static constexpr int kAStage = 16 * MB * kVKC;        // bf16, [16 MB][128]
    static constexpr int kStages = MB == 1 ? 6 : MB == 2 ? 5 : MB == 4 ? 4 : 3;
    static constexpr int kBCopies = kBStage * 2 / 1024 / (kNT / 64);   // 1 KB copies per wave
    static constexpr int kACopies = kAStage * 2 / 1024 / (kNT / 64);
    static constexpr int kCopies = kBCopies + kACopies;
};

// B stage rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r sits in
// slot c ^ b_swz(r), which spreads the 16 rows one transposing read touches
// over all LDS banks. A stage rows are 256 bytes; chunk c of row r sits in
// slot c ^ (r mod 16), spreading the 16 rows of a fragment read.
__device__ __forceinline__ int b_swz(int r) { return (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) << 1; }
__device__ __forceinline__ int a_off(int row, int c) { return row * kVKC + ((c ^ (row & 15)) << 3); }

// How the work is cut (identical on host and device): workgroup w takes
// segment w / strips of strip w % strips.
struct SmallMWork {
    int strips;   // 64-column strips
    int segs;     // K segments per strip (1: no split)
    int cps;      // chunks per segment
};

template <bool EPI>
__device__ __forceinline__ void store_row4(const GemmArgs<uint16_t>& p, int64_t row, int64_t gc,
                                           f32x4 s) {
    if (row >= p.M) return;
    if constexpr (EPI) {
        // Quantisation scales of the row and the columns, then bias and activation.
        const float fr = row_factor(p, row);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            s[r] = activate(fr * col_factor(p, gc + r) * s[r] + bias_at(p, gc + r), p.act);
    } else {
        s *= p.alpha;
    }
    uint16_t* dst = p.C + row * p.ldc + gc;
    if (gc + 3 < p.N) {
        // Four bf16 = 8 bytes, aligned: rows are 16-byte aligned and gc % 4 == 0.
        float v[4] = {s[0], s[1], s[2], s[3]};
        if (p.beta != 0.f) {
            const u32x2 c0 = *reinterpret_cast<const u32x2*>(dst);
            v[0] += p.beta * bf16_to_f32((uint16_t)(c0[0] & 0xffffu));
            v[1] += p.beta * bf16_to_f32((uint16_t)(c0[0] >> 16));
            v[2] += p.beta * bf16_to_f32((uint16_t)(c0[1] & 0xffffu));
            v[3] += p.beta * bf16_to_f32((uint16_t)(c0[1] >> 16));
        }
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (gc + r >= p.N) break;
            float v = s[r];
            if (p.beta != 0.f) v += p.beta * bf16_to_f32(dst[r]);
            dst[r] = f32_to_bf16(v);
        }
    }
}

// ws (only used when wk.segs > 1): [counters: one int per strip, padded to
// 256 bytes][slots: segs x strips tiles of 16 MB x 64 fp32, slot s * strips + strip].
template <int MB, bool EPI, bool TB>
__global__ __launch_bounds__(kNT, 1)
void gemm_bf16_smallm_kernel(GemmArgs<uint16_t> p, SmallMWork wk, unsigned char* ws) {
    using S = SmallM<MB>;
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[S::kStages * S::kBStage];
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[S::kStages * S::kAStage];
    __shared__ int last_flag;

    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int pl = lane & 15, g = lane >> 4;
    const int seg = __builtin_amdgcn_readfirstlane((int)blockIdx.x / wk.strips);
    const int strip = __builtin_amdgcn_readfirstlane((int)blockIdx.x - seg * wk.strips);
    const int64_t n0 = (int64_t)strip * kVBN;
    const int64_t nck = (K + kVKC - 1) / kVKC;
    const int64_t cb = (int64_t)seg * wk.cps;
    const int64_t nc = (cb + wk.cps < nck ? cb + wk.cps : nck) - cb;   // >= 1

    // A descriptor: rows 0 .. M - 1, ending at element K of the last row
    // (rounded up to its 16-byte chunk), so rows past M arrive as zeros.
    const uint32_t a_bytes = (uint32_t)((((M - 1) * lda + K) * 2 + 15) & ~(int64_t)15);
    const rsrc_t a_desc = make_rsrc(p.A, a_bytes);
    // Transposed B: rows n0 .. min(N, n0 + 64) - 1 of the N x K storage, the
    // same way (dead code without TB).
    const int64_t rows_bt = N - n0 < kVBN ? N - n0 : kVBN;
    const uint32_t bt_bytes = (uint32_t)((((rows_bt - 1) * ldb + K) * 2 + 15) & ~(int64_t)15);
    const rsrc_t bt_desc = make_rsrc(p.B + n0 * ldb, bt_bytes);

    // Copies are 1 KB; lane l fills bytes [16 l, 16 l + 16) of the slot, and
    // each copy's whole offset sits in the per-lane offset, which the
    // descriptor's range check covers.
    //   B: copy I fills chunk rows 8 I .. 8 I + 7; lane -> row 8 I + l / 8,
    //      slot l % 8 holding 16-byte chunk (l % 8) ^ b_swz(row).
    //   A: copy J fills rows 4 J .. 4 J + 3; lane -> row 4 J + l / 16, slot
    //      l % 16 holding chunk (l % 16) ^ (row % 16).
    //   Transposed B ([64 n][128 k] chunks): as A.
    auto dma = [&](int64_t chunk, int stage) {
        const int64_t k0 = chunk * kVKC;
        const uint32_t Bs = lds_addr(lds_b + stage * S::kBStage);
        const uint32_t As = lds_addr(lds_a + stage * S::kAStage);
        if constexpr (TB) {
#pragma unroll
            for (int i = 0; i < S::kBCopies; ++i) {
                const int J = wave * S::kBCopies + i;
                const int row = 4 * J + (lane >> 4);
                const int c = (lane & 15) ^ (row & 15);
                dma16(bt_desc, (uint32_t)((row * ldb + k0 + c * 8) * 2), 0, Bs + J * 1024);
            }
        } else {
            const int64_t rem = (((K - k0 - 1) * ldb + (N - n0)) * 2 + 15) & ~(int64_t)15;
            const uint32_t b_bytes = rem < ((int64_t)1 << 31) ? (uint32_t)rem : 0x80000000u;
            const rsrc_t b_desc = make_rsrc(p.B + k0 * ldb + n0, b_bytes);
#pragma unroll
            for (int i = 0; i < S::kBCopies; ++i) {
                const int I = wave * S::kBCopies + i;
                const int row = 8 * I + (lane >> 3);
                const int c = (lane & 7) ^ b_swz(row);
                dma16(b_desc, (uint32_t)(row * ldb * 2 + c * 16), 0, Bs + I * 1024);
            }
        }
#pragma unroll
        for (int i = 0; i < S::kACopies; ++i) {
            const int J = wave * S::kACopies + i;
            const int row = 4 * J + (lane >> 4);
            const int c = (lane & 15) ^ (row & 15);
            dma16(a_desc, (uint32_t)((row * lda + k0 + c * 8) * 2), 0, As + J * 1024);
        }
    };

    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    // Transposing-read role: lane 4 r + q of a 16-lane group addresses 4
    // consecutive columns (4 q ..) of row r of a 4 x 16 block.
    const int tr_row = pl >> 2, tr_c = 2 * wave + ((pl >> 1) & 1), tr_in = (pl & 1) * 4;
    auto compute = [&](int64_t chunk, int stage) {
        const uint16_t* Bs = lds_b + stage * S::kBStage;
        const uint16_t* As = lds_a + stage * S::kAStage;
#pragma unroll
        for (int ks = 0; ks < kVKC / 32; ++ks) {
            bf16x8 fa[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                fa[mb] = *reinterpret_cast<const bf16x8*>(As + a_off(16 * mb + pl, 4 * ks + g));
            bf16x8 fb;
            if constexpr (TB) {
                // B(k = 32 ks + 8 g .. + 7, n = 16 wave + pl): one 128-bit read of row n.
                fb = *reinterpret_cast<const bf16x8*>(Bs + a_off(16 * wave + pl, 4 * ks + g));
            } else {
                // Rows 32 ks + 8 g + tr_row and 4 further down; columns 16 wave + 4 q.
                const int r0 = 32 * ks + 8 * g + tr_row, r1 = r0 + 4;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(Bs + r0 * kVBN + ((tr_c ^ b_swz(r0)) << 3) + tr_in));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4*)(Bs + r1 * kVBN + ((tr_c ^ b_swz(r1)) << 3) + tr_in));
                fb = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            const int64_t kfirst = chunk * kVKC + 32 * ks + 8 * g;   // k of this lane's first element
            if (kfirst + 8 > K) {
                // Ragged K: A(m, k >= K) holds the next row's values, and so
                // does a transposed B(k >= K, n).
                const int valid = kfirst >= K ? 0 : (int)(K - kfirst);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    fa[mb] = __builtin_bit_cast(bf16x8, mask_tail(__builtin_bit_cast(u32x4, fa[mb]), valid));
                if constexpr (TB) fb = __builtin_bit_cast(bf16x8, mask_tail(__builtin_bit_cast(u32x4, fb), valid));
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fa[mb], acc[mb], 0, 0, 0);
        }
    };

    // Ring of kStages chunk slots; copies run kStages - 1 chunks ahead. At
    // chunk c each wave waits for its own copies of chunk c (later ones may
    // stay in flight), then the barrier publishes chunk c and retires all
    // reads of chunk c - 1, whose slot the copy for chunk c + kStages - 1 reuses.
    //
    // With a transposed B, the strips' row blocks lie 64 rows (1 MB at
    // K = 8192) apart, so strips walking their chunks in step would all read
    // at the same offset within their rows. Each group of 8 strips (one per
    // XCD) therefore starts its segment one chunk later than the group
    // before, wrapping around: measured 36.6 -> 29.2 us at 16 x 8192 x 8192.
    // Row-major B reads contiguous rows across strips and keeps the plain
    // order (a rotation measured slower there).
    const int64_t rot = TB ? (int64_t)(strip >> 3) % nc : 0;
    auto rc = [&](int64_t c) { return cb + (c + rot >= nc ? c + rot - nc : c + rot); };
    // Checking builds (no-ops otherwise): every slot starts as NaN and is
    // refilled with NaN once retired (poison); copies are bracketed by
    // barriers (synchronous copies).
    auto retire = [&](int slot) {
        if constexpr (kLdsCheck == 1) {
            lds_retire(lds_b + slot * S::kBStage, S::kBStage * 2, t, kNT);
            lds_retire(lds_a + slot * S::kAStage, S::kAStage * 2, t, kNT);
        }
    };
    for (int slot = 0; slot < S::kStages; ++slot) retire(slot);
    const int64_t pre = nc < S::kStages - 1 ? nc : S::kStages - 1;
    for (int64_t c = 0; c < pre; ++c) {
        copy_begin();
        dma(rc(c), (int)c);
        copy_end();
    }
    int stage = 0;
    for (int64_t c = 0; c < nc; ++c) {
        if (c + S::kStages - 2 <= nc - 1)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((S::kStages - 2) * S::kCopies));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        lds_only_barrier();
        const int prev = stage == 0 ? S::kStages - 1 : stage - 1;   // slot of chunk c - 1, retired
        if (c > 0) retire(prev);
        if (c + S::kStages - 1 < nc) {
            copy_begin();
            dma(rc(c + S::kStages - 1), prev);
            copy_end();
        }
        compute(rc(c), stage);
        stage = stage + 1 == S::kStages ? 0 : stage + 1;
    }

    // acc[mb] register r holds C(16 mb + pl, n0 + 16 wave + 4 g + r).
    const int tcol = 16 * wave + 4 * g;
    if (wk.segs == 1) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) store_row4<EPI>(p, 16 * mb + pl, n0 + tcol, acc[mb]);
        return;
    }

    // Split K: store the partial tile to this unit's slot, count in once the
    // stores have completed, and let a strip's last arrival add its segments
    // in order. Slots and counters are only touched through agent-scope
    // atomics (device-coherent accesses that bypass the per-XCD L2's
    // write-back caching), so no cache write-back or invalidate is needed.
    int* counters = reinterpret_cast<int*>(ws);
    float* slots = reinterpret_cast<float*>(ws + (((int64_t)wk.strips * 4 + 255) & ~(int64_t)255));
    auto slot = [&](int sg, int mb) {
        return slots + ((int64_t)sg * wk.strips + strip) * (16 * MB * kVBN) + (16 * mb + pl) * kVBN + tcol;
    };
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        float* dst = slot(seg, mb);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            __hip_atomic_store(dst + r, acc[mb][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (t == 0)
        last_flag = __hip_atomic_fetch_add(counters + strip, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    wk.segs - 1;
    __syncthreads();
    if (!last_flag) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        // Eight slots' loads in flight at a time; the sum runs in segment order.
        f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int sg0 = 0; sg0 < wk.segs; sg0 += 8) {
            f32x4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[i] = acc[mb];
                if (sg0 + i < wk.segs && sg0 + i != seg) {
                    const float* src = slot(sg0 + i, mb);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[i][r] = __hip_atomic_load(src + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (sg0 + i < wk.segs) sum += v[i];
        }
        store_row4<EPI>(p, 16 * mb + pl, n0 + tcol, sum);
    }
    // Leave the counter at zero for the next call that uses this workspace.
    if (t == 0) __hip_atomic_store(counters + strip, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// Work decomposition of the vector small-M kernel: 64-column strips; with a
// workspace and fewer strips than compute units, K segments (whole chunks,
// every segment non-empty) so that strips x segments fills the chip.
static SmallMWork plan_smallm(int64_t N, int64_t K, bool split) {
    SmallMWork w;
    w.strips = (int)((N + kVBN - 1) / kVBN);
    const int64_t nck = (K + kVKC - 1) / kVKC;
    int64_t segs = 1;
    if (split && w.strips < kMaxWorkgroups) {
        segs = (kMaxWorkgroups + w.strips - 1) / w.strips;
        if (segs > kMaxSegments) segs = kMaxSegments;
        if (segs > nck) segs = nck;
    }
    w.cps = (int)((nck + segs - 1) / segs);
    w.segs = (int)((nck + w.cps - 1) / w.cps);
    return w;
}

// Row blocks of 16 for M rows: 1, 2, 4 or 8.
static int smallm_blocks(int64_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8; }

// True when every buffer offset the vector kernel forms fits in 31 bits: A
// copies reach row 16 MB - 1 (rows past M included) and one chunk past K; B
// copies reach 128 rows below a chunk's first row, or with a transposed B row
// 63 of the strip and one chunk past K.
static bool smallm_fits(const GemmArgs<uint16_t>& a) {
    const int64_t lim = (int64_t)1 << 31;
    const bool b_ok = a.tb ? (kVBN * a.ldb + a.K + kVKC) * 2 < lim : (kVKC * a.ldb + a.N) * 2 < lim;
    return (16 * smallm_blocks(a.M) * a.lda + a.K + kVKC) * 2 < lim && b_ok;
}

// Workspace of the 64-column kernel's split.
static size_t smallm_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > kSkinnyMaxM || N < 1 || K < 1) return 0;
    const SmallMWork w = plan_smallm(N, K, true);
    if (w.segs < 2) return 0;
    const int64_t mb = smallm_blocks(M);
    return (size_t)((((int64_t)w.strips * 4 + 255) & ~(int64_t)255) +
                    (int64_t)w.segs * w.strips * 16 * mb * kVBN * 4);
}

// The larger of the two small-M splits: the streaming kernel takes row-major
// B, the 64-column kernel a transposed B (and shapes the streaming one does
// not cover).
size_t bf16_skinny_workspace(int64_t M, int64_t N, int64_t K) {
    const size_t a = smallm_workspace(M, N, K), b = bf16_stream_workspace(M, N, K);
    return a > b ? a : b;
}

hipError_t launch_bf16_skinny(const GemmArgs<uint16_t>& a, bool vec, void* ws, size_t ws_bytes,
                              int cus, hipStream_t s) {
    GemmArgs<uint16_t> args = a;
    const bool epi = has_epilogue(a);
    // A transposed B, and M > kSkinnyElemMaxM, are handled by the vector
    // kernel only; otherwise the tiled kernels take the call.
    if ((a.tb || a.M > kSkinnyElemMaxM) && !(vec && smallm_fits(a)))
        return launch_bf16_mfma(a, vec, ws, ws_bytes, cus, s);
    if (vec && !a.tb && ws != nullptr && plan_stream(a.N, a.K).phases > 0 &&
        ws_bytes >= bf16_stream_workspace(a.M, a.N, a.K) && bf16_stream_fits(a))
        return launch_bf16_stream(a, ws, s);
    if (vec && smallm_fits(a)) {
        const size_t need = smallm_workspace(a.M, a.N, a.K);
        const bool split = ws != nullptr && need > 0 && ws_bytes >= need;
        SmallMWork w = plan_smallm(a.N, a.K, split);
        unsigned char* wsp = split ? static_cast<unsigned char*>(ws) : nullptr;
        void* kargs[] = {&args, &w, &wsp};
#define DG_SMALLM(MB, EPI) (a.tb ? (const void*)&gemm_bf16_smallm_kernel<MB, EPI, true> \
                              : (const void*)&gemm_bf16_smallm_kernel<MB, EPI, false>)
        const int mb = smallm_blocks(a.M);
        const void* fn = epi ? (mb == 1 ? DG_SMALLM(1, true) : mb == 2 ? DG_SMALLM(2, true)
                                : mb == 4 ? DG_SMALLM(4, true) : DG_SMALLM(8, true))
                             : (mb == 1 ? DG_SMALLM(1, false) : mb == 2 ? DG_SMALLM(2, false)
                                : mb == 4 ? DG_SMALLM(4, false) : DG_SMALLM(8, false));
#undef DG_SMALLM
        if ((int64_t)w.strips * w.segs > kMaxGrid) return hipErrorInvalidConfiguration;
        return hipLaunchKernel(fn, dim3((unsigned)(w.strips * w.segs)), dim3(kNT), kargs, 0, s);
    }
    const int64_t strips = (a.N + kBN - 1) / kBN;
    int st = (int)strips;
    void* kargs[] = {&args, &st};
    const void* fn =
        epi ? (a.M <= 16 ? (vec ? (const void*)&gemm_bf16_skinny_kernel<1, true, true>
                                : (const void*)&gemm_bf16_skinny_kernel<1, false, true>)
                         : (vec ? (const void*)&gemm_bf16_skinny_kernel<2, true, true>
                                : (const void*)&gemm_bf16_skinny_kernel<2, false, true>))
            : (a.M <= 16 ? (vec ? (const void*)&gemm_bf16_skinny_kernel<1, true, false>
                                : (const void*)&gemm_bf16_skinny_kernel<1, false, false>)
                         : (vec ? (const void*)&gemm_bf16_skinny_kernel<2, true, false>
                                : (const void*)&gemm_bf16_skinny_kernel<2, false, false>));
    if (strips > kMaxGrid) return hipErrorInvalidConfiguration;
    return hipLaunchKernel(fn, dim3((unsigned)strips), dim3(kNT), kargs, 0, s);
}

}  // namespace dg
