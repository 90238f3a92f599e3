// Small-M bf16 GEMM (M <= 32): C = alpha * A * B + beta * C with fp32
// accumulation, for the inference shapes where a few rows of activations meet
// a large weight matrix. The Blackwell BF16 GEMM notes (section 5.2) point out
// that such GEMMs reuse almost nothing and are bound by reading B, so the aim
// is to stream B from HBM exactly once with enough of it in flight, while the
// matrix cores do the little arithmetic there is.
//
// Both kernels here give one workgroup (4 waves) a 32-column strip of C and
// all of K, so no partial sums ever leave the workgroup; strips are renumbered
// so that neighbouring strips (which share 128-byte lines of B) run on one
// XCD. The four waves split each chunk's k range, and their fp32 partial tiles
// are summed in LDS in a fixed order before the alpha/beta epilogue.
//
// Vector path (16-byte aligned rows): chunks of 256 rows of B (and the
// matching 256 columns of A) are copied straight from global memory into a
// deep ring of LDS stages with LDS-destined buffer loads, five chunks ahead
// of their use. B stays row-major in LDS and its MFMA fragments come from
// transposing LDS reads (ds_read_b64_tr_b16); A's from 128-bit LDS reads.
// Rows past K and M arrive as zeros through the descriptor bounds; the
// ragged K tail of A is masked in registers.
//
// Element-wise path (any alignment): 8 x 8 blocks of B are read with
// predicated loads, transposed in registers and written k-contiguous to a
// double-buffered LDS tile; A fragments are loaded from global memory.

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
    if (VEC && valid >= 8) return *reinterpret_cast<const u32x4*>(p);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (e < valid) w[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
    return u32x4{w[0], w[1], w[2], w[3]};
}

template <int MB, bool VEC>
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
    gload(0, 0);
    if (nc > 1) gload(1, kKC);
    for (int64_t c = 0; c < nc; c += 2) {
        sstore(0, 0);
        __syncthreads();
        compute(0, 0);
        if (c + 2 < nc) gload(0, (c + 2) * kKC);
        if (c + 1 < nc) {
            sstore(1, 1);
            __syncthreads();
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
        uint16_t* dst = p.C + row * p.ldc + gc;
        if (beta != 0.f) v += beta * bf16_to_f32(*dst);
        *dst = f32_to_bf16(v);
    }
}

// ---- vector path -------------------------------------------------------------

constexpr int kDmaKC = 256;                       // k rows per chunk
template <int MB> struct SmallMDma {
    static constexpr int kBStage = kDmaKC * kBN;          // bf16, [256][32] row-major
    static constexpr int kAStage = 16 * MB * kDmaKC;      // bf16, [16 MB][256]
    static constexpr int kStages = MB == 1 ? 6 : 4;       // 144 / 128 KB of ring
    static constexpr int kBCopies = kBStage * 2 / 1024 / (kNT / 64);   // per wave per chunk
    static constexpr int kACopies = kAStage * 2 / 1024 / (kNT / 64);
    static constexpr int kCopies = kBCopies + kACopies;
    static constexpr int kSteps = kDmaKC / 32 / (kNT / 64);            // k-steps per wave per chunk
};

// A stage row of 256 bf16 = 32 chunks of 16 bytes, XORed with row mod 16 so
// the 16 rows of an MFMA fragment read land on distinct banks.
__device__ __forceinline__ int sa_off(int row, int c) {
    return row * kDmaKC + ((c ^ (row & 15)) << 3);
}

template <int MB>
__global__ __launch_bounds__(kNT, 1)
void gemm_bf16_skinny_dma_kernel(GemmArgs<uint16_t> p, int strips) {
    using S = SmallMDma<MB>;
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[S::kStages * S::kBStage];
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[S::kStages * S::kAStage];
    __shared__ __attribute__((aligned(16))) float part[kNT / 64][MB * 16 * kBN];

    int tm, strip;
    tile_coords(blockIdx.x, gridDim.x, 1, strips, 1, tm, strip);
    const int64_t n0 = (int64_t)strip * kBN;
    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int pl = lane & 15, g = lane >> 4;

    // A descriptor covers rows 0 .. M - 1 up to element K of the last row
    // (rounded up to its 16-byte chunk), so rows past M arrive as zeros.
    const uint32_t a_bytes = (uint32_t)((((M - 1) * lda + K) * 2 + 15) & ~(int64_t)15);
    const rsrc_t a_desc = make_rsrc(p.A, a_bytes);

    // The whole offset of every copy goes in the per-lane offset, which the
    // descriptor's range check always covers.
    // Copies (1 KB each; lane l fills bytes [16 l, 16 l + 16) of the slot):
    //   B: copy I fills chunk rows 16 I .. 16 I + 15 (64 bytes each); lane ->
    //      row 16 I + l / 4, 16-byte column block l % 4.
    //   A: copy J fills rows 2 J, 2 J + 1 (512 bytes each); lane -> row
    //      2 J + l / 32, slot l % 32 holding global chunk (l % 32) ^ (row % 16).
    const uint32_t b_voff = (uint32_t)(((lane >> 2) * ldb + (lane & 3) * 8) * 2);
    auto dma = [&](int64_t chunk, int stage) {
        const int64_t k0 = chunk * kDmaKC;
        const int64_t rem = (((K - k0 - 1) * ldb + (N - n0)) * 2 + 15) & ~(int64_t)15;
        const uint32_t b_bytes = rem < ((int64_t)1 << 31) ? (uint32_t)rem : 0x80000000u;
        const rsrc_t b_desc = make_rsrc(p.B + k0 * ldb + n0, b_bytes);
        const uint32_t Bs = lds_addr(lds_b + stage * S::kBStage);
        const uint32_t As = lds_addr(lds_a + stage * S::kAStage);
#pragma unroll
        for (int i = 0; i < S::kBCopies; ++i) {
            const int I = wave * S::kBCopies + i;
            dma16(b_desc, b_voff + (uint32_t)(16 * I * ldb * 2), 0, Bs + I * 1024);
        }
#pragma unroll
        for (int i = 0; i < S::kACopies; ++i) {
            const int J = wave * S::kACopies + i;
            const int row = 2 * J + (lane >> 5);
            const int c = (lane & 31) ^ (row & 15);
            dma16(a_desc, (uint32_t)(((row * lda + k0) + c * 8) * 2), 0, As + J * 1024);
        }
    };

    f32x4 acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb][0] = acc[mb][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int tr_row = pl >> 2, tr_col = (pl & 3) * 4;   // transposing-read role of this lane
    const int64_t nc = (K + kDmaKC - 1) / kDmaKC;
    auto compute = [&](int64_t chunk, int stage) {
        const uint16_t* Bs = lds_b + stage * S::kBStage;
        const uint16_t* As = lds_a + stage * S::kAStage;
#pragma unroll
        for (int s = 0; s < S::kSteps; ++s) {
            const int ks = wave * S::kSteps + s;                // k-step (32 k) within the chunk
            bf16x8 fa[MB], fb[2];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                fa[mb] = *reinterpret_cast<const bf16x8*>(As + sa_off(16 * mb + pl, 4 * ks + g));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint16_t* q = Bs + (32 * ks + 8 * g + tr_row) * kBN + 16 * h + tr_col;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)q);
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 4 * kBN));
                fb[h] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            const int64_t kfirst = chunk * kDmaKC + 32 * ks + 8 * g;   // k of this lane's first element
            if (kfirst + 8 > K) {
                // Ragged K: A(m, k >= K) holds the next row's values.
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    fa[mb] = __builtin_bit_cast(
                        bf16x8, mask_tail(__builtin_bit_cast(u32x4, fa[mb]), (int)(K - kfirst)));
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    acc[mb][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[h], fa[mb], acc[mb][h], 0, 0, 0);
        }
    };

    // Ring of kStages chunk slots; copies run kStages - 1 chunks ahead. At
    // chunk c each wave waits for its own copies of chunk c (the later ones
    // may stay in flight), then the barrier publishes chunk c and retires all
    // reads of chunk c - 1, whose slot the copy for chunk c + kStages - 1 reuses.
    const int64_t pre = nc < S::kStages - 1 ? nc : S::kStages - 1;
    for (int64_t c = 0; c < pre; ++c) dma(c, (int)c);
    int stage = 0;
    for (int64_t c = 0; c < nc; ++c) {
        if (c + S::kStages - 2 <= nc - 1)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((S::kStages - 2) * S::kCopies));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        lds_only_barrier();
        if (c + S::kStages - 1 < nc) dma(c + S::kStages - 1, stage == 0 ? S::kStages - 1 : stage - 1);
        compute(c, stage);
        stage = stage + 1 == S::kStages ? 0 : stage + 1;
    }

    // Sum the four waves' partial tiles in a fixed order, then the epilogue.
    // acc[mb][h] register r holds C(16 mb + pl, 16 h + 4 g + r) of the strip.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                part[wave][(16 * mb + pl) * kBN + 16 * h + 4 * g + r] = acc[mb][h][r];
    __syncthreads();
    const float alpha = p.alpha, beta = p.beta;
    for (int e = t; e < MB * 16 * kBN; e += kNT) {
        const int row = e / kBN, col = e % kBN;
        const int64_t gc = n0 + col;
        if (row >= M || gc >= N) continue;
        float sum = part[0][e];
#pragma unroll
        for (int w = 1; w < kNT / 64; ++w) sum += part[w][e];
        float v = alpha * sum;
        uint16_t* dst = p.C + row * p.ldc + gc;
        if (beta != 0.f) v += beta * bf16_to_f32(*dst);
        *dst = f32_to_bf16(v);
    }
}

}  // namespace

// True when every buffer offset the vector kernel forms fits in 31 bits: A
// copies reach row 31 (rows past M included) and one chunk past K; B copies
// reach 256 rows below a chunk's first row.
static bool skinny_dma_fits(const GemmArgs<uint16_t>& a) {
    const int64_t lim = (int64_t)1 << 31;
    return (32 * a.lda + a.K + kDmaKC) * 2 < lim && (kDmaKC * a.ldb + a.N) * 2 < lim;
}

hipError_t launch_bf16_skinny(const GemmArgs<uint16_t>& a, bool vec, hipStream_t s) {
    const int64_t strips = (a.N + kBN - 1) / kBN;
    int st = (int)strips;
    GemmArgs<uint16_t> args = a;
    void* kargs[] = {&args, &st};
    const void* fn;
    if (vec && skinny_dma_fits(a))
        fn = a.M <= 16 ? (const void*)&gemm_bf16_skinny_dma_kernel<1>
                       : (const void*)&gemm_bf16_skinny_dma_kernel<2>;
    else if (a.M <= 16)
        fn = vec ? (const void*)&gemm_bf16_skinny_kernel<1, true>
                 : (const void*)&gemm_bf16_skinny_kernel<1, false>;
    else
        fn = vec ? (const void*)&gemm_bf16_skinny_kernel<2, true>
                 : (const void*)&gemm_bf16_skinny_kernel<2, false>;
    return hipLaunchKernel(fn, dim3((unsigned)strips), dim3(kNT), kargs, 0, s);
}

}  // namespace dg
