// Small-M bf16 GEMM (M <= 32): C = alpha * A * B + beta * C with fp32
// accumulation, for the inference shapes where a few rows of activations meet
// a large weight matrix. The Blackwell BF16 GEMM notes (section 5.2) point out
// that such GEMMs reuse almost nothing and are bound by reading B; the plan
// here is to stream B from HBM exactly once with wide loads and enough of it
// in flight, while the matrix cores do the little arithmetic there is.
//
//   * one workgroup (4 waves) per 32-column strip of C, covering all of K, so
//     no partial sums ever leave the workgroup; strips are renumbered so that
//     neighbouring strips (which share 128-byte lines of B) run on one XCD;
//   * K is walked in chunks of 512 rows. A chunk of B (512 x 32 bf16 = 32 KB)
//     is read with 128-bit loads, each thread taking one 8 x 8 block, and two
//     chunks are kept in flight in registers while the previous one is used;
//   * each block is transposed in registers and written k-contiguous to a
//     double-buffered LDS tile, from which v_mfma_f32_16x16x32_bf16 B
//     fragments are single 128-bit reads; A fragments (A is small and stays in
//     cache) are loaded straight from global memory;
//   * the four waves split each chunk's k range, and their fp32 partial tiles
//     are summed in LDS in a fixed order before the alpha/beta epilogue.

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

}  // namespace

hipError_t launch_bf16_skinny(const GemmArgs<uint16_t>& a, bool vec, hipStream_t s) {
    const int64_t strips = (a.N + kBN - 1) / kBN;
    int st = (int)strips;
    GemmArgs<uint16_t> args = a;
    void* kargs[] = {&args, &st};
    const void* fn;
    if (a.M <= 16)
        fn = vec ? (const void*)&gemm_bf16_skinny_kernel<1, true>
                 : (const void*)&gemm_bf16_skinny_kernel<1, false>;
    else
        fn = vec ? (const void*)&gemm_bf16_skinny_kernel<2, true>
                 : (const void*)&gemm_bf16_skinny_kernel<2, false>;
    return hipLaunchKernel(fn, dim3((unsigned)strips), dim3(kNT), kargs, 0, s);
}

}  // namespace dg
