// fp32 GEMM on the vector ALUs (no matrix cores): the comparison kernel.
//
// This is the RTX 3090 SGEMM article's CUDA-core recipe carried to gfx950:
// 128 x 128 tiles of C per workgroup, K in slabs of 16 (section 3.2),
// 128-bit global loads (section 4), per-thread register micro-tiles with an
// unrolled k loop (sections 5.1-5.2) and a double-buffered LDS (section 5.3).
// Differences for CDNA4: 256 threads (four 64-wide waves) each own an 8 x 8
// micro-tile split into 2 x 2 blocks of 4 x 4 that sit 64 rows/columns apart,
// so a wave's LDS reads are 16 distinct 16-byte pieces (broadcast within the
// wave) rather than strided scalars; the A slab is stored transposed ([k][m])
// so each thread reads its 4 rows of A with one 128-bit LDS read.
// It uses plain fp32 fused multiply-adds only.

#include "common.hpp"
#include "kernels.hpp"

namespace dg {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 16, kNT = 256;
constexpr int kPadM = kBM + 4;   // transposed-A row length (keeps 16-byte alignment)
constexpr int kGroupM = 4;

template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float* p, int valid) {
    if (VEC && valid >= 4) return *reinterpret_cast<const f32x4*>(p);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < valid) v[e] = p[e];
    return v;
}

template <bool VEC>
__global__ __launch_bounds__(kNT)
void gemm_f32_valu_kernel(GemmArgs<float> p, int tiles_m, int tiles_n) {
    constexpr int STAGE = kBK * kPadM + kBK * kBN;
    __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, kGroupM, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int t = threadIdx.x, tx = t % 16, ty = t / 16;

    f32x4 ra[2], rb[2];
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {           // A: 128 rows x 4 chunks
            const int r = t / 4 + 64 * i, c = t % 4;
            const int64_t gm = m0 + r, gk = k0 + 4 * c;
            const int valid = (gm < M) ? (int)(K - gk < 4 ? K - gk : 4) : 0;
            ra[i] = valid > 0 ? load4<VEC>(p.A + gm * p.lda + gk, valid) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {           // B: 16 rows x 32 chunks
            const int kr = t / 32 + 8 * i, c = t % 32;
            const int64_t gk = k0 + kr, gn = n0 + 4 * c;
            const int valid = (gk < K) ? (int)(N - gn < 4 ? N - gn : 4) : 0;
            rb[i] = valid > 0 ? load4<VEC>(p.B + gk * p.ldb + gn, valid) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto sstore = [&](int stage) {
        float* As = smem + stage * STAGE;       // [k][m]
        float* Bs = As + kBK * kPadM;           // [k][n]
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = t / 4 + 64 * i, c = t % 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) As[(4 * c + e) * kPadM + r] = ra[i][e];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int kr = t / 32 + 8 * i, c = t % 32;
            *reinterpret_cast<f32x4*>(Bs + kr * kBN + 4 * c) = rb[i];
        }
    };

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    auto compute = [&](int stage) {
        const float* As = smem + stage * STAGE;
        const float* Bs = As + kBK * kPadM;
#pragma unroll
        for (int kk = 0; kk < kBK; ++kk) {
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(As + kk * kPadM + 4 * ty);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(As + kk * kPadM + 64 + 4 * ty);
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(Bs + kk * kBN + 4 * tx);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(Bs + kk * kBN + 64 + 4 * tx);
            float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
    };

    const int64_t nk = (K + kBK - 1) / kBK;
    // Poison build: stage 0 starts as NaN; the other stage is refilled with
    // NaN at the top of each slab, after the barrier that retired it.
    if constexpr (kLdsCheck == 1) lds_retire(smem, STAGE * 4, threadIdx.x, blockDim.x);
    gload(0);
    sstore(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kLdsCheck == 1 && kt + 1 < nk)
            lds_retire(smem + (cur ^ 1) * STAGE, STAGE * 4, threadIdx.x, blockDim.x);
        if (kt + 1 < nk) gload((kt + 1) * kBK);
        compute(cur);
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
        if (row >= M) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t col = n0 + 64 * h + 4 * tx;
            float* dst = p.C + row * p.ldc + col;
            f32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = alpha * acc[i][4 * h + j];
            if (VEC && col + 4 <= N) {
                if (beta != 0.f) {
                    const f32x4 c0 = *reinterpret_cast<const f32x4*>(dst);
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] += beta * c0[j];
                }
                *reinterpret_cast<f32x4*>(dst) = v;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (col + j < N) dst[j] = beta != 0.f ? v[j] + beta * dst[j] : v[j];
            }
        }
    }
}

}  // namespace

hipError_t launch_f32_valu(const GemmArgs<float>& a, bool vec, hipStream_t s) {
    const int64_t tiles_m = (a.M + kBM - 1) / kBM, tiles_n = (a.N + kBN - 1) / kBN;
    int tm = (int)tiles_m, tn = (int)tiles_n;
    GemmArgs<float> args = a;
    void* kargs[] = {&args, &tm, &tn};
    const void* fn = vec ? (const void*)&gemm_f32_valu_kernel<true>
                         : (const void*)&gemm_f32_valu_kernel<false>;
    if (tiles_m * tiles_n > kMaxGrid) return hipErrorInvalidConfiguration;
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n)), dim3(kNT), kargs, 0, s);
}

}  // namespace dg
