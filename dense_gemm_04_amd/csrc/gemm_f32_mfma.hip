// fp32 GEMM (SGEMM) on gfx950 matrix cores: C = alpha * A * B + beta * C,
// row-major, fp32 products and fp32 accumulation (v_mfma_f32_16x16x4_f32).
//
// The RTX 3090 SGEMM article builds its 10.23 TFLOPS kernel from shared-memory
// tiles (section 3), float4 loads (section 4), register accumulators and
// double buffering (section 5). The same ideas are kept here, but the inner
// product runs on the fp32 matrix cores instead of per-thread FMAs:
//   * one workgroup per BM x BN tile of C, renumbered per XCD;
//   * K in slabs of BK = 32; the A slab (BM x 32) is stored [row][k] and the
//     B slab (32 x BN) [k][col] in a double-buffered LDS, loaded with 128-bit
//     global loads one slab ahead (one barrier per slab);
//   * A rows are 8 chunks of 4 floats with an XOR-swizzled chunk position, so
//     the 128-bit fragment reads of a wave are bank-conflict free;
//   * each lane reads 4 consecutive k of A with one 128-bit LDS read and uses
//     them in 4 successive MFMAs; the matching B values are one 128-bit read
//     of 4 consecutive columns at that k, which feed 4 MFMA blocks whose
//     columns are interleaved (block j covers columns 4p + j, p = 0..15);
//   * after the loop each lane holds 4 consecutive columns of a row, so the
//     fused alpha/beta epilogue uses 128-bit loads and stores.
//
// Operand layout of v_mfma_f32_16x16x4_f32: lane l = p + 16 g supplies A(row p,
// k_g) and B(k_g, col p) for one k per lane group g, and receives D(row 4g + i,
// col p) in accumulator register i. A and B use the same k for each g.

#include "common.hpp"
#include "kernels.hpp"

namespace dg {
namespace {

constexpr int kBK = 32;       // k per slab
constexpr int kGroupM = 4;

// Float offset of chunk `c` (4 floats) of row `row` in a [rows][32] tile.
__device__ __forceinline__ int a_off(int row, int c) {
    return row * kBK + ((c ^ ((row ^ (row >> 3)) & 7)) << 2);
}

__device__ __forceinline__ f32x4 load4_elems(const float* p, int valid) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (e < valid) ? p[e] : 0.f;
    return v;
}

template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float* p, int valid) {
    if (VEC && valid >= 4) return *reinterpret_cast<const f32x4*>(p);
    if (valid <= 0) return f32x4{0.f, 0.f, 0.f, 0.f};
    return load4_elems(p, valid);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool VEC>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64)
void gemm_f32_mfma_kernel(GemmArgs<float> p, int tiles_m, int tiles_n) {
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

    __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, kGroupM, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

    f32x4 ra[A_CHUNKS], rb[B_CHUNKS];

    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int r = t / 8 + i * (NT / 8), c = t % 8;
            const int64_t gm = m0 + r, gk = k0 + 4 * c;
            const int valid = (gm < M) ? (int)(K - gk < 4 ? K - gk : 4) : 0;
            ra[i] = load4<VEC>(p.A + (valid > 0 ? gm * p.lda + gk : 0), valid);
        }
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) {
            const int idx = t + i * NT;
            const int kr = idx / (BN / 4), c = idx % (BN / 4);
            const int64_t gk = k0 + kr, gn = n0 + 4 * c;
            const int valid = (gk < K) ? (int)(N - gn < 4 ? N - gn : 4) : 0;
            rb[i] = load4<VEC>(p.B + (valid > 0 ? gk * p.ldb + gn : 0), valid);
        }
    };

    auto sstore = [&](int stage) {
        float* As = smem + stage * STAGE;
        float* Bs = As + BM * kBK;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int r = t / 8 + i * (NT / 8), c = t % 8;
            *reinterpret_cast<f32x4*>(As + a_off(r, c)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) {
            const int idx = t + i * NT;
            const int kr = idx / (BN / 4), c = idx % (BN / 4);
            *reinterpret_cast<f32x4*>(Bs + kr * BN + 4 * c) = rb[i];
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
                    b[gq] = *reinterpret_cast<const f32x4*>(Bs + kr * BN + wn0 + 64 * gq + 4 * pl);
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

    const int64_t nk = (K + kBK - 1) / kBK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nk) gload((kt + 1) * kBK);
        compute(cur);
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm0 + 16 * i + 4 * g + r;
            if (row >= M) continue;
#pragma unroll
            for (int gq = 0; gq < NG; ++gq) {
                const int64_t col = n0 + wn0 + 64 * gq + 4 * pl;
                float* dst = p.C + row * p.ldc + col;
                f32x4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = alpha * acc[i][gq][j][r];
                if (VEC && col + 4 <= N) {
                    if (beta != 0.f) {
                        const f32x4 c0 = *reinterpret_cast<const f32x4*>(dst);
#pragma unroll
                        for (int j = 0; j < 4; ++j) v[j] += beta * c0[j];
                    }
                    *reinterpret_cast<f32x4*>(dst) = v;
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

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_tiles(const GemmArgs<float>& a, bool vec, hipStream_t s) {
    const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int tm = (int)tiles_m, tn = (int)tiles_n;
    GemmArgs<float> args = a;
    void* kargs[] = {&args, &tm, &tn};
    const void* fn = vec ? (const void*)&gemm_f32_mfma_kernel<BM, BN, WAVES_M, WAVES_N, true>
                         : (const void*)&gemm_f32_mfma_kernel<BM, BN, WAVES_M, WAVES_N, false>;
    if (tiles_m * tiles_n > kMaxGrid) return hipErrorInvalidConfiguration;
    return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n)), dim3(WAVES_M * WAVES_N * 64),
                           kargs, 0, s);
}

}  // namespace

hipError_t launch_f32_mfma(const GemmArgs<float>& a, bool vec, hipStream_t s) {
    return launch_tiles<128, 128, 2, 2>(a, vec, s);
}

}  // namespace dg
