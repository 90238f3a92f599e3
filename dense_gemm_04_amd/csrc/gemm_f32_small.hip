// fp32 GEMM for problems with few output tiles: C = alpha * op(A) * op(B) + beta * C
// on v_mfma_f32_16x16x4_f32, with K split over the waves of a workgroup.
//
// A 128 x 128 fp32 tile keeps one compute unit's matrix cores busy for
// 128 * 128 * 2 / 256 = 128 clocks per k, so a product with a handful of such
// tiles (256^3 has four) runs on a handful of CUs and takes as long as one
// tile's whole K loop. Without a workspace the K dimension cannot be shared
// between workgroups, but it can be shared between the waves of one: here a
// workgroup owns a T x T tile (T = 16, 32 or 64, chosen so that most CUs get
// one), each of its S waves multiplies one contiguous K range of it, and the
// S partial tiles are added in LDS in wave order. The split is the
// SGEMM article's K slicing carried into the workgroup; the sums are in a
// fixed order, so the results are the same bits on every call.
//
// No operand is shared between the waves (each has its own K range), so
// there is no LDS staging: each lane loads its MFMA operands straight from
// global memory (L2) into registers, one 16-k chunk ahead of the MFMAs.
// MFMA step j of a chunk starting at k = b gives lane p + 16 g the pair
// A(row p, b + 4 g + j), B(b + 4 g + j, col p): over the chunk's four steps
// every k of the chunk is used once, and a k-contiguous operand (row-major A,
// transposed B) arrives as one 128-bit load per lane and 16 x 16 block for
// all four steps. An m/n-contiguous operand (row-major B, transposed A) is
// read one 4-byte element per lane and step (a 64-byte row segment per lane
// group). Every address is clamped into the operand and every k past the
// wave's range reads as zero, so ragged M, N and K need no special cases.
//
// Operand layout of v_mfma_f32_16x16x4_f32: lane l = p + 16 g supplies A(row p,
// k_g) and B(k_g, col p), and receives D(row 4 g + i, col p) in accumulator
// register i.

#include "common.hpp"
#include "kernels.hpp"

namespace dg {
namespace {

constexpr int kChunk = 16;   // k per chunk: four MFMA steps of k = 4

// Element (i, k) of an operand stored as rows of k (kcontig: at i * ld + k)
// or as rows of i (at k * ld + i), for the four k = k0 .. k0 + 3 of one lane:
// zero at k >= kend; addresses clamped into [0, rows) x [0, K).
template <bool KCONTIG>
__device__ __forceinline__ f32x4 load_k4(const float* __restrict__ X, int64_t ld, int64_t i,
                                         int64_t k0, int64_t kend, int64_t K) {
    f32x4 v;
    if constexpr (KCONTIG) {
        const float* row = X + i * ld;
        if (k0 + 3 < kend) return (f32x4)*reinterpret_cast<const f32x4_a4*>(row + k0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t k = k0 + e;
            const float x = row[k < K ? k : K - 1];
            v[e] = k < kend ? x : 0.f;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t k = k0 + e;
            const float x = X[(k < K ? k : K - 1) * ld + i];
            v[e] = k < kend ? x : 0.f;
        }
    }
    return v;
}

// With `raster`, tiles are renumbered per XCD and walked in groups of 4 tile
// rows, so the tiles of one XCD share A rows and B columns in its L2; without
// it, workgroup b takes tile (b / tiles_n, b mod tiles_n). The renumbering's
// divisions delay a workgroup's first loads by about 0.2 us, which only a
// long enough K loop repays (one MI355X, plain order against renumbered: 256^3
// 2.83 against 3.13 us, 512^3 5.80 against 5.97; 1024^3 26.26 against 25.38,
// 256^2 x 4096 14.62 against 13.27).
constexpr int kGroupM = 4;
constexpr int64_t kRasterMinK = 1024;

// One workgroup per T x T tile of C; wave w multiplies K chunks
// [w * kcw, (w + 1) * kcw) (16 k each) of it.
template <int T, int S, bool TA, bool TB, bool EPI>
__global__ __launch_bounds__(S * 64)
void gemm_f32_small_kernel(GemmArgs<float> p, int tiles_m, int tiles_n, int kcw, int raster) {
    constexpr int NB = T / 16;                 // 16 x 16 blocks per tile side
    constexpr int NT = S * 64;
    constexpr int LD = T + 4;                  // reduction rows, padded against bank conflicts
    __shared__ __attribute__((aligned(16))) float red[S][T][LD];

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int pl = lane & 15, g = lane >> 4;
    int tm, tn;
    if (raster) {
        tile_coords((int)blockIdx.x, (int)gridDim.x, tiles_m, tiles_n, kGroupM, tm, tn);
    } else {
        tm = __builtin_amdgcn_readfirstlane((int)blockIdx.x / tiles_n);
        tn = __builtin_amdgcn_readfirstlane((int)blockIdx.x - tm * tiles_n);
    }
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t m0 = (int64_t)tm * T, n0 = (int64_t)tn * T;
    const int64_t kbeg = (int64_t)wave * kcw * kChunk;
    const int64_t kend = kbeg + (int64_t)kcw * kChunk < K ? kbeg + (int64_t)kcw * kChunk : K;

    // The rows of A and columns of B this lane supplies, clamped into the
    // matrix (a row or column past the edge only feeds outputs not stored).
    int64_t arow[NB], bcol[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int64_t r = m0 + 16 * i + pl, c = n0 + 16 * i + pl;
        arow[i] = r < M ? r : M - 1;
        bcol[i] = c < N ? c : N - 1;
    }

    struct Frag {
        f32x4 a[NB], b[NB];   // component j: MFMA step j of the chunk
    };
    auto load = [&](int64_t base, Frag& f) {
        const int64_t k0 = base + 4 * g;
#pragma unroll
        for (int i = 0; i < NB; ++i) f.a[i] = load_k4<!TA>(p.A, p.lda, arow[i], k0, kend, K);
#pragma unroll
        for (int j = 0; j < NB; ++j) f.b[j] = load_k4<TB>(p.B, p.ldb, bcol[j], k0, kend, K);
    };

    f32x4 acc[NB][NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mfmas = [&](const Frag& f) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[i][s], f.b[j][s], acc[i][j],
                                                                     0, 0, 0);
    };

    // Two chunks in registers: the next one loads while this one multiplies.
    // A chunk past the range (an odd count's last) reads as zeros.
    Frag f0, f1;
    if (kbeg < kend) {
        load(kbeg, f0);
        for (int c = 0; c < kcw; c += 2) {
            const int64_t b = kbeg + (int64_t)c * kChunk;
            load(b + kChunk, f1);
            mfmas(f0);
            if (c + 2 < kcw) load(b + 2 * kChunk, f0);
            mfmas(f1);
        }
    }

    // Partial tiles to LDS, then every output summed over the waves in order.
    // (Storing them column by column, so that each lane writes and reads
    // 128 bits at a time, measured 2-4% slower.)
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][16 * i + 4 * g + r][16 * j + pl] = acc[i][j][r];
    __syncthreads();

    const float alpha = p.alpha, beta = p.beta;
    for (int q = t; q < T * T / 4; q += NT) {
        const int row = q / (T / 4), c4 = 4 * (q % (T / 4));
        const int64_t gr = m0 + row, gc = n0 + c4;
        if (gr >= M || gc >= N) continue;
        f32x4 sum = *reinterpret_cast<const f32x4*>(&red[0][row][c4]);
#pragma unroll
        for (int w = 1; w < S; ++w) sum += *reinterpret_cast<const f32x4*>(&red[w][row][c4]);
        const float fr = EPI ? row_factor(p, gr) : alpha;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = fr * sum[e];
            if constexpr (EPI) v[e] = activate(v[e] * col_factor(p, gc + e) + bias_at(p, gc + e), p.act);
        }
        float* dst = p.C + gr * p.ldc + gc;
        if (gc + 4 <= N) {
            if (beta != 0.f) {
                const f32x4 c0 = (f32x4)*reinterpret_cast<const f32x4_a4*>(dst);
                v += beta * c0;
            }
            *reinterpret_cast<f32x4_a4*>(dst) = (f32x4_a4)v;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (gc + e < N) {
                    float x = v[e];
                    if (beta != 0.f) x += beta * dst[e];
                    dst[e] = x;
                }
            }
        }
    }
}

template <int T, int S, bool EPI>
const void* pick_small(bool ta, bool tb) {
#define DG_SMALL(TA, TB) (const void*)&gemm_f32_small_kernel<T, S, TA, TB, EPI>
    return ta ? (tb ? DG_SMALL(true, true) : DG_SMALL(true, false))
              : (tb ? DG_SMALL(false, true) : DG_SMALL(false, false));
#undef DG_SMALL
}

template <int T, int S>
hipError_t launch_small_cfg(const GemmArgs<float>& a, hipStream_t s) {
    const int64_t tiles_m = (a.M + T - 1) / T, tiles_n = (a.N + T - 1) / T;
    const int64_t chunks = (a.K + kChunk - 1) / kChunk;
    int kcw = (int)((chunks + S - 1) / S);
    int tm = (int)tiles_m, tn = (int)tiles_n;
    int raster = a.K >= kRasterMinK ? 1 : 0;
    GemmArgs<float> args = a;
    void* kargs[] = {&args, &tm, &tn, &kcw, &raster};
    const void* fn = has_epilogue(a) ? pick_small<T, S, true>(a.ta, a.tb)
                                     : pick_small<T, S, false>(a.ta, a.tb);
    const int64_t grid = tiles_m * tiles_n;
    if (grid > kMaxGrid) return hipErrorInvalidConfiguration;
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(S * 64), kargs, 0, s);
}

}  // namespace

// Planning uses a full MI355X (256 CUs) whatever the device, so that a
// shape's tile size and K split, and with them its rounding, do not depend on
// how the GPU is partitioned.
constexpr int64_t kPlanCus = 256;

// Modelled time of the few-tile kernel with T x T tiles, in units of one
// 64 x 64 tile's K loop / 4096 per k: each CU runs ceil(tiles / CUs) tiles
// one after another (or side by side, sharing its matrix cores), and a tile
// costs T^2 over the tile size's measured efficiency relative to T = 64 (at
// 1024 x 1024 x 4096: 89.6 us with T = 64, 104.0 with 32, 197.7 with 16,
// which is 1 : 0.86 : 0.45).
static double small_cost(int64_t M, int64_t N, int T) {
    const int64_t tiles = ((M + T - 1) / T) * ((N + T - 1) / T);
    const double eff = T == 64 ? 1.0 : (T == 32 ? 0.86 : 0.45);
    return (double)((tiles + kPlanCus - 1) / kPlanCus) * T * T / eff;
}

SmallPlan plan_f32_small(int64_t M, int64_t N, int64_t K) {
    int best = 64;
    for (int T : {32, 16})
        if (small_cost(M, N, T) < small_cost(M, N, best)) best = T;
    const int64_t tiles = ((M + best - 1) / best) * ((N + best - 1) / best);
    // Waves per workgroup: 4 for K <= 128 (2 chunks each at most), 16 when a
    // workgroup has its CU to itself and K is long enough to give each wave
    // 8 chunks (2.5 us faster at 64 x 4096 x 4096 and 512^2 x 2048, 1.4 at
    // 256^2 x 4096), else 8. A 64 x 64 tile always takes 8: its 8 partial
    // tiles already fill most of the LDS.
    int waves = 8;
    if (best < 64) {
        if (K <= 128) waves = 4;
        else if (K >= 2048 && tiles <= kPlanCus) waves = 16;
    }
    return SmallPlan{best, waves};
}

// A round of the tiled kernel in the same units: at most one 128 x 128 tile
// per CU takes 128^2 over its efficiency relative to a 64 x 64 few-tile tile,
// 1.45 (1536^2 x 1024: 72.2 us tiled, 61.2 with 32 x 32 tiles; 2048^3: 140.6
// tiled, 180.6 with 64 x 64 tiles at four per CU); two per CU take 1.63 times
// that (4096^3: 943 us for two such rounds of K = 4096).
constexpr double kTiledRound1 = 128.0 * 128.0 / 1.45;
constexpr double kTiledRound2 = 1.63 * kTiledRound1;

static double best_small_cost(int64_t M, int64_t N) {
    double best = small_cost(M, N, 64);
    for (int T : {32, 16}) best = small_cost(M, N, T) < best ? small_cost(M, N, T) : best;
    return best;
}

bool f32_small_preferred(int64_t M, int64_t N, int64_t K, bool split_ws) {
    const int64_t tiles128 = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles128 > kPlanCus) return false;
    const SmallPlan sp = plan_f32_small(M, N, K);
    if (small_cost(M, N, sp.tile) >= kTiledRound1) return false;
    // Given its split-K workspace the tiled kernel shares K between
    // workgroups too, and wins once there are enough tile-k to share:
    // 1024^2 x 4096 86.3 us against 89.6, 1408^2 x 4096 150.4 against 175.4,
    // 1024 x 2048 x 2048 82.9 against 91.6; below 2^18 it loses (1024^3 40.0
    // against 26.3, 64 x 4096 x 4096 55.4 against 30.1).
    if (split_ws && tiles128 * K >= ((int64_t)1 << 18)) return false;
    return true;
}

F32Partition plan_f32_partition(int64_t M, int64_t N, int64_t K, bool split_ws) {
    (void)K;
    F32Partition none{0, 0};
    const int64_t tm = (M + 127) / 128, tn = (N + 127) / 128;
    const int64_t slots = 2 * kPlanCus;       // the tiled kernel's resident workgroups
    const int64_t tiles = tm * tn, tail = tiles % slots;
    if (tiles > kPlanCus && tiles < slots) {
        // 257 .. 511 tiles: one round with two tiles on some CUs, which lasts
        // about as long as a full round (kTiledRound2). The trailing columns
        // (or rows) holding the tiles past one per CU can go to the few-tile
        // kernel instead, leaving the tiled kernel one tile per CU
        // (kTiledRound1). The model overstates the cost of the pair by about
        // a tenth; measured (one MI355X, plain calls, model ratio of the pair
        // to the round in brackets): 2048 x 2304 x 4096 467 -> 328 us (0.74),
        // 2048 x 2560 x 4096 467 -> 363 (0.84), 2304^2 x 4096 467 -> 403
        // (0.94), 3072 x 2048 x 4096 471 -> 451 (1.06), but 2304 x 2816 x
        // 4096 471 -> 503 (1.20) and 2560^2 x 4096 470 -> 528 (1.26). Hence
        // the pair below 1.1. Given a workspace, splitting the round over K
        // beat the pair from 0.94 up (2304^2 x 2048 204 against 207 us,
        // 3072 x 2048 x 4096 432 against 451) and lost below (2048 x 2560 x
        // 4096 408 against 363): the pair only below 0.9 then.
        const int64_t extra = tiles - kPlanCus;
        const int64_t rn = (extra + tm - 1) / tm, rm = (extra + tn - 1) / tn;
        const double cost_n = rn < tn ? best_small_cost(M, N - (tn - rn) * 128) : 1e300;
        const double cost_m = rm < tm ? best_small_cost(M - (tm - rm) * 128, N) : 1e300;
        const bool by_cols = cost_n <= cost_m;
        const double cost = by_cols ? cost_n : cost_m;
        if (kTiledRound1 + cost > (split_ws ? 0.9 : 1.1) * kTiledRound2) return none;
        return by_cols ? F32Partition{1, (tn - rn) * 128} : F32Partition{2, (tm - rm) * 128};
    }
    if (tiles < slots || tail == 0) return none;
    // The last round's cost, and the strip that takes its tiles off the
    // tiled kernel: trailing tile columns (or rows) covering at least `tail`
    // tiles, so that the tiled kernel is left whole rounds.
    const double round = tail <= kPlanCus ? kTiledRound1 : kTiledRound2;
    const int64_t rn = (tail + tm - 1) / tm, rm = (tail + tn - 1) / tn;
    const int64_t nsplit = (tn - rn) * 128, msplit = (tm - rm) * 128;
    const double cost_n = rn < tn ? best_small_cost(M, N - nsplit) : 1e300;
    const double cost_m = rm < tm ? best_small_cost(M - msplit, N) : 1e300;
    const bool by_cols = cost_n <= cost_m;
    const double cost = by_cols ? cost_n : cost_m;
    // Worth it when the strip clearly beats the round it removes. It also
    // beat splitting that round over a workspace wherever both applied (one
    // MI355X: 4095 x 4097 x 1023 313 us against 329, 4096 x 4352 x 2048 531
    // against 603, 2560 x 4096 x 2048 338 against 360), so `split_ws` does not
    // change the choice.
    (void)split_ws;
    if (cost > 0.8 * round) return none;
    return by_cols ? F32Partition{1, nsplit} : F32Partition{2, msplit};
}

hipError_t launch_f32_small(const GemmArgs<float>& a, hipStream_t s) {
    const SmallPlan sp = plan_f32_small(a.M, a.N, a.K);
    switch (sp.tile * 100 + sp.waves) {
        case 1616: return launch_small_cfg<16, 16>(a, s);
        case 1608: return launch_small_cfg<16, 8>(a, s);
        case 1604: return launch_small_cfg<16, 4>(a, s);
        case 3216: return launch_small_cfg<32, 16>(a, s);
        case 3208: return launch_small_cfg<32, 8>(a, s);
        case 3204: return launch_small_cfg<32, 4>(a, s);
        case 6408: return launch_small_cfg<64, 8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dg
