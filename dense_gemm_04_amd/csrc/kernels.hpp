// Host-side launchers for the gfx950 GEMM kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dg {

// Every launcher runs the epilogue instantiation of its kernel when the
// arguments carry a bias or an activation (has_epilogue).
//
// `vec` tells a launcher that every base pointer and row is 16-byte aligned
// (128-bit copies and accesses). Without it each launcher takes the widest
// accesses the actual alignment allows: 4-byte copies for rows aligned to 4
// bytes, unaligned 128-bit or element-wise accesses otherwise.
//
// Workspace arguments (ws may be null): given at least the bytes the matching
// *_workspace function returns for the shape (256-byte aligned, counters
// zero), a kernel splits K for the tiles of a last round that would leave
// most of the `cus` compute units idle; otherwise it runs unsplit.
hipError_t launch_bf16_mfma(const GemmArgs<uint16_t>& a, bool vec, void* ws, size_t ws_bytes,
                            int cus, hipStream_t s);
// The two bf16 MFMA kernels behind launch_bf16_mfma: the tiled kernel (needs
// rows aligned to 16 bytes, or to 4 with `dw`, and offsets that fit its 31-bit
// buffer offsets; splits K with a workspace; products with few tiles go to
// the few-tile kernel, and a partly full last round of 256 x 256 tiles may
// run as a second product, a strip of trailing columns or rows) and the
// element-wise one that takes any alignment.
hipError_t launch_bf16_tiled(const GemmArgs<uint16_t>& a, bool dw, void* ws, size_t ws_bytes,
                             int cus, hipStream_t s);
size_t bf16_tiled_workspace(int64_t M, int64_t N, int64_t K, int cus);
// bf16 products with few 64 x 64 tiles: K split over the 4 waves of each
// workgroup (no workspace). `dw`: rows aligned to 4 bytes only (4-byte copies).
hipError_t launch_bf16_few(const GemmArgs<uint16_t>& a, bool dw, hipStream_t s);
bool bf16_tiled_fits(const GemmArgs<uint16_t>& a);
hipError_t launch_bf16_general(const GemmArgs<uint16_t>& a, bool vec, hipStream_t s);
// fp32 MFMA kernel. Given a workspace of at least f32_mfma_workspace(M, N, K,
// cus) bytes (256-byte aligned, counters zero), a last round of tiles that
// would leave most of the `cus` compute units idle is split over K.
hipError_t launch_f32_mfma(const GemmArgs<float>& a, bool vec, void* ws, size_t ws_bytes, int cus,
                           hipStream_t s);
size_t f32_mfma_workspace(int64_t M, int64_t N, int64_t K, int cus);
hipError_t launch_f32_valu(const GemmArgs<float>& a, bool vec, hipStream_t s);
// fp32 products with few output tiles: T x T tiles with K split over the
// waves of each workgroup (any layout, rows aligned to 4 bytes).
struct SmallPlan {
    int tile;    // 16, 32 or 64
    int waves;   // waves per workgroup, each one K range: 4, 8 or 16
};
// The tile size and wave count this kernel uses for a shape.
SmallPlan plan_f32_small(int64_t M, int64_t N, int64_t K);
// Whether the automatic choice runs this kernel rather than the tiled one;
// `split_ws`: the caller gave the tiled kernel's split-K workspace.
bool f32_small_preferred(int64_t M, int64_t N, int64_t K, bool split_ws);
hipError_t launch_f32_small(const GemmArgs<float>& a, hipStream_t s);
// Products whose 128 x 128 tiles fill whole rounds of the tiled kernel and
// leave a last round partly full: `by` 1 puts columns [split, N) of C, 2 rows
// [split, M), on the few-tile kernel, so that the tiled kernel runs whole
// rounds on the rest; 0: no partition. `split_ws`: the caller gave the tiled
// kernel's split-K workspace, which the partition must then clearly beat.
struct F32Partition {
    int by;
    int64_t split;
};
F32Partition plan_f32_partition(int64_t M, int64_t N, int64_t K, bool split_ws);
// Small-M bf16 (M <= kSkinnyMaxM; without `vec`, M <= kSkinnyElemMaxM). With
// `vec` the 64-column copy-ring kernel runs; given a workspace of at least bf16_skinny_workspace(M, N, K) bytes
// (256-byte aligned, counters zero) it splits K over several workgroups.
hipError_t launch_bf16_skinny(const GemmArgs<uint16_t>& a, bool vec, void* ws, size_t ws_bytes,
                              int cus, hipStream_t s);
// Workspace bytes with which launch_bf16_skinny splits K (0: no split for this
// shape); at least what the streaming kernel below needs when it applies.
size_t bf16_skinny_workspace(int64_t M, int64_t N, int64_t K);

// Small-M streaming kernel (vector path, row-major B, split K): 256-column
// strips with K interleaved over `phases` workgroups per strip in 32-row
// blocks (block b goes to phase b mod phases).
struct StreamWork {
    int strips;   // 256-column strips of C
    int phases;   // workgroups per strip (0: the kernel does not apply)
    int nblk;     // 32-row blocks of K
};
StreamWork plan_stream(int64_t N, int64_t K);
// Workspace bytes the streaming kernel needs (0 when it does not apply).
size_t bf16_stream_workspace(int64_t M, int64_t N, int64_t K);
bool bf16_stream_fits(const GemmArgs<uint16_t>& a);
// Needs M <= kSkinnyMaxM, 16-byte rows, plan_stream(N, K).phases >= 2 and a
// workspace of bf16_stream_workspace(M, N, K) bytes (256-byte aligned, zeros).
hipError_t launch_bf16_stream(const GemmArgs<uint16_t>& a, void* ws, hipStream_t s);

// C <- act(bias[col]) + beta * C, the product-free case (beta == 0 writes
// without reading C; without bias and activation the first term is 0).
hipError_t launch_scale_f32(int64_t M, int64_t N, float beta, float* C, int64_t ldc,
                            const float* bias, int act, hipStream_t s);
hipError_t launch_scale_bf16(int64_t M, int64_t N, float beta, uint16_t* C, int64_t ldc,
                             const uint16_t* bias, int act, hipStream_t s);

// Largest M the small-M kernels accept: the vector kernel (16-byte rows)
// takes up to 128 rows, the element-wise one up to 32.
constexpr int64_t kSkinnyMaxM = 128;
constexpr int64_t kSkinnyElemMaxM = 32;

// Workgroup ids are ints: launchers refuse grids beyond this (a matrix that
// large cannot exist in device memory, so this only guards the arithmetic).
constexpr int64_t kMaxGrid = 0x7fffffff;

}  // namespace dg
