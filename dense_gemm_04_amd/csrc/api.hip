// C-ABI entry points: argument validation, kernel-family planning, device
// check and launch. Validation and planning touch no HIP API, so every error
// path can be exercised without a GPU.

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstring>

#include "gemm.h"
#include "common.hpp"
#include "kernels.hpp"

namespace {

bool aligned(const void* p, size_t bytes) {
    return (reinterpret_cast<uintptr_t>(p) % bytes) == 0;
}

int64_t max1(int64_t x) { return x > 1 ? x : 1; }

// What a call has to do once its arguments are known to be valid. Every
// activation maps 0 to 0, so without a bias the product-free case is the plain
// one: C = beta * C.
enum class Work { kNone, kScale, kGemm };

Work work_of(int64_t M, int64_t N, int64_t K, float alpha, float beta,
             const void* bias = nullptr) {
    if (M == 0 || N == 0) return Work::kNone;
    if (K == 0 || alpha == 0.f)
        return (beta == 1.f && bias == nullptr) ? Work::kNone : Work::kScale;
    return Work::kGemm;
}

// A rows x cols matrix with leading dimension ld spans (rows - 1) * ld + cols
// elements; every offset the kernels form stays exact while that span, in
// bytes, is below 2^60.
bool span_ok(int esz, int64_t rows, int64_t cols, int64_t ld) {
    if (rows <= 1) return true;
    const int64_t lim = ((int64_t)1 << 60) / esz;
    return cols <= lim && ld <= (lim - cols) / (rows - 1);
}

// Returns true when the arguments are valid (header: GEMM_ERR_INVALID_VALUE).
// With ta, A is stored K x M (lda >= M); with tb, B is stored N x K (ldb >= K).
bool valid_args(int esz, int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                int64_t lda, const void* B, int64_t ldb, float beta, const void* C,
                int64_t ldc, bool ta = false, bool tb = false) {
    if (M < 0 || N < 0 || K < 0) return false;
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return false;
    if (lda < max1(ta ? M : K) || ldb < max1(tb ? K : N) || ldc < max1(N)) return false;
    const Work w = work_of(M, N, K, alpha, beta);
    if (w != Work::kNone && C == nullptr) return false;
    if (w == Work::kGemm && (A == nullptr || B == nullptr)) return false;
    if (!span_ok(esz, M, N, ldc)) return false;
    const bool a_ok = ta ? span_ok(esz, K, M, lda) : span_ok(esz, M, K, lda);
    const bool b_ok = tb ? span_ok(esz, N, K, ldb) : span_ok(esz, K, N, ldb);
    if (w == Work::kGemm && (!a_ok || !b_ok)) return false;
    if (!aligned(A, esz) || !aligned(B, esz) || !aligned(C, esz)) return false;
    return true;
}

// 128-bit global accesses need 16-byte aligned bases and rows.
bool vector_ok(int esz, const void* A, int64_t lda, const void* B, int64_t ldb,
               const void* C, int64_t ldc) {
    const int64_t per = 16 / esz;
    return aligned(A, 16) && aligned(B, 16) && aligned(C, 16) && lda % per == 0 &&
           ldb % per == 0 && ldc % per == 0;
}

// Whether the small-M kernels take M rows: the vector kernel (16-byte rows)
// up to kSkinnyMaxM, also with a transposed B; the element-wise one up to
// kSkinnyElemMaxM, row-major B only.
bool small_m_ok(int64_t M, bool vec, bool tb) {
    return vec ? M <= dg::kSkinnyMaxM : (!tb && M <= dg::kSkinnyElemMaxM);
}

// 65 .. 128 rows run faster on the tiled kernels (their few-tile kernel,
// 64 x 64 tiles with K split over each workgroup's waves) whenever those
// tiles fit one round of compute units: the small-M kernel then holds 8 row
// blocks of A per strip and streams B at about half the rate. One MI355X, B
// from HBM (4 rotating operand sets), small-M kernel plain / with its split
// over a workspace / few-tile kernel: 96 x 8192 x 8192 77.9 / 43.2 / 43.7 us,
// 128 x 8192 x 8192 79.2 / 45.8 / 48.4, 128 x 4096 x 8192 73.3 / 45.7 /
// 37.0, 96 x 4096 x 4096 33.1 / 36.8 / 16.7, 96 x 8192 x 2048 18.0 / 27.1 /
// 12.6. With two rounds of those tiles the small-M kernel stays (128 x 12288
// x 4096: 43.6 against 52.3 us). Only 16-byte rows take the small-M kernel
// above 32 rows, so the rule needs no alignment (the workspace size query
// applies it too).
//
// 33 .. 64 rows (4 row blocks in the small-M kernel): the few-tile kernel too,
// while N x K stays within 2^25 (one MI355X, same method, plain small-M / its
// split / few-tile: 48 x 4096 x 8192 39.7 / 28.9 / 33.3 us, 64 x 4096 x 8192
// 40.4 / 30.5 / 35.3, 64 x 2048 x 8192 39.1 / 26.5 / 29.5, 64 x 8192 x 4096
// 22.2 / 24.8 / 20.1, 64 x 4096 x 4096 21.2 / 23.8 / 17.6, 64 x 4096 x 2048
// 11.2 / 21.5 / 11.2, 48 x 8192 x 4096 19.9 / 23.2 / 19.8; but 48 x 8192 x
// 8192 43.1 / 35.4 / 46.9). With K <= 4096 the split never won, so those
// run there with or without a workspace; with longer K only plain calls do
// (small_m_plain_to_tiles).
bool small_m_to_tiles(int64_t M, int64_t N, int64_t K) {
    if (M > 64) return ((M + 63) / 64) * ((N + 63) / 64) <= 256;
    return M > 32 && K <= 4096 && N <= 16384 && N * K <= ((int64_t)1 << 25);
}
bool small_m_plain_to_tiles(int64_t M, int64_t N, int64_t K, bool split_ws) {
    return !split_ws && M > 32 && M <= 64 && N <= 16384 && N * K <= ((int64_t)1 << 25);
}

// The small-M kernels split K over a workspace only from K = 4096 on: with
// shorter K the split's second phase (partial tiles, counters, the fixed-order
// sum) costs more than the extra workgroups save, however few strips there
// are (one MI355X, B from HBM, plain / split: 16 x 8192 x 1024 6.0 / 8.8 us,
// 32 x 8192 x 2048 9.8 / 13.0, 16 x 8192 x 3072 11.8 / 12.6, 16 x 1024 x
// 2048 8.2 / 13.9, 17 x 64 x 1000 5.8 / 11.8; at K = 4096 level or ahead:
// 16 x 8192 x 4096 15.5 / 15.3, 16 x 4096 x 4096 14.3 / 13.0).
constexpr int64_t kSmallMSplitMinK = 4096;

// The kernel family for a valid call that has GEMM work, or -1 if the
// requested family cannot run it. The small-M kernel reads row-major A and
// either a row-major B or, with 16-byte rows, a transposed one; other
// transposed small-M calls go to the tiled kernels.
int choose(int esz, int64_t M, int64_t N, int64_t K, bool vec, int variant, bool ta = false,
           bool tb = false, bool split_ws = false) {
    switch (variant) {
        case GEMM_VARIANT_AUTO:
            if (esz == 2 && !ta && small_m_ok(M, vec, tb) && !small_m_to_tiles(M, N, K) &&
                !(vec && small_m_plain_to_tiles(M, N, K, split_ws)))
                return GEMM_VARIANT_SKINNY;
            if (esz == 4 && dg::f32_small_preferred(M, N, K, false)) return GEMM_VARIANT_SMALL;
            return vec ? GEMM_VARIANT_MFMA : GEMM_VARIANT_GENERAL;
        case GEMM_VARIANT_MFMA:
            return vec ? GEMM_VARIANT_MFMA : -1;
        case GEMM_VARIANT_GENERAL:
            return GEMM_VARIANT_GENERAL;
        case GEMM_VARIANT_VALU:
            return esz == 4 ? GEMM_VARIANT_VALU : -1;
        case GEMM_VARIANT_SKINNY:
            return (esz == 2 && small_m_ok(M, vec, false)) ? GEMM_VARIANT_SKINNY : -1;
        case GEMM_VARIANT_SMALL:
            return esz == 4 ? GEMM_VARIANT_SMALL : -1;
        default:
            return -1;
    }
}

int plan_impl(int esz, int64_t M, int64_t N, int64_t K, float alpha, const void* A,
              int64_t lda, const void* B, int64_t ldb, float beta, const void* C,
              int64_t ldc, int variant, bool ta = false, bool tb = false, bool split_ws = false) {
    if (esz != 2 && esz != 4) return -1;
    if (variant < GEMM_VARIANT_AUTO || variant > GEMM_VARIANT_SMALL) return -1;
    if (!valid_args(esz, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ta, tb)) return -1;
    if (work_of(M, N, K, alpha, beta) != Work::kGemm) return GEMM_VARIANT_AUTO;
    return choose(esz, M, N, K, vector_ok(esz, A, lda, B, ldb, C, ldc), variant, ta, tb, split_ws);
}

// Per-device cache of "is this a gfx950" (0 unknown, 1 yes, 2 no) and of its
// compute-unit count.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];

// Compute units of a full MI355X: the workspace sizes are computed for it.
constexpr int kFullCus = 256;

gemm_status_t check_device(int* cus, int* device = nullptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_ERR_UNSUPPORTED_DEVICE;
    if (device != nullptr) *device = dev;
    if (dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED_DEVICE;
    int state = g_arch[dev].load(std::memory_order_acquire);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_UNSUPPORTED_DEVICE;
        g_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : kFullCus,
                         std::memory_order_relaxed);
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch[dev].store(state, std::memory_order_release);
    }
    *cus = g_cus[dev].load(std::memory_order_relaxed);
    return state == 1 ? GEMM_OK : GEMM_ERR_UNSUPPORTED_DEVICE;
}

// Operation codes of the *_op entry points (gemm_op_t).
bool valid_op(int op) { return op == GEMM_OP_N || op == GEMM_OP_T; }

// Shared argument check of the workspace entry points.
bool workspace_ok(const void* ws, size_t bytes, size_t need) {
    if (ws == nullptr) return bytes == 0;
    return aligned(ws, 256) && bytes >= need;
}

// Bias and activation of the epilogue entry points (valid also when unused).
bool valid_epilogue(int esz, const void* bias, int act) {
    return act >= GEMM_ACT_NONE && act <= GEMM_ACT_GELU_TANH && aligned(bias, esz);
}

// The tiled fp32 kernel as the automatic choice runs it: when its last round
// of tiles would be partly full, the trailing columns (or rows) of C that
// hold those tiles go to the few-tile kernel and the tiled kernel runs whole
// rounds on the rest (plan_f32_partition); otherwise the tiled kernel alone,
// splitting its last round over the workspace if one is given.
hipError_t launch_f32_auto(const dg::GemmArgs<float>& a, bool vec, void* ws, size_t ws_bytes,
                           int cus, hipStream_t s) {
    const size_t need = dg::f32_mfma_workspace(a.M, a.N, a.K, kFullCus);
    const bool split_ws = ws != nullptr && need > 0 && ws_bytes >= need;
    const dg::F32Partition pt = dg::plan_f32_partition(a.M, a.N, a.K, split_ws);
    if (pt.by == 0) return dg::launch_f32_mfma(a, vec, ws, ws_bytes, cus, s);
    dg::GemmArgs<float> head = a, strip = a;
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
    const hipError_t e = dg::launch_f32_mfma(head, vec, nullptr, 0, cus, s);
    if (e != hipSuccess) return e;
    return dg::launch_f32_small(strip, s);
}

template <typename T>
gemm_status_t run(int64_t M, int64_t N, int64_t K, float alpha, const T* A, int64_t lda,
                  const T* B, int64_t ldb, float beta, T* C, int64_t ldc, void* stream,
                  int variant, void* ws = nullptr, size_t ws_bytes = 0,
                  const T* bias = nullptr, int act = GEMM_ACT_NONE, bool ta = false,
                  bool tb = false, const float* row_scale = nullptr,
                  const float* col_scale = nullptr) {
    constexpr int esz = (int)sizeof(T);
    // A workspace the small-M split can use (the size query names it).
    const bool split_ws = esz == 2 && ws != nullptr && ws_bytes > 0 &&
                          ws_bytes >= gemm_bf16_workspace_size(M, N, K) &&
                          gemm_bf16_workspace_size(M, N, K) > 0;
    int v = plan_impl(esz, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant, ta, tb, split_ws);
    if (v < 0) return GEMM_ERR_INVALID_VALUE;
    // An fp32 call whose split-K workspace the tiled kernel asks for (the
    // workspace size query names it) runs the tiled kernel on it.
    if constexpr (esz == 4) {
        if (v == GEMM_VARIANT_SMALL && variant == GEMM_VARIANT_AUTO && ws != nullptr &&
            !dg::f32_small_preferred(M, N, K, true)) {
            const size_t need = dg::f32_mfma_workspace(M, N, K, kFullCus);
            if (need > 0 && ws_bytes >= need)
                v = vector_ok(esz, A, lda, B, ldb, C, ldc) ? GEMM_VARIANT_MFMA : GEMM_VARIANT_GENERAL;
        }
    }
    if (!valid_epilogue(esz, bias, act)) return GEMM_ERR_INVALID_VALUE;
    if (!aligned(row_scale, 4) || !aligned(col_scale, 4)) return GEMM_ERR_INVALID_VALUE;
    const Work w = work_of(M, N, K, alpha, beta, bias);
    if (w == Work::kScale && C == nullptr) return GEMM_ERR_INVALID_VALUE;
    if (w == Work::kNone) return GEMM_OK;
    int cus = kFullCus;
    const gemm_status_t dev = check_device(&cus);
    if (dev != GEMM_OK) return dev;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (w == Work::kScale) {
        if constexpr (esz == 4) e = dg::launch_scale_f32(M, N, beta, C, ldc, bias, act, s);
        else e = dg::launch_scale_bf16(M, N, beta, C, ldc, bias, act, s);
    } else {
        dg::GemmArgs<T> a{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc, bias, act, ta, tb,
                          row_scale, col_scale};
        const bool vec = vector_ok(esz, A, lda, B, ldb, C, ldc);
        if constexpr (esz == 4) {
            if (v == GEMM_VARIANT_VALU) e = dg::launch_f32_valu(a, vec, s);
            else if (v == GEMM_VARIANT_SMALL) e = dg::launch_f32_small(a, s);
            else if (variant == GEMM_VARIANT_AUTO)
                e = launch_f32_auto(a, v == GEMM_VARIANT_MFMA, ws, ws_bytes, cus, s);
            else e = dg::launch_f32_mfma(a, v == GEMM_VARIANT_MFMA, ws, ws_bytes, cus, s);
        } else {
            // The small-M kernels get the workspace only where the size
            // query asks for one (a split that pays).
            e = (v == GEMM_VARIANT_SKINNY)
                    ? dg::launch_bf16_skinny(a, vec, split_ws ? ws : nullptr, split_ws ? ws_bytes : 0, cus, s)
                    : dg::launch_bf16_mfma(a, v == GEMM_VARIANT_MFMA, ws, ws_bytes, cus, s);
        }
    }
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// ---- static scratch of gemm_bf16_ws_noalloc ---------------------------------
//
// The split-K workspace of the entry point for callers that cannot allocate:
// one array per GPU, allocated with the library's code object on that GPU
// and held until the process ends. Like any static-storage object it starts
// zero-filled; every call leaves its counters at zero again.
constexpr size_t kScratchBytes = GEMM_NOALLOC_SCRATCH_BYTES;
// The counters of every split sit in the first bytes of a workspace (one int
// per strip or split tile, padded to 256 bytes); a shape whose slots fit in
// kScratchBytes has fewer than 16384 of them, so this prefix holds them all.
constexpr size_t kScratchCounterBytes = 65536;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Per device: the scratch's device address (host code must use this, never
// the name `scratch`, which on the host is only a stand-in for the symbol),
// and whether its counter prefix has been cleared.
std::atomic<void*> g_scratch[kMaxDevices];
std::atomic<int> g_scratch_cleared[kMaxDevices];

__global__ void clear_words(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The scratch of device `dev` (current), its counter prefix cleared once by a
// kernel on `stream` before the first call that uses it (a fill kernel rather
// than a memset, so that a call under stream capture records an ordinary
// kernel node). Returns nullptr if the symbol cannot be resolved or the clear
// cannot be launched.
void* scratch_for(int dev, hipStream_t stream) {
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    int expected = 0;
    if (g_scratch_cleared[dev].compare_exchange_strong(expected, 1, std::memory_order_acq_rel)) {
        clear_words<<<16, 256, 0, stream>>>(static_cast<uint32_t*>(p), (int)(kScratchCounterBytes / 4));
        if (hipGetLastError() != hipSuccess) {
            g_scratch_cleared[dev].store(0, std::memory_order_release);
            return nullptr;
        }
    }
    return p;
}

}  // namespace

extern "C" {

gemm_status_t gemm_bf16_ws_noalloc(int64_t M, int64_t N, int64_t K, float alpha,
                                   const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                   float beta, uint16_t* C, int64_t ldc, void* stream) {
    // Host-only checks first: arguments, then whether the split fits the scratch.
    if (plan_impl(2, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, GEMM_VARIANT_AUTO) < 0)
        return GEMM_ERR_INVALID_VALUE;
    if (work_of(M, N, K, alpha, beta) != Work::kGemm)
        return gemm_bf16_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO);
    const size_t need = gemm_bf16_workspace_size(M, N, K);
    if (need > kScratchBytes || (N + 63) / 64 * 4 > (int64_t)kScratchCounterBytes)
        return GEMM_ERR_SCRATCH_LIMIT;
    if (need == 0)
        return gemm_bf16_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO);
    int cus = 0, dev = -1;
    const gemm_status_t st = check_device(&cus, &dev);
    if (st != GEMM_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    void* ws = scratch_for(dev, s);
    if (ws == nullptr) return GEMM_ERR_LAUNCH;
    return run<uint16_t>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO,
                         ws, kScratchBytes);
}

gemm_status_t gemm_f32_ex(int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                          int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                          int64_t ldc, void* stream, int variant) {
    return run<float>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant);
}

gemm_status_t gemm_bf16_ex(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t* A,
                           int64_t lda, const uint16_t* B, int64_t ldb, float beta, uint16_t* C,
                           int64_t ldc, void* stream, int variant) {
    return run<uint16_t>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant);
}

size_t gemm_bf16_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0 || M > INT_MAX || N > INT_MAX || K > INT_MAX) return 0;
    if (M <= dg::kSkinnyMaxM && !small_m_to_tiles(M, N, K))
        return K >= kSmallMSplitMinK ? dg::bf16_skinny_workspace(M, N, K) : 0;
    return dg::bf16_tiled_workspace(M, N, K, kFullCus);
}

gemm_status_t gemm_bf16_ws(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t* A,
                           int64_t lda, const uint16_t* B, int64_t ldb, float beta, uint16_t* C,
                           int64_t ldc, void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace_ok(workspace, workspace_bytes, gemm_bf16_workspace_size(M, N, K)))
        return GEMM_ERR_INVALID_VALUE;
    return run<uint16_t>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO,
                         workspace, workspace_bytes);
}

size_t gemm_f32_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0 || M > INT_MAX || N > INT_MAX || K > INT_MAX) return 0;
    // Shapes that the few-tile kernel takes even with a workspace need none,
    // nor do those whose partly full last round is cheaper as a strip on it.
    if (dg::f32_small_preferred(M, N, K, true)) return 0;
    if (dg::plan_f32_partition(M, N, K, true).by != 0) return 0;
    return dg::f32_mfma_workspace(M, N, K, kFullCus);
}

gemm_status_t gemm_f32_ws(int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                          int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                          int64_t ldc, void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace_ok(workspace, workspace_bytes, gemm_f32_workspace_size(M, N, K)))
        return GEMM_ERR_INVALID_VALUE;
    return run<float>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO,
                      workspace, workspace_bytes);
}

gemm_status_t gemm_f32_bias_act(int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                                int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                                int64_t ldc, const float* bias, int act, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (!workspace_ok(workspace, workspace_bytes, gemm_f32_workspace_size(M, N, K)))
        return GEMM_ERR_INVALID_VALUE;
    return run<float>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO,
                      workspace, workspace_bytes, bias, act);
}

gemm_status_t gemm_bf16_bias_act(int64_t M, int64_t N, int64_t K, float alpha,
                                 const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                 float beta, uint16_t* C, int64_t ldc, const uint16_t* bias,
                                 int act, void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace_ok(workspace, workspace_bytes, gemm_bf16_workspace_size(M, N, K)))
        return GEMM_ERR_INVALID_VALUE;
    return run<uint16_t>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO,
                         workspace, workspace_bytes, bias, act);
}

gemm_status_t gemm_f32_op(int opa, int opb, int64_t M, int64_t N, int64_t K, float alpha,
                          const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                          float* C, int64_t ldc, const float* bias, int act, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (!valid_op(opa) || !valid_op(opb)) return GEMM_ERR_INVALID_VALUE;
    if (!workspace_ok(workspace, workspace_bytes, gemm_f32_workspace_size(M, N, K)))
        return GEMM_ERR_INVALID_VALUE;
    return run<float>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO,
                      workspace, workspace_bytes, bias, act, opa == GEMM_OP_T, opb == GEMM_OP_T);
}

gemm_status_t gemm_bf16_op(int opa, int opb, int64_t M, int64_t N, int64_t K, float alpha,
                           const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                           float beta, uint16_t* C, int64_t ldc, const uint16_t* bias, int act,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_op(opa) || !valid_op(opb)) return GEMM_ERR_INVALID_VALUE;
    if (!workspace_ok(workspace, workspace_bytes, gemm_bf16_workspace_size(M, N, K)))
        return GEMM_ERR_INVALID_VALUE;
    return run<uint16_t>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO,
                         workspace, workspace_bytes, bias, act, opa == GEMM_OP_T,
                         opb == GEMM_OP_T);
}

gemm_status_t gemm_f32_scaled(int opa, int opb, int64_t M, int64_t N, int64_t K, float alpha,
                              const float* A, int64_t lda, const float* B, int64_t ldb,
                              float beta, float* C, int64_t ldc, const float* row_scale,
                              const float* col_scale, const float* bias, int act,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_op(opa) || !valid_op(opb)) return GEMM_ERR_INVALID_VALUE;
    if (!workspace_ok(workspace, workspace_bytes, gemm_f32_workspace_size(M, N, K)))
        return GEMM_ERR_INVALID_VALUE;
    return run<float>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO,
                      workspace, workspace_bytes, bias, act, opa == GEMM_OP_T, opb == GEMM_OP_T,
                      row_scale, col_scale);
}

gemm_status_t gemm_bf16_scaled(int opa, int opb, int64_t M, int64_t N, int64_t K, float alpha,
                               const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                               float beta, uint16_t* C, int64_t ldc, const float* row_scale,
                               const float* col_scale, const uint16_t* bias, int act,
                               void* workspace, size_t workspace_bytes, void* stream) {
    if (!valid_op(opa) || !valid_op(opb)) return GEMM_ERR_INVALID_VALUE;
    if (!workspace_ok(workspace, workspace_bytes, gemm_bf16_workspace_size(M, N, K)))
        return GEMM_ERR_INVALID_VALUE;
    return run<uint16_t>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO,
                         workspace, workspace_bytes, bias, act, opa == GEMM_OP_T,
                         opb == GEMM_OP_T, row_scale, col_scale);
}

gemm_status_t gemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                       int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                       int64_t ldc, void* stream) {
    return gemm_f32_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO);
}

gemm_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t* A,
                        int64_t lda, const uint16_t* B, int64_t ldb, float beta, uint16_t* C,
                        int64_t ldc, void* stream) {
    return gemm_bf16_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, GEMM_VARIANT_AUTO);
}

int gemm_plan(int elem_bytes, int64_t M, int64_t N, int64_t K, float alpha, const void* A,
              int64_t lda, const void* B, int64_t ldb, float beta, const void* C, int64_t ldc,
              int variant) {
    return plan_impl(elem_bytes, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant);
}

const char* gemm_status_string(int status) {
    switch (status) {
        case GEMM_OK: return "success";
        case GEMM_ERR_INVALID_VALUE: return "invalid argument";
        case GEMM_ERR_UNSUPPORTED_DEVICE: return "current device is not a gfx950 GPU";
        case GEMM_ERR_LAUNCH: return "kernel launch failed";
        case GEMM_ERR_SCRATCH_LIMIT:
            return "shape needs more split-K scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

}  // extern "C"
