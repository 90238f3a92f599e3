// Shared device/host helpers for the gfx950 GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Arguments every GEMM kernel receives, by value (kernarg segment). `bias`
// (length N, or null), `act` and the scale vectors are read only by the
// epilogue instantiations.
template <typename T>
struct GemmArgs {
    int64_t M, N, K;
    float alpha, beta;
    const T* A; int64_t lda;
    const T* B; int64_t ldb;
    T* C; int64_t ldc;
    const T* bias = nullptr;
    int act = 0;
    // Transposed storage: A(i,k) = A[k*lda + i] (A is K x M) when ta, and
    // B(k,j) = B[j*ldb + k] (B is N x K) when tb.
    bool ta = false, tb = false;
    // Quantisation scales (fp32, or null): the product of row i and column j
    // is multiplied by row_scale[i] * col_scale[j] along with alpha.
    const float* row_scale = nullptr;
    const float* col_scale = nullptr;
};

// 128-bit vectors at addresses aligned only to their element (4 or 2 bytes).
// gfx950 under the HSA runtime runs with unaligned global access enabled, and
// the compiler emits one 128-bit load or store for these types; the kernels
// use them on rows that are not 16-byte aligned.
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// ---- buffer (descriptor-based) global loads ---------------------------------
//
// A raw buffer descriptor covers [base, base + bytes). Loads whose offset lies
// past `bytes` return zero instead of touching memory, which is how the tiled
// kernels read the ragged edges of A and B without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Descriptor word 3 for gfx9-family raw buffers (32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// ---- bf16 helpers ---------------------------------------------------------

// bf16 bit pattern -> fp32 (exact: the pattern is the top half of the word).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---- fused bias + activation epilogue --------------------------------------
//
// out = act(alpha * acc + bias[col]) + beta * C0: the bias is added and the
// activation applied before the residual term, as a fused GELU + residual
// kernel does (Z-Turbo tuning page, section 2.1).

constexpr int kActNone = 0, kActRelu = 1, kActGeluTanh = 2;

// GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
// Since 0.5 (1 + tanh u) is the logistic function of 2u, this equals
// x / (1 + exp(-2u)), evaluated here with the hardware exp2 and reciprocal:
// no cancellation for negative x, and 0 or x in the limits (exp2 -> inf or 0).
__device__ __forceinline__ float gelu_tanh(float x) {
    constexpr float kScale = -2.3022082f;   // -2 sqrt(2/pi) log2(e)
    const float t = kScale * x * __builtin_fmaf(0.044715f * x, x, 1.f);
    return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(t));
}

// Branch-free: both activations are computed and one is selected, so an
// epilogue over many elements runs no per-element branch on `act` (with the
// branches, fp32 4096^3 with bias + GELU ran 4% slower than without them).
__device__ __forceinline__ float activate(float x, int act) {
    const float relu = x > 0.f ? x : 0.f, gelu = gelu_tanh(x);
    return act == kActRelu ? relu : (act == kActGeluTanh ? gelu : x);
}

__device__ __forceinline__ float elem_f32(float v) { return v; }
__device__ __forceinline__ float elem_f32(uint16_t v) { return bf16_to_f32(v); }

// True when a call needs the epilogue instantiations.
template <typename T>
inline bool has_epilogue(const GemmArgs<T>& a) {
    return a.bias != nullptr || a.act != kActNone || a.row_scale != nullptr ||
           a.col_scale != nullptr;
}

// Bias of column `col`: 0 past N or without a bias vector.
template <typename T>
__device__ __forceinline__ float bias_at(const GemmArgs<T>& p, int64_t col) {
    return (p.bias != nullptr && col < p.N) ? elem_f32(p.bias[col]) : 0.f;
}

// The epilogue's factor on the product of row `row`: alpha times the row's
// quantisation scale (alpha alone without row scales or past M).
template <typename T>
__device__ __forceinline__ float row_factor(const GemmArgs<T>& p, int64_t row) {
    return (p.row_scale != nullptr && row < p.M) ? p.alpha * p.row_scale[row] : p.alpha;
}

// Quantisation scale of column `col`: 1 past N or without column scales.
template <typename T>
__device__ __forceinline__ float col_factor(const GemmArgs<T>& p, int64_t col) {
    return (p.col_scale != nullptr && col < p.N) ? p.col_scale[col] : 1.f;
}

// ---- LDS pipelines ----------------------------------------------------------

// Zero the bf16 elements at positions >= valid (0..8) of an 8-element chunk.
__device__ __forceinline__ u32x4 mask_tail(u32x4 v, int valid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t keep = (2 * q + 1 < valid) ? 0xffffffffu : (2 * q < valid ? 0x0000ffffu : 0u);
        v[q] &= keep;
    }
    return v;
}

// LDS byte address of a __shared__ object (what m0 expects).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// One global -> LDS copy of 16 bytes per lane: lane l's bytes land at
// lds + 16 l; out-of-range dwords (per the descriptor) land as zeros.
// Issued as inline assembly so that the compiler neither reorders LDS
// accesses across it nor inserts waits for it: the kernel's own vmcnt wait
// plus barrier (lds_barrier) is the only thing that consumes these copies.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(soff), "s"(lds) : "memory", "m0");
}

// The same with 4 bytes per lane (buffer_load_dword ... lds): lane l's dword
// lands at lds + 4 l. Global addresses need only 4-byte alignment.
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(soff), "s"(lds) : "memory", "m0");
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14).
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xC07F;

// Workgroup barrier ordering LDS traffic only: the release half retires this
// wave's LDS accesses, the acquire half keeps later LDS accesses below the
// barrier. LDS-destined buffer loads are NOT covered (they count in vmcnt):
// callers wait for those explicitly first.
__device__ __forceinline__ void lds_only_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier for a two-stage copy pipeline: this wave's LDS-destined copies have
// landed (vmcnt 0), then an LDS-only workgroup barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_only_barrier();
}

// ---- checking builds of the LDS pipelines -----------------------------------
//
// The library is also built twice more, with DG_LDS_CHECK set, and the tests
// require both builds to give the normal build's results bit for bit:
//   1 (poison): right after the barrier that retires an LDS stage (every read
//     of its previous contents done; the next write into it not yet issued),
//     the workgroup fills the stage with NaN. A read of a retired stage, or of
//     a stage whose copy has not landed yet, then sees NaN rather than stale
//     but plausible data, and the NaN reaches the output.
//   2 (synchronous copies): every batch of global -> LDS copies is preceded
//     by a barrier that retires all outstanding LDS reads and followed by a
//     wait for the copies and a barrier, so no copy is ever in flight while a
//     wave reads LDS: the order a single staging buffer would impose, with
//     none of the overlap that the pipelines' own waits have to protect.
// The normal build (0) compiles every hook to nothing.
#ifndef DG_LDS_CHECK
#define DG_LDS_CHECK 0
#endif
constexpr int kLdsCheck = DG_LDS_CHECK;

// Poison build: fill `bytes` (a multiple of 16) of LDS at `p` with NaN (all
// ones is a NaN in fp32 and in bf16), thread t of nt doing every nt-th
// 16-byte chunk, then a barrier so that no later write into the stage can be
// overtaken by the fill. Every thread of the workgroup must call it.
__device__ __forceinline__ void lds_retire(void* p, int bytes, int t, int nt) {
    if constexpr (kLdsCheck == 1) {
        for (int i = 16 * t; i < bytes; i += 16 * nt)
            *reinterpret_cast<u32x4*>(static_cast<char*>(p) + i) = u32x4{~0u, ~0u, ~0u, ~0u};
        lds_only_barrier();
    }
}

// Synchronous-copy build: the hooks around every call that issues copies
// (reached by every wave of the workgroup, copying or not).
__device__ __forceinline__ void copy_begin() {
    if constexpr (kLdsCheck == 2) lds_barrier();
}
__device__ __forceinline__ void copy_end() {
    if constexpr (kLdsCheck == 2) lds_barrier();
}

// ---- split of the last round of tiles ---------------------------------------
//
// The simplest form of stream-K: workgroups 0 .. full - 1 each own a whole
// tile (tiles 0 .. full - 1 of the raster order); each of the `tail`
// remaining tiles is cut into `parts` ranges of `cps` K slabs, one workgroup
// per range, whose fp32 partial tiles meet in a caller workspace laid out as
// [counters: one int per split tile, padded to 256 bytes][slots: tail x parts
// partial tiles].
struct TailSplit {
    int full;
    int tail;     // 0: no split
    int parts;
    int cps;
};

constexpr int kMaxSplitParts = 8;

// Tail split for `tiles` tiles of `nk` K slabs over `slots` resident
// workgroups, with ranges of at least `min_cps` slabs. Host only.
//   * A last round at most half full is cut into as many ranges as fill it:
//     one round of shorter ranges.
//   * A fuller last round (every tile, when there are fewer tiles than slots)
//     takes the number of ranges p in 2..8 that minimises its length in slab
//     times, ceil(tail p / slots) ceil(nk / p) + p fixup: the split units run
//     in ceil(tail p / slots) rounds, and each tile's last range reads its p
//     partial tiles back (`fixup` slab times each). Ranges span at least
//     `min_cps_full` slabs: shorter ones spend more on their own start and
//     epilogue than the model counts. It splits only when that saves at least
//     an eighth of the unsplit round's nk slabs. A negative `fixup` leaves
//     fuller rounds unsplit.
inline TailSplit plan_tail_split(int64_t tiles, int64_t nk, int64_t slots, int64_t min_cps = 1,
                                 double fixup = 0.25, int64_t min_cps_full = 16) {
    TailSplit t{(int)tiles, 0, 1, (int)nk};
    const int64_t tail = tiles % slots;
    if (tail == 0 || nk < 2 * min_cps) return t;
    int64_t parts = 1;
    if (2 * tail <= slots) {
        parts = slots / tail;
        if (parts > kMaxSplitParts) parts = kMaxSplitParts;
        if (parts > nk / min_cps) parts = nk / min_cps;
    } else {
        if (fixup < 0) return t;
        const int64_t floor_cps = min_cps > min_cps_full ? min_cps : min_cps_full;
        double best = (double)nk;
        for (int64_t p = 2; p <= kMaxSplitParts && p <= nk / floor_cps; ++p) {
            const int64_t rounds = (tail * p + slots - 1) / slots;
            const double cost = (double)(rounds * ((nk + p - 1) / p)) + (double)p * fixup;
            if (cost < best) {
                best = cost;
                parts = p;
            }
        }
        if (best > 0.875 * (double)nk) return t;
    }
    const int64_t cps = (nk + parts - 1) / parts;
    parts = (nk + cps - 1) / cps;                     // every range non-empty
    if (parts < 2) return t;
    t.full = (int)(tiles - tail);
    t.tail = (int)tail;
    t.parts = (int)parts;
    t.cps = (int)cps;
    return t;
}

// Workspace bytes of a split with bm x bn fp32 partial tiles.
inline size_t tail_workspace(const TailSplit& t, int bm, int bn) {
    if (t.tail == 0) return 0;
    return (size_t)((((int64_t)t.tail * 4 + 255) & ~(int64_t)255) +
                    (int64_t)t.tail * t.parts * bm * bn * 4);
}

// ---- workgroup -> output tile mapping ----------------------------------------
//
// The dispatcher hands workgroup w to XCD (w mod 8), and each of the 8 XCDs has
// its own L2. The linear id is first renumbered so that every XCD owns one
// contiguous run of ids; the run is then walked in groups of `group_m` tile
// rows, so the tiles that share an XCD also share A rows and B columns.
__device__ __forceinline__ int xcd_slot(int wg, int nwg) {
    constexpr int kXcds = 8;
    int per = nwg / kXcds, rem = nwg % kXcds;
    int xcd = wg % kXcds, idx = wg / kXcds;
    return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Tile (tm, tn) of linear id `id` walked in groups of `group_m` tile rows.
__device__ __forceinline__ void raster_tile(int id, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn) {
    int group = group_m * tiles_n;
    int gid = id / group;
    int first_m = gid * group_m;
    int gsz = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    int in_group = id - gid * group;
    // The divisions above run on the vector ALU; pin the (wave-uniform)
    // results to scalar registers so everything derived from them, buffer
    // descriptors included, stays scalar.
    tm = __builtin_amdgcn_readfirstlane(first_m + in_group % gsz);
    tn = __builtin_amdgcn_readfirstlane(in_group / gsz);
}

__device__ __forceinline__ void tile_coords(int wg, int nwg, int tiles_m, int tiles_n,
                                            int group_m, int& tm, int& tn) {
    raster_tile(xcd_slot(wg, nwg), tiles_m, tiles_n, group_m, tm, tn);
}

}  // namespace dg
