// Small-M bf16 GEMM with split K over a caller workspace, B row-major with
// 16-byte rows: C = alpha * A * B + beta * C, fp32 accumulation.
//
// A GEMM with a few rows of A is bound by reading B once from HBM (Blackwell
// BF16 GEMM notes, section 5.2: small batches leave nothing to reuse), so the
// whole design is the order in which B is read. Measured on MI355X with B
// 8192 x 8192 (128 MiB, LDS-destined 128-bit copies, no arithmetic):
//   * 64-column strips (128-byte row segments) with K split into contiguous
//     halves: 5.0-5.2 TB/s;
//   * 256-column strips, contiguous K segments: 5.4 TB/s;
//   * 256-column strips with K interleaved: workgroup q of a strip (its
//     phase, of P) takes the 32-row blocks q, q + P, q + 2P, ..., so that the
//     chip as a whole reads one window of consecutive rows at a time: 5.85
//     TB/s, close to the best plain streaming read measured (6.7). Finer
//     interleaving (8-row groups) streams B 2.5% faster, but then each chunk
//     of A is four separate 16-byte pieces per row, and gathering them cost
//     more than that gain.
// This kernel reads B that way: 256 workgroups for 16 x 8192 x 8192 (32
// strips x 8 phases), each reading 512 contiguous bytes of every row it owns.
//
// Per workgroup (4 waves): chunks of 32 rows of B ([32][256], 16 KB) and the
// matching 32 columns of A ([16 MB][32]) stream into a ring of LDS stages
// through LDS-destined buffer loads, kStages - 1 chunks ahead of their use.
// One chunk is one MFMA k step: wave w multiplies A's 16-row blocks by its
// 64 columns of B (transposing LDS reads, as in the tiled kernel), so no
// partial sums cross waves. Each workgroup then stores its fp32 partial tile
// in the workspace, and the strip's last workgroup to finish adds the P
// partials in phase order (results do not depend on timing) and applies the
// epilogue.
//
// Edges: A rows past M and B rows past K arrive as zeros through the
// descriptor bounds; k past K inside A's rows (the next row's values) is
// masked in registers; B columns past N feed only output columns that are
// never stored.

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace dg {
namespace {

constexpr int kNT = 256;          // 4 waves
constexpr int kSW = 256;          // strip width: 512-byte row segments of B
constexpr int kRC = 32;           // rows of B per chunk: one MFMA k step
constexpr int kStages = 4;
constexpr int kWaveCols = kSW / 4;
constexpr int kMaxPhases = 16;

template <int MB> struct Stream {
    static constexpr int kBStage = kRC * kSW;                 // bf16 [32][256]
    static constexpr int kAStage = 16 * MB * kRC;             // bf16 [16 MB][32]
    static constexpr int kBCopies = kBStage * 2 / 1024 / 4;   // 1 KB copies per wave
    // A: one 1 KB copy per 16-row block, issued by wave J mod 4. The wait
    // counts use the fewest copies any wave issues per chunk, so every wave
    // waits at least as long as it must.
    static constexpr int kMinCopies = kBCopies + MB / 4;
    static constexpr int kE = MB * 4;                         // f32x4 accumulators per lane
};

// B stage rows are 512 bytes (32 chunks of 16 bytes); chunk c of row k sits in
// slot c ^ b_swz(k). The XOR term depends on k mod 4 and k / 8 mod 4, the row
// indices that vary across the 16-lane groups of a transposing read, so the
// lanes of each read phase hit distinct banks.
__device__ __forceinline__ int b_swz(int k) { return ((k & 3) | (((k >> 3) & 3) << 2)) << 1; }
__device__ __forceinline__ int b_off(int k, int c) { return k * kSW + ((c ^ b_swz(k)) << 3); }
// A stage rows are 64 bytes (4 chunks); chunk c of row r sits in slot
// c ^ (r / 4 mod 4), so the 16 rows of a fragment read cover all banks.
__device__ __forceinline__ int a_off(int r, int c) { return r * kRC + ((c ^ ((r >> 2) & 3)) << 3); }

template <int MB, bool EPI>
__global__ __launch_bounds__(kNT, 1)
void gemm_bf16_stream_kernel(GemmArgs<uint16_t> p, StreamWork wk, unsigned char* ws) {
    using S = Stream<MB>;
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[kStages * S::kBStage];
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[kStages * S::kAStage];
    __shared__ int last_flag;

    const int64_t M = p.M, N = p.N, K = p.K, lda = p.lda, ldb = p.ldb;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int pl = lane & 15, g = lane >> 4;
    const int q = __builtin_amdgcn_readfirstlane((int)blockIdx.x / wk.strips);
    const int strip = __builtin_amdgcn_readfirstlane((int)blockIdx.x - q * wk.strips);
    const int64_t n0 = (int64_t)strip * kSW;
    // This workgroup's 32-row blocks: q, q + P, ... below nblk (at least one);
    // chunk c is block q + P c.
    const int64_t P = wk.phases;
    const int64_t nc = (wk.nblk - q + P - 1) / P;
    auto chunk_k = [&](int64_t c) { return kRC * (q + P * c); };

    // A descriptor: rows 0 .. M - 1, ending at element K of the last row
    // (rounded up to its 16-byte chunk), so rows past M arrive as zeros.
    const uint32_t a_bytes = (uint32_t)((((M - 1) * lda + K) * 2 + 15) & ~(int64_t)15);
    const rsrc_t a_desc = make_rsrc(p.A, a_bytes);

    // Copies are 1 KB; lane l fills bytes [16 l, 16 l + 16) of the copy's
    // destination, and each copy's whole offset sits in the per-lane offset,
    // which the descriptor's range check covers.
    //   B: copy I fills rows 2 I, 2 I + 1; lane -> row 2 I + l / 32, slot
    //      l % 32 holding chunk (l % 32) ^ b_swz(row).
    //   A: copy J fills rows 16 J .. 16 J + 15; lane -> row 16 J + l / 4, slot
    //      l % 4 holding chunk (l % 4) ^ (row / 4 mod 4).
    auto dma = [&](int64_t c, int stage) {
        const int64_t k0 = chunk_k(c);
        const uint32_t Bs = __builtin_amdgcn_readfirstlane(lds_addr(lds_b + stage * S::kBStage));
        const uint32_t As = __builtin_amdgcn_readfirstlane(lds_addr(lds_a + stage * S::kAStage));
        // Rows k0 .. K - 1 of B, ending after column N of row K - 1: rows past
        // K arrive as zeros.
        const int64_t rem = (((K - k0 - 1) * ldb + (N - n0)) * 2 + 15) & ~(int64_t)15;
        const uint32_t b_bytes = rem < ((int64_t)1 << 31) ? (uint32_t)rem : 0x80000000u;
        const rsrc_t b_desc = make_rsrc(p.B + k0 * ldb + n0, b_bytes);
#pragma unroll
        for (int i = 0; i < S::kBCopies; ++i) {
            const int I = wave * S::kBCopies + i;
            const int row = 2 * I + (lane >> 5);
            const int c16 = (lane & 31) ^ b_swz(row);
            dma16(b_desc, (uint32_t)(row * ldb * 2 + c16 * 16), 0, Bs + I * 1024);
        }
#pragma unroll
        for (int J = 0; J < MB; ++J) {
            if (J % 4 != wave) continue;
            const int row = 16 * J + (lane >> 2);
            const int c16 = (lane & 3) ^ ((row >> 2) & 3);
            dma16(a_desc, (uint32_t)((row * lda + k0 + c16 * 8) * 2), 0, As + J * 1024);
        }
    };

    f32x4 acc[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    // Transposing-read role: lane 4 r + x of a 16-lane group addresses row r
    // (and r + 4) and columns 4 x .. 4 x + 3 of a 4 x 16 block.
    const int tr_row = pl >> 2, tr_col = (pl & 3) * 4;
    auto compute = [&](int64_t c, int stage) {
        const uint16_t* Bs = lds_b + stage * S::kBStage;
        const uint16_t* As = lds_a + stage * S::kAStage;
        bf16x8 fa[MB], fb[4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            fa[mb] = *reinterpret_cast<const bf16x8*>(As + a_off(16 * mb + pl, g));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = kWaveCols * wave + 16 * j + tr_col;
            const int r0 = 8 * g + tr_row;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(Bs + b_off(r0, col >> 3) + (col & 7)));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(Bs + b_off(r0 + 4, col >> 3) + (col & 7)));
            fb[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        // Ragged K: A(m, k >= K) holds the next row's values (B's rows past K
        // are zeros, but 0 * NaN would not be).
        const int64_t kfirst = chunk_k(c) + 8 * g;
        if (kfirst + 8 > K) {
            const int valid = kfirst >= K ? 0 : (int)(K - kfirst);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                fa[mb] = __builtin_bit_cast(bf16x8, mask_tail(__builtin_bit_cast(u32x4, fa[mb]), valid));
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[mb], acc[mb][j], 0, 0, 0);
    };

    // Ring of kStages chunk slots; copies run kStages - 1 chunks ahead. At
    // chunk c each wave waits for its own copies of chunk c (later ones may
    // stay in flight), then the barrier publishes chunk c and retires every
    // read of chunk c - 1, whose slot the copy for chunk c + kStages - 1 reuses.
    // Checking builds (no-ops otherwise): every slot starts as NaN and is
    // refilled with NaN once retired (poison); copies are bracketed by
    // barriers (synchronous copies).
    auto retire = [&](int slot) {
        if constexpr (kLdsCheck == 1) {
            lds_retire(lds_b + slot * S::kBStage, S::kBStage * 2, t, kNT);
            lds_retire(lds_a + slot * S::kAStage, S::kAStage * 2, t, kNT);
        }
    };
    for (int slot = 0; slot < kStages; ++slot) retire(slot);
    const int64_t pre = nc < kStages - 1 ? nc : kStages - 1;
    for (int64_t c = 0; c < pre; ++c) {
        copy_begin();
        dma(c, (int)c);
        copy_end();
    }
    int stage = 0;
    for (int64_t c = 0; c < nc; ++c) {
        if (c + kStages - 2 <= nc - 1)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((kStages - 2) * S::kMinCopies));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        lds_only_barrier();
        const int prev = stage == 0 ? kStages - 1 : stage - 1;   // slot of chunk c - 1, retired
        if (c > 0) retire(prev);
        if (c + kStages - 1 < nc) {
            copy_begin();
            dma(c + kStages - 1, prev);
            copy_end();
        }
        compute(c, stage);
        stage = stage + 1 == kStages ? 0 : stage + 1;
    }

    if (wk.phases > 1) {
        // Store this phase's partial tile with device-coherent stores (sc1:
        // written through the per-XCD L2), count in once they have completed,
        // and let the strip's last arrival read the phases back the same way
        // and add them in phase order. Value e of thread t sits at byte
        // (e * kNT + t) * 16 of a slot.
        constexpr int kSc1 = 16;                           // cache-policy bit sc1
        constexpr int kSlotBytes = S::kE * kNT * 16;
        int* counters = reinterpret_cast<int*>(ws);
        const unsigned char* slots = ws + (((int64_t)wk.strips * 4 + 255) & ~(int64_t)255);
        const rsrc_t sd = make_rsrc(slots + (int64_t)strip * wk.phases * kSlotBytes,
                                    (uint32_t)(wk.phases * kSlotBytes));
        auto voff = [&](int ph, int e) { return (uint32_t)(ph * kSlotBytes + (e * kNT + t) * 16); };
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[mb][j]), sd,
                                                       voff(q, mb * 4 + j), 0, kSc1);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        if (t == 0)
            last_flag = __hip_atomic_fetch_add(counters + strip, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) == wk.phases - 1;
        __syncthreads();
        if (!last_flag) return;
        // Every phase's values come back in batches loaded all at once, one
        // round trip per batch (loading and adding them value by value cost
        // 1.3 us more at 16 x 8192 x 8192, selecting loads by phase 0.85 us):
        // 8 or 16 slots per value whether or not the strip has that many
        // phases, since slots past the descriptor's P read as zeros. Each
        // sum runs in phase order.
        auto reduce = [&](auto batch_tag, auto slots_tag) {
            constexpr int kB = decltype(batch_tag)::value, kP = decltype(slots_tag)::value;
#pragma unroll
            for (int e0 = 0; e0 < S::kE; e0 += kB) {
                f32x4 v[kB][kP];
#pragma unroll
                for (int b = 0; b < kB; ++b)
#pragma unroll
                    for (int ph = 0; ph < kP; ++ph)
                        if (e0 + b < S::kE)
                            v[b][ph] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                     sd, voff(ph, e0 + b), 0, kSc1));
#pragma unroll
                for (int b = 0; b < kB; ++b) {
                    if (e0 + b >= S::kE) continue;
                    f32x4 sum = v[b][0];
#pragma unroll
                    for (int ph = 1; ph < kP; ++ph) sum += v[b][ph];
                    acc[(e0 + b) / 4][(e0 + b) % 4] = sum;
                }
            }
        };
        if (P <= 8)
            reduce(std::integral_constant<int, (S::kE < 4 ? S::kE : 4)>{}, std::integral_constant<int, 8>{});
        else
            reduce(std::integral_constant<int, 2>{}, std::integral_constant<int, kMaxPhases>{});
        // Leave the counter at zero for the next call that uses this workspace.
        if (t == 0) __hip_atomic_store(counters + strip, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // Epilogue: acc[mb][j] register r holds C(16 mb + pl, n0 + 64 wave + 16 j + 4 g + r).
    const float beta = p.beta;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int64_t row = 16 * mb + pl;
        if (row >= M) continue;
        uint16_t* crow = p.C + row * p.ldc;
        const float fr = EPI ? row_factor(p, row) : p.alpha;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + kWaveCols * wave + 16 * j + 4 * g;
            if (col >= N) continue;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                v[r] = fr * acc[mb][j][r];
                if constexpr (EPI) v[r] = activate(v[r] * col_factor(p, col + r) + bias_at(p, col + r), p.act);
            }
            if (col + 4 <= N) {
                // Four bf16 = 8 bytes, aligned: rows are 16-byte aligned and col % 4 == 0.
                u32x2* dst = reinterpret_cast<u32x2*>(crow + col);
                if (beta != 0.f) {
                    const u32x2 c0 = *dst;
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

// Row blocks of 16 for M rows: 1, 2, 4 or 8.
int stream_blocks(int64_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8; }

}  // namespace

// The streaming split: 256-column strips, and P phases per strip so that
// strips x P is at least the 256 compute units of an MI355X, up to 16 phases
// (every phase's 16 MB x 256 fp32 partial is read back by the strip's last
// workgroup) and with at least four 32-row blocks of K per phase (shorter
// phases would spend more on the partials than they save). It applies only
// when that reaches the full chip (N > 15 strips) with at least two phases.
StreamWork plan_stream(int64_t N, int64_t K) {
    StreamWork w{0, 0, 0};
    const int64_t strips = (N + kSW - 1) / kSW;
    const int64_t nblk = (K + kRC - 1) / kRC;
    if (strips < 16 || strips > kMaxGrid / kMaxPhases) return w;
    int64_t phases = (256 + strips - 1) / strips;
    if (phases > kMaxPhases) phases = kMaxPhases;
    if (phases > nblk / 4) phases = nblk / 4;
    if (phases < 2) return w;
    w.strips = (int)strips;
    w.phases = (int)phases;
    w.nblk = nblk > 0x7fffffff ? 0x7fffffff : (int)nblk;
    return w;
}

size_t bf16_stream_workspace(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > kSkinnyMaxM || N < 1 || K < 1) return 0;
    const StreamWork w = plan_stream(N, K);
    if (w.phases == 0) return 0;
    const int64_t mb = stream_blocks(M);
    return (size_t)((((int64_t)w.strips * 4 + 255) & ~(int64_t)255) +
                    (int64_t)w.strips * w.phases * mb * 4 * kNT * 16);
}

// True when every buffer offset the kernel forms fits in 31 bits: B copies
// reach 32 rows below a chunk's first row plus a 512-byte segment, A copies
// row 16 MB - 1 (rows past M included) and one chunk past K.
bool bf16_stream_fits(const GemmArgs<uint16_t>& a) {
    const int64_t lim = (int64_t)1 << 31;
    return (kRC * a.ldb + kSW) * 2 < lim && (16 * stream_blocks(a.M) * a.lda + a.K + kRC) * 2 < lim;
}

hipError_t launch_bf16_stream(const GemmArgs<uint16_t>& a, void* ws, hipStream_t s) {
    GemmArgs<uint16_t> args = a;
    StreamWork w = plan_stream(a.N, a.K);
    unsigned char* wsp = static_cast<unsigned char*>(ws);
    void* kargs[] = {&args, &w, &wsp};
    const bool epi = has_epilogue(a);
    const int mb = stream_blocks(a.M);
#define DG_STREAM(MB) (epi ? (const void*)&gemm_bf16_stream_kernel<MB, true> \
                           : (const void*)&gemm_bf16_stream_kernel<MB, false>)
    const void* fn = mb == 1 ? DG_STREAM(1) : mb == 2 ? DG_STREAM(2) : mb == 4 ? DG_STREAM(4)
                                                                              : DG_STREAM(8);
#undef DG_STREAM
    return hipLaunchKernel(fn, dim3((unsigned)(w.strips * w.phases)), dim3(kNT), kargs, 0, s);
}

}  // namespace dg
