/*
 * dense_gemm_04_amd — dense GEMM for AMD Instinct MI355X (gfx950), C ABI.
 *
 * Operation (Blackwell BF16 GEMM notes, section 1.1: "C = Alpha*A*B + Beta*C"):
 *
 *     C(i,j) <- alpha * sum_k A(i,k) * B(k,j) + beta * C(i,j)
 *
 * for 0 <= i < M, 0 <= j < N, 0 <= k < K. All three matrices are ROW-MAJOR
 * with unit column stride and a leading dimension (the element distance
 * between the starts of two rows), as in the RTX 3090 SGEMM article's
 * indexing A[row*K + k], B[k*N + col] (section 2.1), generalised to
 * A(i,k) = A[i*lda + k], B(k,j) = B[k*ldb + j], C(i,j) = C[i*ldc + j].
 *
 * gemm_f32  : A, B, C are IEEE fp32; products and sums in fp32.
 * gemm_bf16 : A, B, C hold bf16 bit patterns (1 sign, 8 exponent, 7 mantissa
 *             bits; same notes, section 1.2). Products and sums are fp32;
 *             the result alpha*acc + beta*C is formed in fp32 and rounded once
 *             to bf16, to nearest with ties to even (same notes, sections 1.2
 *             and 6.3: accumulate in FP32, convert back to BF16 at the end).
 * alpha and beta are fp32 on both paths.
 *
 * Summation order over k is unspecified; results agree with an exact-product,
 * binary64-sum reference to within |alpha| * sum_k |A(i,k)||B(k,j)| *
 * (a small multiple of K * 2^-24) plus the output rounding.
 *
 * Special values of the arguments (BLAS convention):
 *   - M == 0 or N == 0: nothing is read or written.
 *   - beta == 0: C is write-only; its old contents (even NaN) are not read.
 *   - K == 0 or alpha == 0: A and B are not read; C <- beta * C
 *     (beta == 1 leaves C untouched and launches nothing).
 *
 * gemm_f32_op and gemm_bf16_op (below) also take transposed A or B.
 *
 * Ownership and memory: every pointer is a DEVICE pointer owned by the
 * caller, valid on the current HIP device for the duration of the work.
 * The library keeps no reference after the work completes and allocates no
 * device memory; the *_ws and *_bias_act entry points take a caller-owned
 * workspace instead, and gemm_bf16_ws_noalloc uses a static array that the
 * library's code object holds on each GPU. C must not overlap A, B or the
 * workspace (undefined results otherwise).
 *
 * Streams and errors: `stream` is a hipStream_t passed as void* (NULL = the
 * null stream). Calls are asynchronous: they validate the arguments, enqueue
 * one or more kernels on `stream` and return; completion and device-side
 * faults are observed at the caller's next synchronisation. On any error
 * status nothing has been enqueued. The library is reentrant (except that
 * gemm_bf16_ws_noalloc calls share one scratch per GPU); its global state is
 * a per-device cache of the device architecture and of the scratch address.
 */
#ifndef DENSE_GEMM_04_AMD_GEMM_H
#define DENSE_GEMM_04_AMD_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    /* A size is negative or above INT_MAX, a leading dimension is smaller
     * than max(1, row length), a matrix would span 2^60 bytes or more
     * ((rows - 1) * ld + cols elements), a pointer that must be read or
     * written is NULL, a pointer is not aligned to its element size, or
     * `variant` is unknown or does not apply to the call. */
    GEMM_ERR_INVALID_VALUE = 1,
    /* No HIP device is current, or it is not a gfx950 (MI355X-class) device. */
    GEMM_ERR_UNSUPPORTED_DEVICE = 2,
    /* The kernel launch was rejected by the HIP runtime (or the grid would
     * exceed 2^31 - 1 workgroups, which no matrix in device memory needs). */
    GEMM_ERR_LAUNCH = 3,
    /* gemm_bf16_ws_noalloc only: the shape's split-K workspace is larger than
     * GEMM_NOALLOC_SCRATCH_BYTES. Nothing is launched. */
    GEMM_ERR_SCRATCH_LIMIT = 4
} gemm_status_t;

/* Kernel family selection for the *_ex entry points. AUTO is what gemm_f32 and
 * gemm_bf16 use; the others force one family (for measurements and tests).
 * An fp32 AUTO call whose 128 x 128 tiles fill whole rounds of the MFMA
 * kernel and leave a last round partly full runs two kernels on one stream:
 * the MFMA kernel on whole rounds and GEMM_VARIANT_SMALL on the strip of
 * trailing columns (or rows) that held the last round's tiles (4095 x 4097:
 * C's last column). So does one whose 257 .. 511 tiles would put two tiles
 * on some compute units, when a model says the pair is faster: the MFMA
 * kernel then runs at most one tile per compute unit and the strip holds the
 * rest (2048 x 2560: columns 2048 .. 2559). A bf16 AUTO call with at least
 * one whole round of 256 x 256 tiles and a partly full last one likewise runs
 * the trailing columns (or rows) that hold the last round's tiles as a second
 * product when a model says the pair is faster (4352 x 4096: rows 4096 ..
 * 4351, on the few-tile kernel). gemm_plan reports the MFMA family for such
 * calls. */
typedef enum {
    GEMM_VARIANT_AUTO = 0,
    /* LDS-tiled MFMA kernel with 128-bit global loads; needs every pointer
     * 16-byte aligned and lda, ldb, ldc multiples of 16 bytes / element size. */
    GEMM_VARIANT_MFMA = 1,
    /* The MFMA kernels for rows that are not 16-byte aligned (RTX 3090 SGEMM
     * article, section 6.2: a fallback when float4 alignment does not hold);
     * any alignment and leading dimension. Where every base and row is
     * 4-byte aligned (always for fp32; bf16 with even lda, ldb, ldc) the
     * tiles of GEMM_VARIANT_MFMA are filled by 4-byte copies; otherwise (bf16
     * with an odd leading dimension or base) a kernel with unaligned 128-bit
     * and element-wise loads runs. Leading dimensions past the copies' 31-bit
     * offset range load through registers. AUTO picks this family whenever
     * the rows are not 16-byte aligned. */
    GEMM_VARIANT_GENERAL = 2,
    /* fp32 only: vector-FMA (non-matrix-core) kernel with per-thread register
     * micro-tiles, kept as a measured comparison (same article, sections 5.1-5.3). */
    GEMM_VARIANT_VALU = 3,
    /* bf16 only, M <= 128 with 16-byte rows (M <= 32 otherwise): small-M
     * kernel that streams B once (Blackwell BF16 GEMM notes, section 5.2:
     * small-batch GEMMs are bandwidth bound). AUTO takes it for such calls
     * except 65 .. 128 rows whose 64 x 64 tiles fit one round of compute
     * units (N <= 8192), with or without a workspace, and 33 .. 64 rows with
     * N x K <= 2^25 without one: those run faster on the MFMA family's
     * few-tile kernel. */
    GEMM_VARIANT_SKINNY = 4,
    /* fp32 only, any shape and alignment: few-tile kernel. Each workgroup owns
     * a 16 x 16, 32 x 32 or 64 x 64 tile of C and its waves split K between
     * them, adding their partial tiles in a fixed order (RTX 3090 SGEMM
     * article, section 3: K is walked in slices; here the slices run on
     * different waves). AUTO picks it when the 128 x 128 tiles of
     * GEMM_VARIANT_MFMA would leave most compute units idle: up to about 150
     * such tiles (fp32 256^3 has 4), fewer with a split-K workspace and long K. */
    GEMM_VARIANT_SMALL = 5
} gemm_variant_t;

/* fp32 GEMM. A: M x K (lda >= max(1,K)), B: K x N (ldb >= max(1,N)),
 * C: M x N (ldc >= max(1,N)); all fp32, 4-byte aligned. */
gemm_status_t gemm_f32(int64_t M, int64_t N, int64_t K, float alpha,
                       const float* A, int64_t lda, const float* B, int64_t ldb,
                       float beta, float* C, int64_t ldc, void* stream);

/* bf16 GEMM with fp32 accumulation. A, B, C hold bf16 bit patterns
 * (uint16_t), 2-byte aligned; shapes and leading dimensions as for gemm_f32. */
gemm_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, float alpha,
                        const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                        float beta, uint16_t* C, int64_t ldc, void* stream);

/* As above with an explicit kernel family (gemm_variant_t). A forced variant
 * whose preconditions do not hold returns GEMM_ERR_INVALID_VALUE. */
gemm_status_t gemm_f32_ex(int64_t M, int64_t N, int64_t K, float alpha,
                          const float* A, int64_t lda, const float* B, int64_t ldb,
                          float beta, float* C, int64_t ldc, void* stream, int variant);
gemm_status_t gemm_bf16_ex(int64_t M, int64_t N, int64_t K, float alpha,
                           const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                           float beta, uint16_t* C, int64_t ldc, void* stream, int variant);

/* Split-K for small M (RTX 3090 SGEMM article, section 7.2: cutting K into
 * pieces that run in parallel and summing their partial results brings more
 * multiprocessors to work). With M <= 128 one workgroup per 64-column strip of
 * C leaves half the GPU idle at N = 8192; a workspace gives each strip several
 * workgroups, each over a part of K: with row-major 16-byte rows and at least
 * 16 strips of 256 columns, a streaming kernel whose workgroups take
 * interleaved 32-row blocks of K (16 x 8192 x 8192: 32 strips x 8), otherwise
 * the small-M kernel over contiguous K segments. Only K >= 4096 splits:
 * shorter K runs unsplit, which is faster there. Each workgroup stores its
 * fp32 partial tile in the workspace, and the strip's last workgroup to
 * finish adds the partials in a fixed order (so results do not depend on
 * timing) and forms alpha * sum + beta * C.
 *
 * For M > 128 the tiled bf16 kernel splits the same way as the fp32 one (see
 * gemm_f32_ws), on 128 x 128 tiles: when fewer than half as many such tiles
 * as compute units, or a last round at most half full, would leave CUs idle,
 * each tile of that round is cut into up to 8 K ranges of at least 1024 k,
 * with 64 KB fp32 partial tiles. Products whose 64 x 64 tiles fit one round
 * of compute units and are at least as many as the split's workgroups run
 * on the few-tile kernel instead (K split over the waves of a workgroup, no
 * workspace): 1024 x 1024 x 4096 needs none. Products whose 256 x 256
 * tiles form one partly full round (129 .. 256 tiles) may run 128 x 128
 * tiles with a workspace instead, one round of them whole and the rest split,
 * when a model of the two says it pays (3072 x 3072: 512 tiles and 64 split),
 * unless B is stored N x K (then the workspace is left unused).
 *
 * gemm_bf16_workspace_size: workspace bytes gemm_bf16_ws needs to split this
 * shape; 0 when it would not split (small M: K below 4096, where the
 * unsplit kernels are at least as fast, or N already fills the GPU; M > 128:
 * no idle CUs, or K below 2048) or the sizes are invalid. Host only, no HIP call. Sized for a full MI355X (256 compute
 * units). */
size_t gemm_bf16_workspace_size(int64_t M, int64_t N, int64_t K);

/* gemm_bf16 with a workspace: device memory owned by the caller, 256-byte
 * aligned, at least gemm_bf16_workspace_size(M, N, K) bytes, and filled with
 * zeros before its first use (every call leaves it ready for the next). With
 * workspace == NULL (and workspace_bytes == 0) this is gemm_bf16. Calls that
 * share a workspace must not overlap in time (same stream, or ordered by the
 * caller). GEMM_ERR_INVALID_VALUE also when the workspace is misaligned, too
 * small, or NULL with a non-zero size. Alignment and shape rules otherwise as
 * for gemm_bf16; shapes that do not take the split leave the workspace unused. */
gemm_status_t gemm_bf16_ws(int64_t M, int64_t N, int64_t K, float alpha,
                           const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                           float beta, uint16_t* C, int64_t ldc,
                           void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * gemm_bf16_ws with the library's own scratch instead of a caller workspace.
 * Each GPU the library runs on holds one static scratch array of
 * GEMM_NOALLOC_SCRATCH_BYTES (32 MiB + 64 KiB) from the library's load until
 * the process ends. This call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); on its first use on a device it looks up that
 * device's array and enqueues one small kernel on `stream` that clears the
 * array's counters.
 * Results are those of gemm_bf16_ws with a workspace of
 * gemm_bf16_workspace_size(M, N, K) bytes (bit for bit). Shapes whose
 * workspace would exceed the scratch return GEMM_ERR_SCRATCH_LIMIT and
 * launch nothing (16 x 8192 x 8192 needs 4 MiB and 128 x 16384 x 8192 32 MiB,
 * which fit; 128 x 8256 x 8192 needs 33 MiB, which does not; shapes that
 * would not split need none and run as gemm_bf16). All calls on one GPU share its scratch: calls that overlap
 * in time on one GPU (different streams, or threads without ordering) race
 * and give undefined results; calls ordered on one stream are safe. Other
 * rules as for gemm_bf16. */
#define GEMM_NOALLOC_SCRATCH_BYTES (((size_t)32 << 20) + ((size_t)64 << 10))
gemm_status_t gemm_bf16_ws_noalloc(int64_t M, int64_t N, int64_t K, float alpha,
                                   const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                   float beta, uint16_t* C, int64_t ldc, void* stream);

/* Split-K for the last round of tiles (fp32). The fp32 kernel covers C with
 * 128 x 128 tiles, two resident workgroups per compute unit. When the tiles
 * leave a last round that is at most half full (4095 x 4097: 1056 tiles on
 * 512 slots leave 32 tiles for a third round), the tiles of that round are
 * cut into up to 8 ranges of K (RTX 3090 SGEMM article, section 7.2:
 * splitting K to bring more multiprocessors to work). Each range's fp32
 * partial tile goes to the workspace and the last range to finish adds them
 * in a fixed order before the alpha/beta epilogue. Full tiles are computed as
 * in gemm_f32. A fuller last round is split too when a model of its length
 * says the split ranges finish sooner. Products with few tiles run on the
 * few-tile kernel (GEMM_VARIANT_SMALL), which splits K inside each workgroup
 * and needs no workspace, unless they hold at least 2^18 tile-k (128 x 128
 * tiles times K), where splitting over workgroups wins.
 *
 * gemm_f32_workspace_size: workspace bytes gemm_f32_ws needs for this shape
 * on a full MI355X (256 compute units); 0 when it would not split (no last
 * round, or one the model leaves whole, or K below two 32-deep slabs), when
 * the few-tile kernel takes the shape or a strip of it (see
 * GEMM_VARIANT_AUTO), or when the sizes are invalid. Host only, no HIP call. On a device with fewer compute
 * units the split is planned for that device and uses the workspace only if
 * it is large enough.
 *
 * gemm_f32_ws: gemm_f32 with such a workspace; the workspace contract
 * (alignment, zero fill, no overlapping calls, NULL with size 0) is that of
 * gemm_bf16_ws. */
size_t gemm_f32_workspace_size(int64_t M, int64_t N, int64_t K);
gemm_status_t gemm_f32_ws(int64_t M, int64_t N, int64_t K, float alpha,
                          const float* A, int64_t lda, const float* B, int64_t ldb,
                          float beta, float* C, int64_t ldc,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Fused epilogues (Blackwell BF16 GEMM notes, section 3.3: GELU, residual
 * adds and scaling are the work a GEMM epilogue takes on; Z-Turbo tuning
 * page, section 2.1: one kernel that applies GELU in its tanh form and then
 * adds the residual, instead of separate passes over memory):
 *
 *     C(i,j) <- act(alpha * sum_k A(i,k) * B(k,j) + bias[j]) + beta * C(i,j)
 *
 * The bias is added and the activation applied before the beta * C term,
 * which plays the residual. Everything is formed in fp32 from the fp32
 * accumulator and rounded once at the end (to bf16 on the bf16 path). */
typedef enum {
    GEMM_ACT_NONE = 0,
    /* max(x, 0) */
    GEMM_ACT_RELU = 1,
    /* GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))),
     * evaluated in fp32 as x / (1 + exp(-2 sqrt(2/pi) (x + 0.044715 x^3))),
     * the same function, with the hardware exp2 and reciprocal (a few ulp of
     * relative error on top of the pre-activation's). */
    GEMM_ACT_GELU_TANH = 2
} gemm_act_t;

/* GEMM with a bias and activation epilogue.
 * bias: device pointer to N elements of the matrices' type (fp32, or bf16
 *       bit patterns), element-aligned; NULL for no bias.
 * act:  a gemm_act_t value; anything else is GEMM_ERR_INVALID_VALUE.
 * workspace, workspace_bytes: as for gemm_f32_ws / gemm_bf16_ws (NULL and 0
 *       for none); with one, the same shapes take the split-K paths.
 * Shapes, alignment, streams and errors otherwise as for gemm_f32 / gemm_bf16.
 * Special values: M == 0 or N == 0 does nothing; K == 0 or alpha == 0 stores
 * act(bias[j]) + beta * C(i,j) without reading A or B (with no bias that is
 * beta * C, since every activation maps 0 to 0, and beta == 1 then launches
 * nothing); beta == 0 never reads C. With bias == NULL and GEMM_ACT_NONE the
 * results are bit-identical to gemm_f32 / gemm_bf16 (and their _ws forms). */
gemm_status_t gemm_f32_bias_act(int64_t M, int64_t N, int64_t K, float alpha,
                                const float* A, int64_t lda, const float* B, int64_t ldb,
                                float beta, float* C, int64_t ldc, const float* bias, int act,
                                void* workspace, size_t workspace_bytes, void* stream);
gemm_status_t gemm_bf16_bias_act(int64_t M, int64_t N, int64_t K, float alpha,
                                 const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                                 float beta, uint16_t* C, int64_t ldc, const uint16_t* bias,
                                 int act, void* workspace, size_t workspace_bytes, void* stream);

/* Transposed operands: C <- act(alpha * op(A) op(B) + bias) + beta * C, where
 * op(X) is X (GEMM_OP_N) or its transpose (GEMM_OP_T). op(A) is M x K and
 * op(B) is K x N:
 *   opa == GEMM_OP_N: A is M x K row-major, A(i,k) = A[i*lda + k], lda >= max(1,K);
 *   opa == GEMM_OP_T: A is stored K x M row-major, op(A)(i,k) = A[k*lda + i],
 *                     lda >= max(1,M);
 *   opb == GEMM_OP_N: B is K x N row-major, B(k,j) = B[k*ldb + j], ldb >= max(1,N);
 *   opb == GEMM_OP_T: B is stored N x K row-major, op(B)(k,j) = B[j*ldb + k],
 *                     ldb >= max(1,K). A column-major K x N matrix with leading
 *                     dimension ldb is exactly this storage.
 * The backward pass of y = x W needs both forms (dx = dy W^T, dW = x^T dy),
 * and the CUTLASS example of the Blackwell BF16 GEMM notes (section 3.3)
 * takes B column-major. bias, act, workspace and all other rules are those of
 * gemm_*_bias_act (with opa == opb == GEMM_OP_N the two calls are the same);
 * an opa or opb other than the two codes is GEMM_ERR_INVALID_VALUE. The
 * small-M kernel (bf16, M <= 128) reads a row-major A and a row-major or,
 * with 16-byte rows, transposed B; other transposed small-M calls, like the
 * 65 .. 128-row calls that GEMM_VARIANT_SKINNY describes, run on the tiled
 * kernels. */
typedef enum { GEMM_OP_N = 0, GEMM_OP_T = 1 } gemm_op_t;

gemm_status_t gemm_f32_op(int opa, int opb, int64_t M, int64_t N, int64_t K, float alpha,
                          const float* A, int64_t lda, const float* B, int64_t ldb,
                          float beta, float* C, int64_t ldc, const float* bias, int act,
                          void* workspace, size_t workspace_bytes, void* stream);
gemm_status_t gemm_bf16_op(int opa, int opb, int64_t M, int64_t N, int64_t K, float alpha,
                           const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                           float beta, uint16_t* C, int64_t ldc, const uint16_t* bias, int act,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Quantisation scales (Blackwell BF16 GEMM notes, section 3.3: quantisation
 * scaling is epilogue work beside GELU and the residual):
 *
 *     C(i,j) <- act(alpha * row_scale[i] * col_scale[j] * sum_k op(A)(i,k) op(B)(k,j)
 *                   + bias[j]) + beta * C(i,j)
 *
 * row_scale: device pointer to M fp32 values (the dequantisation factor of
 *            each row of op(A), e.g. of a per-token quantised activation), or
 *            NULL for 1;
 * col_scale: device pointer to N fp32 values (the factor of each column of
 *            op(B), e.g. of a per-channel quantised weight), or NULL for 1.
 * Both 4-byte aligned (GEMM_ERR_INVALID_VALUE otherwise). The factors multiply
 * the fp32 accumulator in the epilogue, before the bias, the activation and
 * the beta term, and cost no extra pass over memory; they apply to the same
 * operand types as the other entry points (fp32 or bf16 operands, fp32
 * accumulation). opa, opb, bias, act, workspace and every other rule are
 * those of gemm_*_op; with both scales NULL the two calls are the same. When
 * K == 0 or alpha == 0 the product term is zero and the scales are not read. */
gemm_status_t gemm_f32_scaled(int opa, int opb, int64_t M, int64_t N, int64_t K, float alpha,
                              const float* A, int64_t lda, const float* B, int64_t ldb,
                              float beta, float* C, int64_t ldc, const float* row_scale,
                              const float* col_scale, const float* bias, int act,
                              void* workspace, size_t workspace_bytes, void* stream);
gemm_status_t gemm_bf16_scaled(int opa, int opb, int64_t M, int64_t N, int64_t K, float alpha,
                               const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                               float beta, uint16_t* C, int64_t ldc, const float* row_scale,
                               const float* col_scale, const uint16_t* bias, int act,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Host-only planning (no HIP call): the variant a call with these arguments
 * would run (a gemm_variant_t value; GEMM_VARIANT_AUTO when the call would
 * launch no GEMM kernel), or -1 when the arguments are invalid. `elem_bytes`
 * is 4 (fp32) or 2 (bf16); pointers are used only for their alignment. The
 * operands are taken as row-major (gemm_f32 / gemm_bf16 / their _ex forms);
 * with transposed operands (gemm_*_op) a bf16 small-M call may run on the
 * tiled families instead (see gemm_bf16_op). */
int gemm_plan(int elem_bytes, int64_t M, int64_t N, int64_t K, float alpha,
              const void* A, int64_t lda, const void* B, int64_t ldb,
              float beta, const void* C, int64_t ldc, int variant);

/* Static string for a gemm_status_t value ("unknown status" otherwise). */
const char* gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_04_AMD_GEMM_H */
