/*
 * CPU oracle for C = alpha * A * B + beta * C0, row-major.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. It shares no source,
 * header or helper with the HIP library.
 *
 * What it computes (the plain definition, nothing faster):
 *   - GEMM is C = Alpha*A*B + Beta*C (Blackwell BF16 GEMM notes, section 1.1).
 *   - BF16 is 1 sign, 8 exponent and 7 mantissa bits, i.e. the top half of an
 *     fp32 word; products are accumulated in a wider format (same notes,
 *     section 1.2). Here the widening is exact: bits << 16 gives the fp32
 *     value, and every fp32 value is exact in binary64.
 *   - Every optimised kernel is checked in full against a plain GEMM that
 *     walks k in order for each output (RTX 3090 SGEMM article, section 2.1
 *     for the one-output-per-thread loop and section 2.2 for its role as the
 *     correctness baseline).
 *
 * For each requested entry (i, j):
 *   s   = sum_{k=0..K-1} a_ik * b_kj      in binary64, k increasing
 *   r   = alpha * s + beta * c0_ij         (the beta term is skipped when beta == 0,
 *                                           so C0 is never read then)
 *   D   = |alpha| * sum_k |a_ik| * |b_kj| + |beta| * |c0_ij|
 * r and D are returned unrounded.
 *
 * The epilogue variant (oracle_gemm_*_epi) adds what a GEMM epilogue can fuse
 * (Blackwell BF16 GEMM notes, section 3.3: bias, GELU, residual; the Z-Turbo
 * tuning page, section 2.1: a fused kernel that applies GELU in its tanh form
 * and then adds the residual):
 *   z   = alpha * s + bias_j               (no bias term when bias is NULL)
 *   r   = act(z) + beta * c0_ij            (c0 is the residual)
 *   D   = L * (|alpha| * sum_k |a_ik| * |b_kj| + |bias_j|) + |beta| * |c0_ij|
 * with act one of: identity; ReLU, max(z, 0); GELU, tanh form,
 *   0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))),
 * and L a bound on |act'| (1, 1 and ORACLE_GELU_SLOPE), so that an error in z
 * moves r by at most L times as much. The products of two fp32 (or bf16) values
 * are exact in binary64, so contraction into an FMA cannot change r; the
 * file is still built with -ffp-contract=off and without -ffast-math.
 *
 * The scaled variant (oracle_gemm_*_scaled) adds the third kind of epilogue
 * work the Blackwell BF16 GEMM notes name in section 3.3, quantisation
 * scaling: one fp32 factor per row of A (u_i) and one per column of B (v_j),
 * the dequantisation scales of a row-wise and a column-wise quantised operand,
 * which multiply the product before anything else is added:
 *   z   = alpha * u_i * v_j * s + bias_j
 *   r   = act(z) + beta * c0_ij
 *   D   = L * (|alpha * u_i * v_j| * sum_k |a_ik| * |b_kj| + |bias_j|) + |beta| * |c0_ij|
 * A missing scale vector (NULL) is the factor 1 for every row (column). The
 * factor alpha * u_i * v_j is formed in binary64 (one rounding, at 2^-53).
 *
 * Rows are independent and are spread over OpenMP threads; within a row the
 * loop order is k outer, j inner, which keeps every entry's own sum in
 * increasing k (the row-wise loop of the CPU matmul in the CUDA shared-memory
 * chapters, section 3.3, without its k blocking).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEM 2

static double from_f32(const void* base, int64_t idx) {
    return (double)((const float*)base)[idx];
}

/* bf16 storage: the value is the fp32 word whose top 16 bits are the pattern. */
static double from_bf16(const void* base, int64_t idx) {
    uint32_t word = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

typedef double (*load_fn)(const void*, int64_t);

#define ACT_NONE 0
#define ACT_RELU 1
#define ACT_GELU_TANH 2

/* Upper bound on the slope of the tanh-form GELU over the reals (the maximum
 * is about 1.1289, near z = 1.5). */
#define ORACLE_GELU_SLOPE 1.13

static double activate(double z, int act) {
    if (act == ACT_RELU) return z > 0.0 ? z : 0.0;
    if (act == ACT_GELU_TANH)
        return 0.5 * z * (1.0 + tanh(sqrt(2.0 / acos(-1.0)) * (z + 0.044715 * z * z * z)));
    return z;
}

static double act_slope(int act) { return act == ACT_GELU_TANH ? ORACLE_GELU_SLOPE : 1.0; }

double oracle_activate(double z, int act) { return activate(z, act); }

double oracle_bf16_bits_to_double(uint16_t bits) { return from_bf16(&bits, 0); }

static int oracle_gemm(load_fn load, int64_t M, int64_t N, int64_t K, double alpha,
                       const void* A, int64_t lda, const void* B, int64_t ldb,
                       double beta, const void* C0, int64_t ldc,
                       const float* row_scale, const float* col_scale,
                       const void* bias, int act,
                       const int64_t* rows, int64_t nrows,
                       const int64_t* cols, int64_t ncols,
                       double* R, double* D, int nthreads) {
    if (M < 0 || N < 0 || K < 0) return ORACLE_BAD_ARG;
    if (act < ACT_NONE || act > ACT_GELU_TANH) return ORACLE_BAD_ARG;
    if (rows == NULL) nrows = M;
    if (cols == NULL) ncols = N;
    if (nrows < 0 || ncols < 0) return ORACLE_BAD_ARG;
    for (int64_t t = 0; rows && t < nrows; ++t)
        if (rows[t] < 0 || rows[t] >= M) return ORACLE_BAD_ARG;
    for (int64_t t = 0; cols && t < ncols; ++t)
        if (cols[t] < 0 || cols[t] >= N) return ORACLE_BAD_ARG;
    if (nrows == 0 || ncols == 0) return ORACLE_OK;
    if (K > 0 && (A == NULL || B == NULL || lda < K || ldb < N)) return ORACLE_BAD_ARG;
    if (beta != 0.0 && (C0 == NULL || ldc < N)) return ORACLE_BAD_ARG;

    /* The requested columns of B, widened once: Bw[k * ncols + c] = b(k, col_c). */
    double* Bw = NULL;
    if (K > 0) {
        Bw = (double*)malloc(sizeof(double) * (size_t)K * (size_t)ncols);
        if (!Bw) return ORACLE_NO_MEM;
        for (int64_t k = 0; k < K; ++k)
            for (int64_t c = 0; c < ncols; ++c) {
                int64_t j = cols ? cols[c] : c;
                Bw[k * ncols + c] = load(B, k * ldb + j);
            }
    }

    int status = ORACLE_OK;
    int team = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(team)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)ncols);
        double* mag = (double*)malloc(sizeof(double) * (size_t)ncols);
        if (!s || !mag) {
#pragma omp atomic write
            status = ORACLE_NO_MEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t) {
            if (!s || !mag) continue;
            int64_t i = rows ? rows[t] : t;
            for (int64_t c = 0; c < ncols; ++c) { s[c] = 0.0; mag[c] = 0.0; }
            for (int64_t k = 0; k < K; ++k) {
                double a = load(A, i * lda + k);
                const double* brow = Bw + k * ncols;
                for (int64_t c = 0; c < ncols; ++c) {
                    s[c] += a * brow[c];
                    mag[c] += fabs(a) * fabs(brow[c]);
                }
            }
            /* The product's factor for this row: alpha * u_i (u_i = 1 without row scales). */
            double f_row = alpha * (row_scale ? (double)row_scale[i] : 1.0);
            for (int64_t c = 0; c < ncols; ++c) {
                int64_t j = cols ? cols[c] : c;
                double f = f_row * (col_scale ? (double)col_scale[j] : 1.0);
                double r = f * s[c];
                double d = fabs(f) * mag[c];
                if (bias) {
                    double b = load(bias, j);
                    r += b;
                    d += fabs(b);
                }
                r = activate(r, act);
                d *= act_slope(act);
                if (beta != 0.0) {
                    double c0 = load(C0, i * ldc + j);
                    r += beta * c0;
                    d += fabs(beta) * fabs(c0);
                }
                R[t * ncols + c] = r;
                D[t * ncols + c] = d;
            }
        }
        free(s);
        free(mag);
    }
    free(Bw);
    return status;
}

int oracle_gemm_f32(int64_t M, int64_t N, int64_t K, double alpha,
                    const float* A, int64_t lda, const float* B, int64_t ldb,
                    double beta, const float* C0, int64_t ldc,
                    const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                    double* R, double* D, int nthreads) {
    return oracle_gemm(from_f32, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, NULL, NULL,
                       NULL, ACT_NONE,
                       rows, nrows, cols, ncols, R, D, nthreads);
}

int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K, double alpha,
                     const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                     double beta, const uint16_t* C0, int64_t ldc,
                     const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                     double* R, double* D, int nthreads) {
    return oracle_gemm(from_bf16, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, NULL, NULL,
                       NULL, ACT_NONE,
                       rows, nrows, cols, ncols, R, D, nthreads);
}

/* The epilogue variants: bias (length N, same element type, or NULL) and act. */
int oracle_gemm_f32_epi(int64_t M, int64_t N, int64_t K, double alpha,
                        const float* A, int64_t lda, const float* B, int64_t ldb,
                        double beta, const float* C0, int64_t ldc, const float* bias, int act,
                        const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                        double* R, double* D, int nthreads) {
    return oracle_gemm(from_f32, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, NULL, NULL,
                       bias, act,
                       rows, nrows, cols, ncols, R, D, nthreads);
}

int oracle_gemm_bf16_epi(int64_t M, int64_t N, int64_t K, double alpha,
                         const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                         double beta, const uint16_t* C0, int64_t ldc, const uint16_t* bias,
                         int act, const int64_t* rows, int64_t nrows, const int64_t* cols,
                         int64_t ncols, double* R, double* D, int nthreads) {
    return oracle_gemm(from_bf16, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, NULL, NULL,
                       bias, act,
                       rows, nrows, cols, ncols, R, D, nthreads);
}

/* The scaled variants: row_scale (length M) and col_scale (length N), fp32,
 * each NULL for none, then the bias and activation as above. */
int oracle_gemm_f32_scaled(int64_t M, int64_t N, int64_t K, double alpha,
                           const float* A, int64_t lda, const float* B, int64_t ldb,
                           double beta, const float* C0, int64_t ldc, const float* row_scale,
                           const float* col_scale, const float* bias, int act,
                           const int64_t* rows, int64_t nrows, const int64_t* cols,
                           int64_t ncols, double* R, double* D, int nthreads) {
    return oracle_gemm(from_f32, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, row_scale,
                       col_scale, bias, act, rows, nrows, cols, ncols, R, D, nthreads);
}

int oracle_gemm_bf16_scaled(int64_t M, int64_t N, int64_t K, double alpha,
                            const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                            double beta, const uint16_t* C0, int64_t ldc, const float* row_scale,
                            const float* col_scale, const uint16_t* bias, int act,
                            const int64_t* rows, int64_t nrows, const int64_t* cols,
                            int64_t ncols, double* R, double* D, int nthreads) {
    return oracle_gemm(from_bf16, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, row_scale,
                       col_scale, bias, act, rows, nrows, cols, ncols, R, D, nthreads);
}

int oracle_max_threads(void) { return omp_get_max_threads(); }
