"""Pins for the CPU oracle, independent of the oracle itself (CPU only).

The pages print no GEMM output values, so the oracle is pinned by what the
mathematics fixes:
  * exact rational brute force on tiny shapes (Python ``fractions``), with
    the rounding bound of an in-order binary64 dot product;
  * integer inputs, where the oracle must be exact;
  * identity, permutation and all-ones operands, whose results are closed forms;
  * numpy's float64 matmul on moderate shapes (a library special case);
  * bf16 widening against torch's own bf16 -> fp32 conversion, and the
    oracle's bf16 rounding against torch's fp32 -> bf16 conversion;
  * the acceptance metric's special cases.
A last test plants mistakes (in Python wrappers around the oracle, on the
CPU) and checks that each is caught by at least one pin.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle

SHAPES_TINY = [(1, 1, 1), (2, 3, 5), (3, 2, 1), (5, 8, 3), (8, 5, 17), (17, 3, 8), (1, 17, 2),
               (3, 5, 17)]
DYADIC = [(1.0, 0.0), (-1.5, 0.5), (0.5, 2.0), (2.25, -1.0), (0.0, 1.5)]


def _exact_values(x: torch.Tensor):
    """Exact rationals of a CPU fp32/bf16 tensor, via torch's conversion."""
    return [[Fraction(float(v)) for v in row] for row in x.to(torch.float32).tolist()]


def _exact_gemm(A, B, C0, alpha, beta):
    Af, Bf = _exact_values(A), _exact_values(B)
    Cf = _exact_values(C0) if C0 is not None else None
    M, K, N = len(Af), len(Bf), len(Bf[0]) if Bf else 0
    a, b = Fraction(alpha), Fraction(beta)
    R = [[None] * N for _ in range(M)]
    Dm = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
            m = sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0))
            r, d = a * s, abs(a) * m
            if beta != 0.0:
                r += b * Cf[i][j]
                d += abs(b) * abs(Cf[i][j])
            R[i][j], Dm[i][j] = r, d
    return R, Dm


def _run(A, B, C0, alpha, beta, dtype, **kw):
    return oracle.gemm(gi.as_numpy(A), gi.as_numpy(B),
                       None if C0 is None else gi.as_numpy(C0), alpha, beta, dtype, **kw)


def _pin_rational(f, dtype, integer=False):
    """Returns True when ``f`` (an oracle-like callable) meets the brute-force pins."""
    for si, (M, N, K) in enumerate(SHAPES_TINY):
        for ai, (alpha, beta) in enumerate(DYADIC):
            seed = 7000 + 31 * si + ai
            if integer:
                A = gi.small_int_matrix(M, K, dtype, seed)
                B = gi.small_int_matrix(K, N, dtype, seed + 1)
                C0 = gi.small_int_matrix(M, N, dtype, seed + 2)
            else:
                A = gi.random_matrix(M, K, dtype, seed)
                B = gi.random_matrix(K, N, dtype, seed + 1, dist="n")
                C0 = gi.random_matrix(M, N, dtype, seed + 2)
            R, D = f(A, B, C0 if beta != 0 else None, alpha, beta, dtype)
            Rx, Dx = _exact_gemm(A, B, C0 if beta != 0 else None, alpha, beta)
            bound = oracle.gamma(K + 2)
            for i in range(M):
                for j in range(N):
                    if integer:
                        if Fraction(R[i, j]) != Rx[i][j] or Fraction(D[i, j]) != Dx[i][j]:
                            return False
                    else:
                        tol = bound * float(Dx[i][j])
                        if abs(Fraction(R[i, j]) - Rx[i][j]) > Fraction(tol):
                            return False
                        if abs(Fraction(D[i, j]) - Dx[i][j]) > Fraction(tol):
                            return False
    return True


def _pin_identity(f, dtype):
    """A = I gives alpha*B + beta*C0 exactly; B = I gives alpha*A + beta*C0."""
    K, N = 13, 9
    B = gi.random_matrix(K, N, dtype, 8101)
    C0 = gi.random_matrix(K, N, dtype, 8102)
    I = torch.eye(K, dtype=torch.float32).to(B.dtype)
    for alpha, beta in [(1.0, 0.0), (-1.5, 0.5)]:
        R, _ = f(I, B, C0 if beta else None, alpha, beta, dtype)
        Bx, Cx = _exact_values(B), _exact_values(C0)
        for i in range(K):
            for j in range(N):
                want = Fraction(alpha) * Bx[i][j] + (Fraction(beta) * Cx[i][j] if beta else 0)
                if Fraction(R[i, j]) != want:
                    return False
    A = gi.random_matrix(7, N, dtype, 8103)
    I = torch.eye(N, dtype=torch.float32).to(A.dtype)
    R, _ = f(A, I, None, 1.0, 0.0, dtype)
    return np.array_equal(R, A.to(torch.float64).numpy())


def _pin_permutation(f, dtype):
    M, K, N = 6, 6, 11
    sigma = [3, 0, 5, 1, 4, 2]
    P = torch.zeros(M, K)
    for i, s in enumerate(sigma):
        P[i, s] = 1.0
    B = gi.random_matrix(K, N, dtype, 8201)
    R, _ = f(P.to(B.dtype), B, None, 1.0, 0.0, dtype)
    Bd = B.to(torch.float64).numpy()
    if not np.array_equal(R, Bd[sigma, :]):
        return False
    # Column permutation: B[k, j] = 1 iff k == tau[j]  =>  R[:, j] = A[:, tau[j]]
    tau = [4, 1, 0, 5, 2, 3]
    Q = torch.zeros(6, 6)
    for j, t in enumerate(tau):
        Q[t, j] = 1.0
    A = gi.random_matrix(5, 6, dtype, 8202)
    R, _ = f(A, Q.to(A.dtype), None, 1.0, 0.0, dtype)
    return np.array_equal(R, A.to(torch.float64).numpy()[:, tau])


def _pin_all_ones(f, dtype):
    M, N, K = 4, 7, 300
    A = torch.ones(M, K).to(torch.float32 if dtype == "f32" else torch.bfloat16)
    B = torch.ones(K, N).to(A.dtype)
    C0 = gi.random_matrix(M, N, dtype, 8301)
    alpha, beta = 0.75, -2.0
    R, D = f(A, B, C0, alpha, beta, dtype)
    c0 = C0.to(torch.float64).numpy()
    return (np.array_equal(R, K * alpha + beta * c0)
            and np.array_equal(D, abs(alpha) * K + abs(beta) * np.abs(c0)))


def _pin_numpy(f, dtype):
    M, N, K = 40, 33, 301
    A = gi.random_matrix(M, K, dtype, 8401, dist="n")
    B = gi.random_matrix(K, N, dtype, 8402)
    C0 = gi.random_matrix(M, N, dtype, 8403)
    alpha, beta = 1.25, -0.5
    R, D = f(A, B, C0, alpha, beta, dtype)
    a64, b64 = A.to(torch.float64).numpy(), B.to(torch.float64).numpy()
    c64 = C0.to(torch.float64).numpy()
    ref = alpha * (a64 @ b64) + beta * c64
    dref = abs(alpha) * (np.abs(a64) @ np.abs(b64)) + abs(beta) * np.abs(c64)
    tol = 2 * oracle.gamma(K + 2) * dref
    return bool(np.all(np.abs(R - ref) <= tol) and np.all(np.abs(D - dref) <= tol))


PINS = [_pin_rational, _pin_identity, _pin_permutation, _pin_all_ones, _pin_numpy]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin, dtype):
    assert pin(_run, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_integers_exact(dtype):
    assert _pin_rational(_run, dtype, integer=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sampled_entries_equal_full(dtype):
    M, N, K = 37, 29, 64
    A = gi.random_matrix(M, K, dtype, 8501)
    B = gi.random_matrix(K, N, dtype, 8502)
    C0 = gi.random_matrix(M, N, dtype, 8503)
    R, D = _run(A, B, C0, 0.5, 2.0, dtype)
    rows, cols = [36, 0, 5, 5, 17], [28, 3, 0]
    Rs, Ds = _run(A, B, C0, 0.5, 2.0, dtype, rows=rows, cols=cols)
    assert np.array_equal(Rs, R[np.ix_(rows, cols)])
    assert np.array_equal(Ds, D[np.ix_(rows, cols)])


def test_thread_count_does_not_change_bits():
    A = gi.random_matrix(50, 200, "f32", 8601)
    B = gi.random_matrix(200, 45, "f32", 8602)
    R1, D1 = _run(A, B, None, 1.0, 0.0, "f32", threads=1)
    R8, D8 = _run(A, B, None, 1.0, 0.0, "f32", threads=8)
    assert np.array_equal(R1, R8) and np.array_equal(D1, D8)


def test_beta_zero_never_reads_c0():
    """BLAS convention taken for beta == 0: C0 is not read, so NaN cannot leak."""
    import ctypes
    A = gi.as_numpy(gi.random_matrix(4, 5, "f32", 8701))
    B = gi.as_numpy(gi.random_matrix(5, 3, "f32", 8702))
    C0 = np.full((4, 3), np.nan, dtype=np.float32)
    R = np.empty((4, 3)); D = np.empty((4, 3))
    lib = oracle._load()
    st = lib.oracle_gemm_f32(4, 3, 5, 1.0, A.ctypes.data, 5, B.ctypes.data, 3, 0.0,
                             C0.ctypes.data, 3, None, 0, None, 0, R.ctypes.data,
                             D.ctypes.data, 0)
    assert st == 0 and np.isfinite(R).all() and np.isfinite(D).all()


def test_empty_shapes():
    A = np.zeros((3, 0), np.float32)
    B = np.zeros((0, 4), np.float32)
    C0 = np.ones((3, 4), np.float32)
    R, D = oracle.gemm(A, B, C0, 2.0, 3.0)
    assert np.array_equal(R, np.full((3, 4), 3.0)) and np.array_equal(D, np.full((3, 4), 3.0))
    R, D = oracle.gemm(np.zeros((0, 5), np.float32), np.zeros((5, 4), np.float32))
    assert R.shape == (0, 4)


def test_bf16_widening_matches_torch_on_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    mine = oracle.bf16_bits_to_f64(bits)
    finite = np.isfinite(t)
    assert np.array_equal(mine[finite], t[finite])
    assert np.array_equal(np.isnan(mine), np.isnan(t))
    assert np.array_equal(np.isinf(mine), np.isinf(t))
    # A few hand-checked patterns: 1.0, -2.0, pi rounded to 8 bits, smallest subnormal.
    assert list(oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x4049, 0x0001], np.uint16))) \
        == [1.0, -2.0, 3.140625, 2.0 ** -133]


def test_bf16_rounding_matches_torch():
    g = torch.Generator().manual_seed(8801)
    x = torch.randn(200000, generator=g) * torch.exp2(torch.randint(-140, 120, (200000,),
                                                                    generator=g).float())
    # Exact ties: low 16 bits == 0x8000 must round to even.
    ties = torch.from_numpy((np.arange(1, 5001, dtype=np.uint32) << 16 | 0x8000)
                            .view(np.int32).copy()).view(torch.float32)
    x = torch.cat([x, ties, -ties]).to(torch.float32)
    want = x.to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(x.to(torch.float64).numpy())
    assert np.array_equal(got, want)


def test_error_metric_special_cases():
    R = np.array([[1.0, 0.0, 0.0]]); D = np.array([[2.0, 0.0, 0.0]])
    C = np.array([[1.5, 0.0, 1e-30]])
    e = oracle.err_ratio(C, R, D)
    assert e[0, 0] == 0.25 and e[0, 1] == 0.0 and e[0, 2] == np.inf
    assert oracle.max_rel_err(np.array([[np.nan]]), np.array([[1.0]]), np.array([[1.0]])) == np.inf
    # Scale invariance: scaling C, R and D together leaves the ratio unchanged.
    assert oracle.max_rel_err(C[:, :1] * 1024, R[:, :1] * 1024, D[:, :1] * 1024) == 0.25


def test_planted_mistakes_are_caught():
    """Each plausible oracle bug fails at least one pin (mutants wrap the real oracle)."""
    def transposed_b(A, B, C0, alpha, beta, dtype):  # uses B^T where B is square
        if B.shape[0] == B.shape[1]:
            B = B.t().contiguous()
        return _run(A, B, C0, alpha, beta, dtype)

    def dropped_beta(A, B, C0, alpha, beta, dtype):
        R, D = _run(A, B, None, alpha, 0.0, dtype)
        return R, D

    def sign_flip(A, B, C0, alpha, beta, dtype):
        return _run(A, B, C0, -alpha, beta, dtype)

    def dropped_last_k(A, B, C0, alpha, beta, dtype):
        if A.shape[1] > 1:
            A, B = A[:, :-1].contiguous(), B[:-1].contiguous()
        return _run(A, B, C0, alpha, beta, dtype)

    def signed_denominator(A, B, C0, alpha, beta, dtype):
        R, D = _run(A, B, C0, alpha, beta, dtype)
        return R, np.abs(R)

    def swapped_index(A, B, C0, alpha, beta, dtype):
        R, D = _run(A, B, C0, alpha, beta, dtype)
        return (R.T.copy(), D.T.copy()) if R.shape[0] == R.shape[1] else (R[::-1].copy(), D)

    for mutant in [transposed_b, dropped_beta, sign_flip, dropped_last_k,
                   signed_denominator, swapped_index]:
        caught = any(not pin(mutant, "f32") for pin in PINS)
        assert caught, mutant.__name__
