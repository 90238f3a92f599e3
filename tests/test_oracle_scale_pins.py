"""Pins for the oracle's scaled form (CPU only).

The scaled form adds the quantisation scaling that the Blackwell BF16 GEMM
notes (section 3.3) list beside GELU and the residual as epilogue work: one
fp32 factor u_i per row of A and one v_j per column of B (the dequantisation
scales of a row-wise and a column-wise quantised operand), applied to the
product before the bias:

    r = act(alpha * u_i * v_j * sum_k a_ik b_kj + bias_j) + beta * c0_ij
    D = L * (|alpha u_i v_j| * sum_k |a_ik b_kj| + |bias_j|) + |beta| |c0_ij|

What pins it, without re-evaluating the oracle's own formula:
  * exact rational brute force (``fractions``) on tiny shapes, with dyadic
    scales and scalars: integer inputs must match bit for bit (every value is
    then exact in binary64), random fp32 / bf16 inputs within the in-order
    binary64 bound plus one rounding of the factor;
  * a matrix identity: diag(u) (A B) diag(v) = (diag(u) A)(B diag(v)). With
    power-of-two scales, scaling the operands is exact, so the scaled form
    must equal the plain oracle on pre-scaled operands bit for bit;
  * planted mistakes (wrappers around the oracle): scales dropped from D,
    scales applied after the bias, scales applied to the residual, the row
    and column vectors swapped, a scale's sign dropped. Each must be caught.
"""
from fractions import Fraction

import numpy as np
import pytest

import gemm_inputs as gi
import oracle

SHAPES = [(1, 1, 1), (2, 3, 5), (5, 8, 3), (3, 7, 17), (4, 1, 2), (6, 6, 4)]
SCALARS = [(1.0, 0.0), (-1.5, 0.5), (0.5, 2.0)]


def _dyadic(n: int, seed: int, pow2: bool = False) -> np.ndarray:
    """n seeded dyadic fp32 values: +-m * 2^e with m in {1, 3, 5, 7} (1 only
    when pow2) and e in -3 .. 3."""
    rng = np.random.default_rng(seed)
    m = np.ones(n) if pow2 else rng.choice([1.0, 3.0, 5.0, 7.0], n)
    e = rng.integers(-3, 4, n)
    s = rng.choice([-1.0, 1.0], n)
    return (s * m * np.exp2(e)).astype(np.float32)


def _inputs(M, N, K, dtype, seed, integer):
    if integer:
        mk = lambda r, c, s: gi.small_int_matrix(r, c, dtype, s)
    else:
        mk = lambda r, c, s: gi.random_matrix(r, c, dtype, s)
    A, B, C0, bias = mk(M, K, seed), mk(K, N, seed + 1), mk(M, N, seed + 2), mk(1, N, seed + 3)[0]
    return (gi.as_numpy(A), gi.as_numpy(B), gi.as_numpy(C0), gi.as_numpy(bias),
            _dyadic(M, seed + 4), _dyadic(N, seed + 5))


def _widen(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float64)
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _real(A, B, C0, bias, u, v, alpha, beta, dtype, act):
    return oracle.gemm(A, B, C0, alpha, beta, dtype, bias=bias, act=act,
                       row_scale=u, col_scale=v)


def _exact(A, B, C0, bias, u, v, alpha, beta, dtype, act):
    """Exact rationals of r and D for act in {none, relu}."""
    Af = [[Fraction(float(x)) for x in row] for row in _widen(A, dtype)]
    Bf = [[Fraction(float(x)) for x in row] for row in _widen(B, dtype)]
    Cf = [[Fraction(float(x)) for x in row] for row in _widen(C0, dtype)]
    bf = [Fraction(float(x)) for x in _widen(bias, dtype)] if bias is not None else None
    M, K, N = len(Af), len(Bf), len(Bf[0]) if Bf else 0
    R = np.empty((M, N), dtype=object)
    D = np.empty((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            s = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
            m = sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0))
            f = Fraction(alpha) * Fraction(float(u[i])) * Fraction(float(v[j]))
            z = f * s + (bf[j] if bf is not None else 0)
            d = abs(f) * m + (abs(bf[j]) if bf is not None else 0)
            y = z if act == "none" else max(z, Fraction(0))
            if beta != 0.0:
                y += Fraction(beta) * Cf[i][j]
                d += abs(Fraction(beta)) * abs(Cf[i][j])
            R[i, j], D[i, j] = y, d
    return R, D


def _brute_force_ok(f, integer: bool) -> bool:
    """The brute-force pin, for any oracle-like callable f."""
    for n, (M, N, K) in enumerate(SHAPES):
        for dtype in ("f32", "bf16"):
            for (alpha, beta) in SCALARS:
                for act in ("none", "relu"):
                    seed = 9100 + 17 * n + (0 if dtype == "f32" else 7)
                    A, B, C0, bias, u, v = _inputs(M, N, K, dtype, seed, integer)
                    for b in (None, bias):
                        R, D = f(A, B, C0 if beta != 0 else None, b, u, v, alpha, beta, dtype, act)
                        Rx, Dx = _exact(A, B, C0, b, u, v, alpha, beta, dtype, act)
                        if integer:
                            if not (np.array_equal(R, Rx.astype(np.float64)) and
                                    np.array_equal(D, Dx.astype(np.float64))):
                                return False
                        else:
                            bound = oracle.gamma(K + 2)
                            for i in range(M):
                                for j in range(N):
                                    d = float(Dx[i, j])
                                    if abs(Fraction(float(R[i, j])) - Rx[i, j]) > bound * d + 1e-300:
                                        return False
                                    if abs(float(D[i, j]) - d) > bound * d + 1e-300:
                                        return False
    return True


def _identity_ok(f) -> bool:
    """diag(u)(AB)diag(v) = (diag(u)A)(B diag(v)), exact for power-of-two
    scales: the scaled form against the plain form on pre-scaled operands."""
    for n, (M, N, K) in enumerate([(3, 5, 7), (8, 2, 33), (16, 24, 40)]):
        for (alpha, beta) in SCALARS:
            A = gi.as_numpy(gi.random_matrix(M, K, "f32", 9300 + n))
            B = gi.as_numpy(gi.random_matrix(K, N, "f32", 9310 + n))
            C0 = gi.as_numpy(gi.random_matrix(M, N, "f32", 9320 + n))
            u, v = _dyadic(M, 9330 + n, pow2=True), _dyadic(N, 9340 + n, pow2=True)
            c0 = C0 if beta != 0 else None
            R, D = f(A, B, c0, None, u, v, alpha, beta, "f32", "none")
            As = (A * u[:, None]).astype(np.float32)
            Bs = (B * v[None, :]).astype(np.float32)
            R2, D2 = oracle.gemm(As, Bs, c0, alpha, beta, "f32")
            if not (np.array_equal(R, R2) and np.array_equal(D, D2)):
                return False
    return True


@pytest.mark.parametrize("integer", [True, False], ids=["integer_exact", "random_bound"])
def test_scaled_brute_force(integer):
    assert _brute_force_ok(_real, integer)


def test_scaled_matches_prescaled_operands():
    assert _identity_ok(_real)


def test_missing_scale_is_one():
    A, B, C0, bias, u, v = _inputs(4, 5, 6, "bf16", 9400, False)
    ones_m, ones_n = np.ones(4, np.float32), np.ones(5, np.float32)
    R1, D1 = oracle.gemm(A, B, C0, 0.5, 2.0, "bf16", bias=bias, act="relu", row_scale=u)
    R2, D2 = oracle.gemm(A, B, C0, 0.5, 2.0, "bf16", bias=bias, act="relu", row_scale=u,
                         col_scale=ones_n)
    assert np.array_equal(R1, R2) and np.array_equal(D1, D2)
    R3, D3 = oracle.gemm(A, B, C0, 0.5, 2.0, "bf16", bias=bias, act="relu", col_scale=v)
    R4, D4 = oracle.gemm(A, B, C0, 0.5, 2.0, "bf16", bias=bias, act="relu", row_scale=ones_m,
                         col_scale=v)
    assert np.array_equal(R3, R4) and np.array_equal(D3, D4)


def test_scaled_rejects_bad_vectors():
    A, B, C0, bias, u, v = _inputs(4, 5, 6, "f32", 9500, False)
    with pytest.raises(ValueError):
        oracle.gemm(A, B, row_scale=v, col_scale=v)
    with pytest.raises(ValueError):
        oracle.gemm(A, B, row_scale=u.astype(np.float64))


def _pieces(A, B, C0, bias, alpha, beta, dtype):
    """Plain sums S and magnitudes from the unscaled oracle (alpha 1, beta 0)."""
    S, Mag = oracle.gemm(A, B, None, 1.0, 0.0, dtype)
    bw = _widen(bias, dtype) if bias is not None else np.zeros(S.shape[1])
    cw = _widen(C0, dtype) if C0 is not None else np.zeros(S.shape)
    return S, Mag, bw, cw


def _act(z, act):
    return np.where(z > 0, z, 0.0) if act == "relu" else z


def _mut_d_unscaled(A, B, C0, bias, u, v, alpha, beta, dtype, act):
    R, _ = _real(A, B, C0, bias, u, v, alpha, beta, dtype, act)
    _, D = oracle.gemm(A, B, C0, alpha, beta, dtype, bias=bias, act=act)
    return R, D


def _mut_after_bias(A, B, C0, bias, u, v, alpha, beta, dtype, act):
    S, Mag, bw, cw = _pieces(A, B, C0, bias, alpha, beta, dtype)
    f = np.outer(u.astype(np.float64), v.astype(np.float64))
    R = _act(f * (alpha * S + bw), act) + beta * cw
    _, D = _real(A, B, C0, bias, u, v, alpha, beta, dtype, act)
    return R, D


def _mut_on_residual(A, B, C0, bias, u, v, alpha, beta, dtype, act):
    S, Mag, bw, cw = _pieces(A, B, C0, bias, alpha, beta, dtype)
    f = np.outer(u.astype(np.float64), v.astype(np.float64))
    R = f * (_act(alpha * S + bw, act) + beta * cw)
    _, D = _real(A, B, C0, bias, u, v, alpha, beta, dtype, act)
    return R, D


def _mut_swapped(A, B, C0, bias, u, v, alpha, beta, dtype, act):
    # The row vector indexed by column and vice versa (wrapped when lengths differ).
    M, N = A.shape[0], B.shape[1]
    uu = np.resize(v, M).astype(np.float32)
    vv = np.resize(u, N).astype(np.float32)
    return _real(A, B, C0, bias, uu, vv, alpha, beta, dtype, act)


def _mut_abs_scale(A, B, C0, bias, u, v, alpha, beta, dtype, act):
    return _real(A, B, C0, bias, np.abs(u), v, alpha, beta, dtype, act)


@pytest.mark.parametrize("mutant", [_mut_d_unscaled, _mut_after_bias, _mut_on_residual,
                                    _mut_swapped, _mut_abs_scale],
                         ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught(mutant):
    caught = (not _brute_force_ok(mutant, True)) or (not _brute_force_ok(mutant, False)) or \
             (not _identity_ok(mutant))
    assert caught, f"{mutant.__name__} passed every pin"
