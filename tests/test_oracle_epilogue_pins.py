"""Pins for the oracle's epilogue form (CPU only).

The epilogue form computes r = act(alpha * s + bias_j) + beta * c0_ij (bias,
then activation, then the residual, the order of the Z-Turbo tuning page's
fused GELU + residual kernel, section 2.1) with act the identity, ReLU or the
tanh form of GELU, and D = L * (|alpha| sum_k |a_ik b_kj| + |bias_j|) +
|beta| |c0_ij| with L a bound on the activation's slope.

What pins it, without re-evaluating the oracle's own formula:
  * the tanh-form GELU stays within 5e-4 of the exact GELU z * Phi(z) (written
    here with ``math.erf``) over [-10, 10]; the tanh form is an approximation
    of that function, with a maximum deviation of about 4.7e-4, and a wrong
    constant or a dropped cubic term moves it by far more;
  * GELU(z) - GELU(-z) = z (tanh is odd), GELU(0) = 0, GELU(z) -> z for large z
    and -> 0 for very negative z;
  * the slope bound L holds (finite differences over a dense grid) and is tight;
  * ReLU and the identity, with integer or dyadic inputs, against exact
    rational brute force (bias and residual placement, signs, indices);
  * with GELU, the epilogue equals the pinned activation applied to the
    exactly computed pre-activation, plus the residual.
A last test plants mistakes (wrappers around the oracle) and checks that each
is caught.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle

SHAPES = [(1, 1, 1), (2, 3, 5), (5, 8, 3), (3, 7, 17), (4, 1, 2)]
SCALARS = [(1.0, 0.0), (-1.5, 0.5), (0.5, 2.0)]


def _erf_gelu(z: float) -> float:
    return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))


def _act_ok(act_fn) -> bool:
    """The activation pins, for any callable z-array -> GELU(z)-array."""
    z = np.linspace(-10.0, 10.0, 4001)
    g = act_fn(z)
    ref = np.array([_erf_gelu(v) for v in z])
    if np.abs(g - ref).max() > 5e-4:
        return False
    if np.abs((g - act_fn(-z)) - z).max() > 1e-12 * (1 + np.abs(z)).max():
        return False
    if act_fn(np.array([0.0]))[0] != 0.0:
        return False
    big = np.array([10.0, 20.0, 50.0])
    if np.abs(act_fn(big) - big).max() > 1e-12 or np.abs(act_fn(-big)).max() > 1e-12:
        return False
    return True


def test_gelu_tanh_pins():
    assert _act_ok(lambda z: oracle.activate(z, "gelu_tanh"))


def test_gelu_slope_bound_holds_and_is_tight():
    z = np.linspace(-8.0, 8.0, 32001)
    h = 1e-6
    d = (oracle.activate(z + h, "gelu_tanh") - oracle.activate(z - h, "gelu_tanh")) / (2 * h)
    _, D = oracle.gemm(np.ones((1, 1), np.float32), np.ones((1, 1), np.float32), act="gelu_tanh")
    slope = D[0, 0]       # |alpha| * 1 * 1 scaled by the slope bound
    assert np.abs(d).max() <= slope < np.abs(d).max() + 0.005


def test_relu_and_identity_pointwise():
    z = np.array([-3.5, -1e-30, -0.0, 0.0, 1e-30, 2.25, 7.0])
    assert np.array_equal(oracle.activate(z, "relu"), np.where(z > 0, z, 0.0))
    assert np.array_equal(oracle.activate(z, "none"), z)


def _exact(x: torch.Tensor):
    return [[Fraction(float(v)) for v in row] for row in x.to(torch.float32).tolist()]


def _exact_epi(A, B, C0, bias, alpha, beta, act):
    """Exact rationals of the epilogue for act in {none, relu}; also the exact z."""
    Af, Bf = _exact(A), _exact(B)
    Cf = _exact(C0) if C0 is not None else None
    bf = _exact(bias.reshape(1, -1))[0] if bias is not None else None
    M, K, N = len(Af), len(Bf), len(Bf[0])
    R, Dm, Z = [], [], []
    for i in range(M):
        rr, dd, zz = [], [], []
        for j in range(N):
            s = sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
            m = sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0))
            z = Fraction(alpha) * s + (bf[j] if bf is not None else 0)
            d = abs(Fraction(alpha)) * m + (abs(bf[j]) if bf is not None else 0)
            y = z if act == "none" else (z if z > 0 else Fraction(0))
            if beta != 0.0:
                y += Fraction(beta) * Cf[i][j]
            rr.append(y)
            dd.append(d)
            zz.append(z)
        R.append(rr); Dm.append(dd); Z.append(zz)
    return R, Dm, Z


def _inputs(M, N, K, dtype, seed, integer):
    if integer:
        mk = lambda r, c, s: gi.small_int_matrix(r, c, dtype, s)
    else:
        mk = lambda r, c, s: gi.random_matrix(r, c, dtype, s)
    return mk(M, K, seed), mk(K, N, seed + 1), mk(M, N, seed + 2), mk(1, N, seed + 3)[0]


def _call(f, A, B, C0, bias, alpha, beta, dtype, act):
    return f(gi.as_numpy(A), gi.as_numpy(B), None if C0 is None else gi.as_numpy(C0),
             None if bias is None else gi.as_numpy(bias), alpha, beta, dtype, act)


def _real(A, B, C0, bias, alpha, beta, dtype, act):
    return oracle.gemm(A, B, C0, alpha, beta, dtype, bias=bias, act=act)


def _pin_exact(f, dtype, integer=False):
    for si, (M, N, K) in enumerate(SHAPES):
        for ai, (alpha, beta) in enumerate(SCALARS):
            for act in ("none", "relu"):
                for with_bias in (True, False):
                    A, B, C0, bias = _inputs(M, N, K, dtype, 9000 + 17 * si + 3 * ai, integer)
                    bias = bias if with_bias else None
                    c0 = C0 if beta != 0 else None
                    R, D = _call(f, A, B, c0, bias, alpha, beta, dtype, act)
                    Rx, Dx, _ = _exact_epi(A, B, c0, bias, alpha, beta, act)
                    Cf = _exact(C0)
                    for i in range(M):
                        for j in range(N):
                            dfull = Dx[i][j] + (abs(Fraction(beta)) * abs(Cf[i][j])
                                                if beta else 0)
                            tol = Fraction(oracle.gamma(K + 3)) * dfull
                            if integer and Fraction(R[i, j]) != Rx[i][j]:
                                return False
                            if abs(Fraction(R[i, j]) - Rx[i][j]) > tol:
                                return False
                            if abs(Fraction(D[i, j]) - dfull) > tol:
                                return False
    return True


def _pin_gelu_composition(f, dtype):
    """GELU epilogue == pinned activation of the exact pre-activation + residual."""
    slope = 1.13
    for si, (M, N, K) in enumerate(SHAPES):
        alpha, beta = -1.5, 0.5
        A, B, C0, bias = _inputs(M, N, K, dtype, 9500 + si, False)
        R, D = _call(f, A, B, C0, bias, alpha, beta, dtype, "gelu_tanh")
        _, Dx, Z = _exact_epi(A, B, None, bias, alpha, 0.0, "none")
        Cf = _exact(C0)
        for i in range(M):
            zs = np.array([float(z) for z in Z[i]])
            want = oracle.activate(zs, "gelu_tanh") + beta * np.array([float(c) for c in Cf[i]])
            dfull = np.array([slope * float(Dx[i][j]) + abs(beta) * abs(float(Cf[i][j]))
                              for j in range(N)])
            tol = 4 * oracle.gamma(K + 8) * dfull + 1e-300
            if np.any(np.abs(R[i] - want) > tol) or np.any(np.abs(D[i] - dfull) > tol):
                return False
    return True


PINS = [_pin_exact, _pin_gelu_composition]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_epilogue_meets_pin(pin, dtype):
    assert pin(_real, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_epilogue_integers_exact(dtype):
    assert _pin_exact(_real, dtype, integer=True)


def test_plain_form_unchanged_by_identity_epilogue():
    A = gi.as_numpy(gi.random_matrix(9, 21, "f32", 9601))
    B = gi.as_numpy(gi.random_matrix(21, 13, "f32", 9602))
    C0 = gi.as_numpy(gi.random_matrix(9, 13, "f32", 9603))
    R0, D0 = oracle.gemm(A, B, C0, 0.5, 2.0)
    R1, D1 = oracle.gemm(A, B, C0, 0.5, 2.0, act="none")
    assert np.array_equal(R0, R1) and np.array_equal(D0, D1)


def test_epilogue_k_zero_and_alpha_zero():
    """With no product term the epilogue still applies: r = act(bias_j) + beta c0."""
    bias = np.array([-2.0, -0.5, 0.0, 1.5], np.float32)
    C0 = np.full((3, 4), 1.0, np.float32)
    for A, B, alpha in [(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32), 1.0),
                        (np.ones((3, 5), np.float32), np.ones((5, 4), np.float32), 0.0)]:
        R, _ = oracle.gemm(A, B, C0, alpha, 2.0, bias=bias, act="relu")
        assert np.array_equal(R, np.tile([2.0, 2.0, 2.0, 3.5], (3, 1)))


def test_planted_epilogue_mistakes_are_caught():
    def bias_after_act(A, B, C0, bias, alpha, beta, dtype, act):
        R, D = oracle.gemm(A, B, None, alpha, 0.0, dtype, act=act)
        if bias is not None:
            R = R + (oracle.bf16_bits_to_f64(bias) if dtype == "bf16" else bias.astype(np.float64))
        if beta:
            c0 = oracle.bf16_bits_to_f64(C0) if dtype == "bf16" else C0.astype(np.float64)
            R = R + beta * c0
        return R, _real(A, B, C0, bias, alpha, beta, dtype, act)[1]

    def residual_inside_act(A, B, C0, bias, alpha, beta, dtype, act):
        Rz, D = oracle.gemm(A, B, C0, alpha, beta, dtype, bias=bias, act="none")
        return oracle.activate(Rz, act), _real(A, B, C0, bias, alpha, beta, dtype, act)[1]

    def bias_dropped(A, B, C0, bias, alpha, beta, dtype, act):
        return _real(A, B, C0, None, alpha, beta, dtype, act)

    def bias_by_row(A, B, C0, bias, alpha, beta, dtype, act):
        if bias is not None and A.shape[0] <= bias.shape[0]:
            bias = np.concatenate([bias[:A.shape[0]][::-1], bias[A.shape[0]:]]).astype(bias.dtype)
        return _real(A, B, C0, bias, alpha, beta, dtype, act)

    def no_slope_in_d(A, B, C0, bias, alpha, beta, dtype, act):
        R, _ = _real(A, B, C0, bias, alpha, beta, dtype, act)
        _, D = _real(A, B, C0, bias, alpha, beta, dtype, "none")
        return R, D

    for mutant in [bias_after_act, residual_inside_act, bias_dropped, bias_by_row,
                   no_slope_in_d]:
        caught = any(not pin(mutant, "f32") for pin in PINS)
        assert caught, mutant.__name__

    def gelu_no_cubic(z):
        z = np.asarray(z, np.float64)
        return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * z))

    def gelu_wrong_scale(z):
        z = np.asarray(z, np.float64)
        return 0.5 * z * (1 + np.tanh(math.sqrt(math.pi / 2) * (z + 0.044715 * z ** 3)))

    def gelu_sign(z):
        z = np.asarray(z, np.float64)
        return 0.5 * z * (1 - np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))

    for mutant in [gelu_no_cubic, gelu_wrong_scale, gelu_sign]:
        assert not _act_ok(mutant), mutant.__name__
