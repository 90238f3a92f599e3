"""CPU oracle for C = alpha*A*B + beta*C0 — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never imports it and it
never imports the HIP library.

The arithmetic lives in ``oracle_gemm.c`` (binary64, in-order k sums; see its
header for the definition and the passages it follows). This module only
marshals numpy arrays into it and holds the acceptance metric:

    err = max_ij |c_ij - r_ij| / D_ij,   0/0 := 0,  x/0 := +inf

with D_ij = |alpha| * sum_k |a_ik||b_kj| + |beta||c0_ij|. The bound is the
usual forward-error bound of a dot product, so it is independent of the
scale of the inputs.

``gemm(..., bias=, act=)`` runs the epilogue form of the same oracle:
r = act(alpha * s + bias_j) + beta * c0_ij, with act the identity, ReLU or
the tanh form of GELU, and D scaled by a bound on the activation's slope (see
``oracle_gemm.c``). ``row_scale=`` / ``col_scale=`` (fp32 vectors of length
M and N) add the quantisation scales: r = act(alpha * u_i * v_j * s + bias_j)
+ beta * c0_ij.

It also holds ``bf16_round``: round-to-nearest-even of a binary64 value to
the bf16 grid (1 sign, 8 exponent and 7 stored mantissa bits, as the
Blackwell BF16 GEMM notes describe in section 1.2), written from that
definition, for the pins whose exact result must be reproduced bit for bit.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    for name in ("oracle_gemm_f32", "oracle_gemm_bf16"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64,
                       vp, i64, vp, i64, vp, vp, ctypes.c_int]
    for name in ("oracle_gemm_f32_epi", "oracle_gemm_bf16_epi"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64, vp, ctypes.c_int,
                       vp, i64, vp, i64, vp, vp, ctypes.c_int]
    for name in ("oracle_gemm_f32_scaled", "oracle_gemm_bf16_scaled"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [i64, i64, i64, dbl, vp, i64, vp, i64, dbl, vp, i64, vp, vp, vp,
                       ctypes.c_int, vp, i64, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_activate.restype = dbl
    lib.oracle_activate.argtypes = [dbl, ctypes.c_int]
    lib.oracle_bf16_bits_to_double.restype = dbl
    lib.oracle_bf16_bits_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _rows_arg(x: Optional[Sequence[int]]):
    if x is None:
        return None, 0
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int64))
    return a, a.size


def _ld(x: np.ndarray, itemsize: int) -> int:
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    if x.size == 0:
        return max(x.shape[1], 1)
    if (x.shape[1] > 1 and x.strides[1] != itemsize) or x.strides[0] % itemsize:
        raise ValueError("expected a 2-D array with unit column stride")
    return max(x.strides[0] // itemsize, x.shape[1], 1)


# Activation codes of the epilogue form.
ACTS = {"none": 0, "relu": 1, "gelu_tanh": 2}


def activate(z, act: str) -> np.ndarray:
    """The oracle's activation (binary64), element by element."""
    lib = _load()
    code = ACTS[act]
    flat = np.asarray(z, dtype=np.float64).ravel()
    out = np.fromiter((lib.oracle_activate(float(v), code) for v in flat), dtype=np.float64,
                      count=flat.size)
    return out.reshape(np.shape(z))


def gemm(A: np.ndarray, B: np.ndarray, C0: Optional[np.ndarray] = None,
         alpha: float = 1.0, beta: float = 0.0, dtype: str = "f32",
         rows: Optional[Sequence[int]] = None, cols: Optional[Sequence[int]] = None,
         threads: int = 0, bias: Optional[np.ndarray] = None, act: Optional[str] = None,
         row_scale: Optional[np.ndarray] = None, col_scale: Optional[np.ndarray] = None):
    """Return (R, D) as float64 arrays of shape (len(rows), len(cols)).

    ``dtype`` "f32": A, B, C0 are float32 arrays. ``dtype`` "bf16": they are
    uint16 arrays holding bf16 bit patterns. ``rows``/``cols`` select a
    sub-grid of C (default: all). ``alpha``/``beta`` are taken as given
    (pass the fp32 value the GPU sees). ``beta == 0`` never reads C0.
    ``bias`` (length N, same element type) and ``act`` (a key of ``ACTS``)
    select the epilogue form. ``row_scale`` (length M) and ``col_scale``
    (length N), float32, select the scaled form.
    """
    lib = _load()
    scaled = row_scale is not None or col_scale is not None
    epi = bias is not None or act is not None
    if dtype == "f32":
        want, isz = np.float32, 4
        fn = (lib.oracle_gemm_f32_scaled if scaled else
              lib.oracle_gemm_f32_epi if epi else lib.oracle_gemm_f32)
    elif dtype == "bf16":
        want, isz = np.uint16, 2
        fn = (lib.oracle_gemm_bf16_scaled if scaled else
              lib.oracle_gemm_bf16_epi if epi else lib.oracle_gemm_bf16)
    else:
        raise ValueError(dtype)
    for name, x in (("A", A), ("B", B)):
        if x.dtype != want:
            raise TypeError(f"{name} must be {want.__name__}")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    lda, ldb = _ld(A, isz), _ld(B, isz)
    c0_ptr, ldc = None, max(N, 1)
    if beta != 0.0:
        if C0 is None or C0.dtype != want or C0.shape != (M, N):
            raise ValueError("beta != 0 needs C0 of shape (M, N) and the same dtype")
        c0_ptr, ldc = C0.ctypes.data, _ld(C0, isz)
    r_idx, nr = _rows_arg(rows)
    c_idx, nc = _rows_arg(cols)
    nr = M if r_idx is None else nr
    nc = N if c_idx is None else nc
    R = np.empty((nr, nc), dtype=np.float64)
    D = np.empty((nr, nc), dtype=np.float64)
    extra = ()
    scales = ()
    if scaled:
        # Contiguous copies held in local names, so they outlive the call.
        row_scale = None if row_scale is None else np.ascontiguousarray(row_scale)
        col_scale = None if col_scale is None else np.ascontiguousarray(col_scale)
        for name, v, n in (("row_scale", row_scale, M), ("col_scale", col_scale, N)):
            if v is not None and (v.dtype != np.float32 or v.shape != (n,)):
                raise ValueError(f"{name} must be float32 of shape ({n},)")
            scales += (None if v is None or v.size == 0 else v.ctypes.data,)
    if epi or scaled:
        if bias is not None:
            bias = np.ascontiguousarray(bias)
            if bias.dtype != want or bias.shape != (N,):
                raise ValueError("bias must have shape (N,) and the dtype of A and B")
        code = ACTS[act if act is not None else "none"]
        extra = (None if bias is None or bias.size == 0 else bias.ctypes.data, code)
    st = fn(M, N, K, float(alpha), A.ctypes.data if A.size else None, lda,
            B.ctypes.data if B.size else None, ldb, float(beta), c0_ptr, ldc, *scales, *extra,
            None if r_idx is None else r_idx.ctypes.data, nr,
            None if c_idx is None else c_idx.ctypes.data, nc,
            R.ctypes.data, D.ctypes.data, int(threads))
    if st != 0:
        raise RuntimeError(f"oracle rejected its arguments (status {st})")
    return R, D


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns, via the oracle's own widening."""
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.fromiter((lib.oracle_bf16_bits_to_double(int(b)) for b in flat),
                      dtype=np.float64, count=flat.size)
    return out.reshape(np.shape(bits))


def bf16_round(r: np.ndarray) -> np.ndarray:
    """Round binary64 values to the nearest bf16 value, ties to even.

    For a finite nonzero r with 2**e <= |r| < 2**(e+1), the bf16 grid near r
    has spacing 2**(e-7) (8 significant bits); below the smallest normal
    2**-126 the spacing stays 2**-133. ``np.round`` rounds halves to even,
    which is the tie rule. Values past the largest finite bf16 become inf.
    """
    r = np.asarray(r, dtype=np.float64)
    out = np.zeros_like(r)
    nz = (r != 0) & np.isfinite(r)
    _, ex = np.frexp(r[nz])              # |r| = m * 2**ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -126)
    ulp = np.ldexp(1.0, e - 7)
    q = np.round(r[nz] / ulp) * ulp
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    q = np.where(np.abs(q) > max_bf16, np.copysign(np.inf, q), q)
    out[nz] = q
    out[~np.isfinite(r)] = r[~np.isfinite(r)]
    return out


def err_ratio(C: np.ndarray, R: np.ndarray, D: np.ndarray) -> np.ndarray:
    """Per-entry |C - R| / D with 0/0 := 0 and x/0 := +inf."""
    C = np.asarray(C, dtype=np.float64)
    diff = np.abs(C - R)
    out = np.full(diff.shape, np.inf)
    pos = D > 0
    out[pos] = diff[pos] / D[pos]
    out[(~pos) & (diff == 0)] = 0.0
    out[np.isnan(diff)] = np.inf
    return out


def max_rel_err(C: np.ndarray, R: np.ndarray, D: np.ndarray) -> float:
    e = err_ratio(C, R, D)
    return float(e.max()) if e.size else 0.0


# Acceptance bounds for the GPU results (fp32 output; bf16 output compared
# against the oracle run on the same bf16 inputs).
TOL_F32 = 1e-5
TOL_BF16 = 8e-3


def gamma(n: int, u: float = 2.0 ** -53) -> float:
    """Higham's gamma_n = n u / (1 - n u): the classic bound on n rounded operations."""
    return n * u / (1.0 - n * u)
