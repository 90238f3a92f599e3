"""Python binding of libdense_gemm_04_amd.so (argument marshalling only).

The functions carry the C names and arguments of ``include/gemm.h``: raw
device pointers (ints), sizes, leading dimensions and a stream handle (int,
0 = null stream). All arithmetic runs in the HIP kernels of the library; if
the library is missing or cannot be loaded, every call raises.

``matmul_f32`` / ``matmul_bf16`` are conveniences that take torch CUDA
tensors (row-major, unit column stride), pass their pointers, strides and
torch's current stream, and raise ``GemmError`` on a non-zero status.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdense_gemm_04_amd.so")

GEMM_OK = 0
GEMM_ERR_INVALID_VALUE = 1
GEMM_ERR_UNSUPPORTED_DEVICE = 2
GEMM_ERR_LAUNCH = 3
GEMM_ERR_SCRATCH_LIMIT = 4
# Size of the static scratch behind gemm_bf16_ws_noalloc (per GPU).
NOALLOC_SCRATCH_BYTES = (32 << 20) + (64 << 10)

VARIANT_AUTO = 0
VARIANT_MFMA = 1
VARIANT_GENERAL = 2
VARIANT_VALU = 3
VARIANT_SKINNY = 4
VARIANT_SMALL = 5
VARIANT_NAMES = {0: "auto", 1: "mfma", 2: "general", 3: "valu", 4: "skinny", 5: "small"}

ACT_NONE = 0
ACT_RELU = 1
ACT_GELU_TANH = 2
ACT_NAMES = {0: "none", 1: "relu", 2: "gelu_tanh"}

OP_N = 0
OP_T = 1

EXPORTS = ("gemm_f32", "gemm_bf16", "gemm_f32_ex", "gemm_bf16_ex", "gemm_bf16_ws",
           "gemm_bf16_workspace_size", "gemm_bf16_ws_noalloc", "gemm_f32_ws", "gemm_f32_workspace_size",
           "gemm_f32_bias_act", "gemm_bf16_bias_act", "gemm_f32_op", "gemm_bf16_op",
           "gemm_f32_scaled", "gemm_bf16_scaled", "gemm_plan",
           "gemm_status_string")

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"GEMM failed with status {status}: {gemm_status_string(status)}")


def load() -> ctypes.CDLL:
    """Load the native library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _bind(LIB_PATH)
    return _lib


def load_check_build(check: str) -> ctypes.CDLL:
    """One of the LDS-checking builds ("poison" or "sync"; see build.py), as
    a separate library handle with the same C functions, for the tests that
    compare it with the normal build."""
    if check not in ("poison", "sync"):
        raise ValueError(check)
    return _bind(os.path.join(PKG, f"libdense_gemm_04_amd_{check}.so"))


def _bind(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    i64, f32, vp, ci = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
    base = [i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp]
    for name in ("gemm_f32", "gemm_bf16"):
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = ci, base
    lib.gemm_bf16_ws_noalloc.restype, lib.gemm_bf16_ws_noalloc.argtypes = ci, base
    for name in ("gemm_f32_ex", "gemm_bf16_ex"):
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = ci, base + [ci]
    for name in ("gemm_bf16_ws", "gemm_f32_ws"):
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = ci, base[:11] + [vp, ctypes.c_size_t, vp]
    for name in ("gemm_f32_bias_act", "gemm_bf16_bias_act"):
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = ci, base[:11] + [vp, ci, vp, ctypes.c_size_t, vp]
    for name in ("gemm_f32_op", "gemm_bf16_op"):
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = ci, [ci, ci] + base[:11] + [vp, ci, vp, ctypes.c_size_t, vp]
    for name in ("gemm_f32_scaled", "gemm_bf16_scaled"):
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = ci, [ci, ci] + base[:11] + [vp, vp, vp, ci, vp, ctypes.c_size_t,
                                                              vp]
    for name in ("gemm_bf16_workspace_size", "gemm_f32_workspace_size"):
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = ctypes.c_size_t, [i64, i64, i64]
    lib.gemm_plan.restype = ci
    lib.gemm_plan.argtypes = [ci, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, ci]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_status_string.argtypes = [ci]
    return lib


def gemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().gemm_f32(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_bf16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().gemm_bf16(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_f32_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0, variant=0) -> int:
    return load().gemm_f32_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant)


def gemm_bf16_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0, variant=0) -> int:
    return load().gemm_bf16_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant)


def gemm_bf16_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes,
                 stream=0) -> int:
    return load().gemm_bf16_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                               workspace_bytes, stream)


def gemm_bf16_ws_noalloc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    return load().gemm_bf16_ws_noalloc(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_bf16_workspace_size(M, N, K) -> int:
    return load().gemm_bf16_workspace_size(M, N, K)


def gemm_f32_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace, workspace_bytes,
                stream=0) -> int:
    return load().gemm_f32_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                              workspace_bytes, stream)


def gemm_f32_workspace_size(M, N, K) -> int:
    return load().gemm_f32_workspace_size(M, N, K)


def gemm_f32_bias_act(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, workspace=0,
                      workspace_bytes=0, stream=0) -> int:
    return load().gemm_f32_bias_act(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act,
                                    workspace, workspace_bytes, stream)


def gemm_bf16_bias_act(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act, workspace=0,
                       workspace_bytes=0, stream=0) -> int:
    return load().gemm_bf16_bias_act(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act,
                                     workspace, workspace_bytes, stream)


def gemm_f32_op(opa, opb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias=None, act=0,
                workspace=None, workspace_bytes=0, stream=0) -> int:
    return load().gemm_f32_op(opa, opb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act,
                              workspace, workspace_bytes, stream)


def gemm_bf16_op(opa, opb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias=None, act=0,
                 workspace=None, workspace_bytes=0, stream=0) -> int:
    return load().gemm_bf16_op(opa, opb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act,
                               workspace, workspace_bytes, stream)


def gemm_f32_scaled(opa, opb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, row_scale=None,
                    col_scale=None, bias=None, act=0, workspace=None, workspace_bytes=0,
                    stream=0) -> int:
    return load().gemm_f32_scaled(opa, opb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                  row_scale, col_scale, bias, act, workspace, workspace_bytes,
                                  stream)


def gemm_bf16_scaled(opa, opb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, row_scale=None,
                     col_scale=None, bias=None, act=0, workspace=None, workspace_bytes=0,
                     stream=0) -> int:
    return load().gemm_bf16_scaled(opa, opb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                   row_scale, col_scale, bias, act, workspace, workspace_bytes,
                                   stream)


def gemm_plan(elem_bytes, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant=0) -> int:
    return load().gemm_plan(elem_bytes, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant)


def gemm_status_string(status: int) -> str:
    return load().gemm_status_string(status).decode()


# ---- torch-tensor conveniences (pointers, strides and stream only) ----------

def _ld(t, rows_of: int, cols: int) -> int:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if cols > 1 and t.stride(1) != 1:
        raise ValueError("expected unit column stride (row-major)")
    return max(t.stride(0) if rows_of > 1 else cols, cols, 1)


def _stream_handle(stream) -> int:
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _matmul(kind: str, A, B, C, alpha: float, beta: float, variant: int, stream) -> None:
    import torch
    want = torch.float32 if kind == "f32" else torch.bfloat16
    for name, t in (("A", A), ("B", B), ("C", C)):
        if t.dtype != want or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA tensor of dtype {want}")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    lda, ldb, ldc = _ld(A, M, K), _ld(B, K, N), _ld(C, M, N)
    fn = gemm_f32_ex if kind == "f32" else gemm_bf16_ex
    st = fn(M, N, K, float(alpha), A.data_ptr(), lda, B.data_ptr(), ldb, float(beta),
            C.data_ptr(), ldc, _stream_handle(stream), int(variant))
    if st != GEMM_OK:
        raise GemmError(st)


def matmul_f32(A, B, C, alpha: float = 1.0, beta: float = 0.0, variant: int = VARIANT_AUTO,
               stream=None) -> None:
    """C <- alpha * A @ B + beta * C for fp32 CUDA tensors (in place on C)."""
    _matmul("f32", A, B, C, alpha, beta, variant, stream)


def matmul_bf16(A, B, C, alpha: float = 1.0, beta: float = 0.0, variant: int = VARIANT_AUTO,
                stream=None) -> None:
    """C <- alpha * A @ B + beta * C for bf16 CUDA tensors (fp32 accumulation)."""
    _matmul("bf16", A, B, C, alpha, beta, variant, stream)
