"""GPU parity of the fp32 kernels at their edges, against the oracle: the
tiled kernel's global -> LDS copy path (row-major A and B with 16-byte rows)
and, at the shapes it takes, the few-tile kernel:

* ragged M, N and K, with every padding element of A and B set to NaN, so a
  copy that let a padding element into the product (a row past M, a column of
  A at k >= K, a row of B at k >= K) would show up as NaN in C;
* split K over a workspace, where only the range that ends at K holds the
  ragged tail;
* a leading dimension of A just inside and just past the copies' 31-bit
  offset range (past it the call takes the register-staged path);
* B stored N x K (A B^T), A stored K x M (A^T B) and both (A^T B^T), each
  operand staged in LDS the way it is stored, with the same NaN padding,
  ragged shapes and split K;
* more tiles than resident workgroups, so that each workgroup walks two or
  three tiles in every layout, with and without the bias/activation epilogue.
"""
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, padded, to_f64, tol
from test_transpose_gpu import check as check_op

pytestmark = pytest.mark.gpu


def run_nan_padded(A, B, lda, ldb, ldc, alpha=1.0, beta=0.0, C0=None, ws=False,
                   variant=dg.VARIANT_MFMA):
    """One call on NaN-padded operands: gemm_f32_ws with a workspace, else
    gemm_f32_ex with `variant` (the tiled kernel by default)."""
    M, K = A.shape
    N = B.shape[1]
    _, a = padded(M, K, lda, "f32", fill=float("nan"))
    _, b = padded(K, N, ldb, "f32", fill=float("nan"))
    _, c = padded(M, N, ldc, "f32", fill=float("nan"))
    a.copy_(A.cuda())
    b.copy_(B.cuda())
    if C0 is not None:
        c.copy_(C0.cuda())
    nbytes = dg.gemm_f32_workspace_size(M, N, K) if ws else 0
    wbuf = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    if ws:
        st = dg.gemm_f32_ws(M, N, K, alpha, a.data_ptr(), lda, b.data_ptr(), ldb, beta,
                            c.data_ptr(), ldc, wbuf.data_ptr() if nbytes else None, nbytes, 0)
    else:
        st = dg.gemm_f32_ex(M, N, K, alpha, a.data_ptr(), lda, b.data_ptr(), ldb, beta,
                            c.data_ptr(), ldc, 0, variant)
    torch.cuda.synchronize()
    return c.cpu(), st, nbytes


def check(A, B, C, alpha=1.0, beta=0.0, C0=None):
    R, D = oracle.gemm(gi.as_numpy(A), gi.as_numpy(B),
                       None if (C0 is None or beta == 0) else gi.as_numpy(C0),
                       float(alpha), float(beta), "f32")
    err = oracle.max_rel_err(to_f64(C), R, D)
    assert err <= tol("f32"), f"max error ratio {err:.3e}"


# (M, N, K): one and several tiles, K from a single partial slab to several
# slabs with a ragged tail, M and N ragged inside the last tile.
SHAPES = [(1, 4, 1), (5, 12, 31), (128, 128, 32), (129, 130, 33), (200, 260, 63),
          (300, 136, 100), (77, 300, 257), (256, 384, 1000)]


# The tiled kernel (forced: the copy path, and the register-staged path that
# element-aligned C rows take) and the few-tile kernel that gemm_f32 runs at
# these shapes.
KERNELS = [dg.VARIANT_MFMA, dg.VARIANT_GENERAL, dg.VARIANT_SMALL]


@pytest.mark.parametrize("variant", KERNELS, ids=lambda v: dg.VARIANT_NAMES[v])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_nan_padding_never_reaches_c(shape, variant):
    M, N, K = shape
    A = gi.random_matrix(M, K, "f32", 5100 + M)
    B = gi.random_matrix(K, N, "f32", 5200 + N)
    # 16-byte rows of A and B with at least one padding chunk after each row;
    # C rows 16-byte aligned for the copy path, 4-byte aligned otherwise.
    lda, ldb = (K + 3) // 4 * 4 + 4, (N + 3) // 4 * 4 + 8
    ldc = (N + 3) // 4 * 4 + 4 if variant == dg.VARIANT_MFMA else N + 3
    note(f"f32 NaN padding variant={variant} M={M} N={N} K={K} lda={lda} ldb={ldb}")
    C, st, _ = run_nan_padded(A, B, lda, ldb, ldc, variant=variant)
    assert st == dg.GEMM_OK
    assert torch.isfinite(C).all()
    check(A, B, C)


# Few tiles with enough tile-k that gemm_f32_ws splits them over workgroups:
# 81 tiles in 6 K ranges, 154 tiles in 3.
@pytest.mark.parametrize("shape", [(1100, 1030, 4100), (1700, 1300, 2100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_split_k_with_ragged_tail_and_nan_padding(shape):
    M, N, K = shape
    A = gi.random_matrix(M, K, "f32", 5300 + M)
    B = gi.random_matrix(K, N, "f32", 5400 + N)
    C0 = gi.random_matrix(M, N, "f32", 5500 + K)
    lda, ldb, ldc = (K + 3) // 4 * 4 + 4, (N + 3) // 4 * 4 + 4, N
    note(f"f32 copy path split K M={M} N={N} K={K}")
    C, st, nbytes = run_nan_padded(A, B, lda, ldb, ldc, alpha=0.5, beta=-1.5, C0=C0, ws=True)
    assert nbytes > 0
    assert st == dg.GEMM_OK
    check(A, B, C, 0.5, -1.5, C0)


@pytest.mark.parametrize("variant", [dg.VARIANT_MFMA, dg.VARIANT_SMALL],
                         ids=lambda v: dg.VARIANT_NAMES[v])
@pytest.mark.parametrize("lda", [4_000_000, 4_200_000])
def test_leading_dimension_at_the_copy_offset_limit(lda, variant):
    """128 rows of A span (128 * lda + 32) * 4 bytes: inside 2^31 at 4.0 M
    (copy path), past it at 4.2 M (register-staged path). Only 3 rows exist,
    so the copies of rows 8 .. 127 fall past the descriptor and read nothing."""
    M, N, K = 3, 40, 50
    A = gi.random_matrix(M, K, "f32", 5600)
    B = gi.random_matrix(K, N, "f32", 5601)
    note(f"f32 lda={lda} variant={variant}")
    C, st, _ = run_nan_padded(A, B, lda, N + 4, N, variant=variant)
    assert st == dg.GEMM_OK
    check(A, B, C)


def run_op_nan_padded(opa, opb, A, B, alpha, beta, C0, ws, pad):
    """C = alpha * op(A) op(B) + beta * C0 through gemm_f32_op, with A stored
    K x M when opa and B stored N x K when opb; every padding element NaN."""
    M, K = A.shape
    N = B.shape[1]
    As = A.t().contiguous() if opa else A
    Bs = B.t().contiguous() if opb else B
    lda = (As.shape[1] + 3) // 4 * 4 + pad
    ldb = (Bs.shape[1] + 3) // 4 * 4 + 2 * pad
    ldc = N + 1
    _, a = padded(As.shape[0], As.shape[1], lda, "f32", fill=float("nan"))
    _, b = padded(Bs.shape[0], Bs.shape[1], ldb, "f32", fill=float("nan"))
    _, c = padded(M, N, ldc, "f32", fill=float("nan"))
    a.copy_(As.cuda())
    b.copy_(Bs.cuda())
    if C0 is not None:
        c.copy_(C0.cuda())
    nbytes = dg.gemm_f32_workspace_size(M, N, K) if ws else 0
    wbuf = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    st = dg.gemm_f32_op(opa, opb, M, N, K, alpha, a.data_ptr(), lda, b.data_ptr(), ldb,
                        beta, c.data_ptr(), ldc, None, 0,
                        wbuf.data_ptr() if nbytes else None, nbytes, 0)
    torch.cuda.synchronize()
    return c.cpu(), st


@pytest.mark.parametrize("ops", [(0, 1), (1, 0), (1, 1)], ids=["ABt", "AtB", "AtBt"])
# SHAPES run on the few-tile kernel; 2100 x 2000 (272 tiles) on the tiled
# one, and 1100 x 1030 x 4100 on the tiled one split over a workspace.
@pytest.mark.parametrize("shape", SHAPES + [(1100, 1030, 2100), (2100, 2000, 100), (1100, 1030, 4100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_transposed_nan_padding_never_reaches_c(shape, ops):
    M, N, K = shape
    A = gi.random_matrix(M, K, "f32", 5700 + M)
    B = gi.random_matrix(K, N, "f32", 5800 + N)
    C0 = gi.random_matrix(M, N, "f32", 5900 + K)
    ws = M * N > 1_000_000
    note(f"f32 copy path ops={ops} NaN padding M={M} N={N} K={K} ws={ws}")
    C, st = run_op_nan_padded(ops[0], ops[1], A, B, 1.25, 0.5, C0, ws, pad=4)
    assert st == dg.GEMM_OK
    assert torch.isfinite(C).all()
    check(A, B, C, 1.25, 0.5, C0)


# More tiles than resident workgroups (two per CU, 512 on a full MI355X): 576,
# 1089 and 561 tiles of 128 x 128, so workgroups walk two or three tiles, and
# the ragged last row and column of tiles (and the ragged K tail) fall on
# workgroups that computed full tiles before them.
WALK_SHAPES = [(3000, 3000, 70), (4200, 4200, 40), (4100, 2100, 45)]


@pytest.mark.parametrize("ops", [(0, 0), (0, 1), (1, 0), (1, 1)], ids=["AB", "ABt", "AtB", "AtBt"])
@pytest.mark.parametrize("shape", WALK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_workgroups_walking_several_tiles(shape, ops):
    M, N, K = shape
    A = gi.random_matrix(M, K, "f32", 6000 + M)
    B = gi.random_matrix(K, N, "f32", 6100 + N)
    C0 = gi.random_matrix(M, N, "f32", 6200 + K)
    note(f"f32 copy path, tiles walked, ops={ops} M={M} N={N} K={K}")
    C, st = run_op_nan_padded(ops[0], ops[1], A, B, 0.75, -0.5, C0, False, pad=4)
    assert st == dg.GEMM_OK
    assert torch.isfinite(C).all()
    check(A, B, C, 0.75, -0.5, C0)


@pytest.mark.parametrize("act", ["relu", "gelu_tanh"])
def test_walking_tiles_with_bias_and_activation(act):
    check_op("f32", 0, 0, 3000, 3000, 72, 6300, alpha=1.25, beta=0.5, bias=True, act=act)
