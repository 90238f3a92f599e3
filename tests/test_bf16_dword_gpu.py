"""bf16 operands whose rows are aligned to 4 bytes but not to 16 (even
leading dimensions that are not multiples of 8, or bases 4 bytes past a
16-byte boundary), through the C ABI: the 4-byte copies of the tiled and
few-tile kernels.

* Those copies fill the same LDS layouts as the 1 KB copies of 16-byte rows,
  and the arithmetic is the same, so a product stored with 4-byte rows must
  equal the same product stored with 16-byte rows bit for bit: every operand
  layout, every tile size, ragged M, N and K, beta = 0 and beta != 0.
* Against the oracle: ragged edges in every layout, bases offset by 2
  elements, the fused bias + GELU epilogue, quantisation scales, a split-K
  workspace, and a leading dimension just inside and just past the copies'
  31-bit offset range (16-byte and 4-byte rows). Products with at most 256
  tiles of 64 x 64 run on the few-tile kernel, the rest on the tiled one.
"""
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, padded, to_f64, tol
from test_transpose_gpu import oracle_op

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
OP_IDS = ["NN", "NT", "TN", "TT"]
ACTS = {"none": dg.ACT_NONE, "relu": dg.ACT_RELU, "gelu_tanh": dg.ACT_GELU_TANH}


def _ld(cols, four):
    """The smallest leading dimension >= cols that is even but not a multiple
    of 8 (four) or a multiple of 8 (not four)."""
    ld = max(cols, 1)
    while not ((ld % 2 == 0 and ld % 8 != 0) if four else ld % 8 == 0):
        ld += 1
    return ld


def _store(X, trans, four, offset):
    S = X.t().contiguous() if trans else X
    rows, cols = S.shape
    ld = _ld(cols, four)
    buf, view = padded(rows, cols, ld, "bf16", offset=offset, fill=float("nan"))
    view.copy_(S.cuda())
    return buf, view, ld


def run(ops, A, B, C0, alpha, beta, four=True, offset=0, bias=None, act="none", ws=False,
        scales=None):
    """One bf16 call with 4-byte (four) or 16-byte rows; bases `offset`
    elements into their buffers. Returns C on the host."""
    M, K = A.shape
    N = B.shape[1]
    _, a, lda = _store(A, ops[0], four, offset)
    _, b, ldb = _store(B, ops[1], four, offset)
    ldc = _ld(N, four)
    _, c = padded(M, N, ldc, "bf16", offset=offset, fill=float("nan"))
    if C0 is not None:
        c.copy_(C0.cuda())
    keep = []

    def dev(t):
        if t is None:
            return None
        keep.append(t.cuda())
        return keep[-1].data_ptr()
    nbytes = dg.gemm_bf16_workspace_size(M, N, K) if ws else 0
    wbuf = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    wsp = wbuf.data_ptr() if nbytes else None
    if scales is not None:
        st = dg.gemm_bf16_scaled(ops[0], ops[1], M, N, K, float(alpha), a.data_ptr(), lda,
                                 b.data_ptr(), ldb, float(beta), c.data_ptr(), ldc,
                                 dev(scales[0]), dev(scales[1]), dev(bias), ACTS[act], wsp,
                                 nbytes, 0)
    else:
        st = dg.gemm_bf16_op(ops[0], ops[1], M, N, K, float(alpha), a.data_ptr(), lda,
                             b.data_ptr(), ldb, float(beta), c.data_ptr(), ldc, dev(bias),
                             ACTS[act], wsp, nbytes, 0)
    torch.cuda.synchronize()
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    return c.cpu()


def inputs(M, N, K, seed, beta):
    A = gi.random_matrix(M, K, "bf16", seed, dist="n")
    B = gi.random_matrix(K, N, "bf16", seed + 1)
    C0 = gi.random_matrix(M, N, "bf16", seed + 2) if beta != 0 else None
    return A, B, C0


# 1500 x 1530: 144 tiles of 128 x 128, so 576 tiles of 64 x 64 (more than
# the few-tile kernel, which 16-byte rows would otherwise take, runs in two
# rounds); 2048 x 1500: 192 tiles of 128 x 128; 3000 x 2998: 144 tiles of
# 256 x 256 (576 small ones would cost more); ragged in M, N and K.
@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape", [(1500, 1530, 1001), (2048, 1500, 300), (3000, 2998, 200)],
                         ids=lambda s: "x".join(map(str, s)))
def test_same_bits_as_16_byte_rows(shape, ops):
    M, N, K = shape
    for rep, (alpha, beta) in enumerate(((1.0, 0.0), (0.75, -1.5))):
        A, B, C0 = inputs(M, N, K, 9900 + 7 * M + rep, beta)
        note(f"bf16 4-byte rows {ops} M={M} N={N} K={K} alpha={alpha} beta={beta}")
        four = run(ops, A, B, C0, alpha, beta, four=True)
        wide = run(ops, A, B, C0, alpha, beta, four=False)
        assert torch.equal(four.view(torch.int16), wide.view(torch.int16)), f"call {rep}"


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
def test_oracle_ragged(ops):
    M, N, K = 300, 522, 129
    A, B, C0 = inputs(M, N, K, 9950 + 3 * ops[0] + ops[1], 0.5)
    note(f"bf16 4-byte rows vs oracle {ops} M={M} N={N} K={K}")
    C = run(ops, A, B, C0, 0.75, 0.5)
    R, D = oracle_op("bf16", A, B, C0, 0.75, 0.5)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
def test_oracle_offset_bases(ops):
    # Leading dimensions that are multiples of 8, bases 4 bytes past a
    # 16-byte boundary.
    M, N, K = 257, 264, 100
    A, B, C0 = inputs(M, N, K, 9960 + 3 * ops[0] + ops[1], 2.0)
    note(f"bf16 bases offset by 2 elements {ops} M={M} N={N} K={K}")
    C = run(ops, A, B, C0, 1.0, 2.0, four=False, offset=2)
    R, D = oracle_op("bf16", A, B, C0, 1.0, 2.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


def test_oracle_large_tiles_bias_gelu():
    M, N, K = 3000, 2998, 136
    A, B, C0 = inputs(M, N, K, 9970, 1.0)
    bias = gi.random_matrix(1, N, "bf16", 9973)[0].contiguous()
    note(f"bf16 4-byte rows, bias + GELU, M={M} N={N} K={K}")
    C = run((0, 0), A, B, C0, 1.25, 1.0, bias=bias, act="gelu_tanh")
    R, D = oracle_op("bf16", A, B, C0, 1.25, 1.0, bias, "gelu_tanh")
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


def test_oracle_scaled():
    from test_scale_gpu import oracle_scaled, scales
    M, N, K = 300, 522, 130
    A, B, C0 = inputs(M, N, K, 9980, 1.0)
    u, v = scales(M, 9983), scales(N, 9984)
    bias = gi.random_matrix(1, N, "bf16", 9985)[0].contiguous()
    note(f"bf16 4-byte rows, scaled, M={M} N={N} K={K}")
    C = run((0, 1), A, B, C0, 0.5, 1.0, bias=bias, act="relu", scales=(u, v))
    R, D = oracle_scaled("bf16", A, B, C0, u, v, bias, "relu", 0.5, 1.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


@pytest.mark.parametrize("ops", [(0, 0), (1, 1)], ids=["NN", "TT"])
def test_oracle_split_k(ops):
    # 72 tiles of 128 x 128 split over K with a workspace.
    M, N, K = 1024, 1026, 4100
    assert dg.gemm_bf16_workspace_size(M, N, K) > 0
    A, B, C0 = inputs(M, N, K, 9990 + ops[0], 1.0)
    note(f"bf16 4-byte rows, split K {ops} M={M} N={N} K={K}")
    C = run(ops, A, B, C0, 1.0, 1.0, ws=True)
    R, D = oracle_op("bf16", A, B, C0, 1.0, 1.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")
    plain = run(ops, A, B, C0, 1.0, 1.0, ws=False)      # tiled kernel, 272 tiles of 64 x 64
    R2 = oracle.max_rel_err(to_f64(plain), R, D)
    assert R2 <= tol("bf16")


# B stored N x K is copied k-contiguous: 256 rows of its storage span
# (256 ldb + K) * 2 bytes, inside 2^31 at 4.0 M elements and past it at
# 4.2 M, where the call takes the element-wise kernel. 16-byte rows
# (multiples of 8) and 4-byte rows (even, not multiples of 8); the padding
# between rows holds NaN.
@pytest.mark.parametrize("ldb", [4_000_000, 4_200_000, 4_000_002, 4_200_002])
def test_leading_dimension_at_the_copy_offset_limit(ldb):
    M, N, K = 200, 40, 50
    A, B, C0 = inputs(M, N, K, 9995, 0.5)
    note(f"bf16 A B^T with ldb={ldb} M={M} N={N} K={K}")
    _, a = padded(M, K, 56, "bf16", fill=float("nan"))
    a.copy_(A.cuda())
    bbuf, b = padded(N, K, ldb, "bf16", fill=float("nan"))
    b.copy_(B.t().contiguous().cuda())
    _, c = padded(M, N, 48, "bf16", fill=float("nan"))
    c.copy_(C0.cuda())
    st = dg.gemm_bf16_op(0, 1, M, N, K, 0.75, a.data_ptr(), 56, b.data_ptr(), ldb, 0.5,
                         c.data_ptr(), 48, None, dg.ACT_NONE, None, 0, 0)
    torch.cuda.synchronize()
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    del bbuf, b
    R, D = oracle_op("bf16", A, B, C0, 0.75, 0.5)
    assert oracle.max_rel_err(to_f64(c.cpu()), R, D) <= tol("bf16")
