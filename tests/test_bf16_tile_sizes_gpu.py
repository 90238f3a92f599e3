"""The bf16 tiled kernel's three tile sizes, 256 x 256 (products with many
tiles, 8 waves of 128 x 64), 128 x 128 (fewer, 8 waves of 64 x 32) and 64 x 64
(at most 160 tiles of 128 x 128 and no split, 4 waves of 32 x 32; products
with at most 512 of them and 16-byte rows go to the few-tile kernel instead),
through the C ABI.

* All accumulate each output over K in the same order, so the first 640 rows
  of a 4096-row product (256 x 256 tiles) and of a 2048-row one (128 x 128
  tiles) must equal a 640-row product of the same rows (64 x 64 tiles) bit
  for bit, in all four operand layouts, with ragged N and K.
* Ragged 256 x 256 tiles against the oracle in every layout, with the fused
  bias + GELU epilogue and with quantisation scales (the smaller test shapes
  elsewhere run on 128 x 128 tiles).
* 128 x 128 tiles split over a workspace against the oracle.
* Ragged 128 x 128 tiles alone on their CUs and 64 x 64 tiles in every layout,
  with 16-byte rows.
"""
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, padded, to_f64, tol
from test_transpose_gpu import check as check_op

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
OP_IDS = ["NN", "NT", "TN", "TT"]


def _store(X, trans):
    S = X.t().contiguous() if trans else X
    buf, view = padded(S.shape[0], S.shape[1], S.shape[1], "bf16", fill=float("nan"))
    view.copy_(S.cuda())
    return buf, view, S.shape[1]


def _op(opa, opb, A, B):
    M, K = A.shape
    N = B.shape[1]
    _, a, lda = _store(A, opa)
    _, b, ldb = _store(B, opb)
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = dg.gemm_bf16_op(opa, opb, M, N, K, 1.0, a.data_ptr(), lda, b.data_ptr(), ldb, 0.0,
                         c.data_ptr(), N, None, 0, None, 0, 0)
    torch.cuda.synchronize()
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    return c.cpu()


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
def test_tile_sizes_give_the_same_bits(ops):
    # 640 x 4000: 5 x 32 = 160 tiles of 128 x 128 and 630 of 64 x 64 (more
    # than two rounds of the few-tile kernel), so 64 x 64 tiles; 2048 x 4000:
    # 512 tiles of 128 x 128 (cost 0.61 against a round of 128 large ones);
    # 4096 x 4000: 256 large tiles (cost 1 against 1.22 for 1024 small ones).
    # The sizes also run different wave shapes.
    M_small, N, K = 640, 4000, 1000
    A = gi.random_matrix(M_small, K, "bf16", 8300, dist="n")
    B = gi.random_matrix(K, N, "bf16", 8301)
    note(f"bf16 tile sizes {ops}: 640, 2048 and 4096 rows, N={N} K={K}")
    small = _op(ops[0], ops[1], A, B)
    for M_big in (2048, 4096):
        A_big = torch.zeros(M_big, K, dtype=A.dtype)
        A_big[:M_small] = A
        big = _op(ops[0], ops[1], A_big, B)
        assert torch.equal(small.view(torch.int16), big[:M_small].view(torch.int16)), M_big
        assert bool((big[M_small:].float() == 0).all())


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
def test_large_tiles_ragged(ops):
    # 4000 x 4000 x 136: 16 x 16 tiles of 256 x 256, the last row and column
    # of tiles ragged, K of two slabs plus a tail.
    check_op("bf16", ops[0], ops[1], 4000, 4000, 136, 8400 + 7 * ops[0] + ops[1], alpha=0.75,
             beta=0.5, pad=(8, 8, 8))


def test_large_tiles_ragged_bias_gelu():
    check_op("bf16", 0, 0, 4000, 4000, 136, 8500, alpha=1.25, beta=1.0, bias=True, act="gelu_tanh")


def test_large_tiles_ragged_scaled():
    from test_scale_gpu import oracle_scaled, run_scaled, scales
    M, N, K = 4000, 4000, 136
    A = gi.random_matrix(M, K, "bf16", 8600, dist="n")
    B = gi.random_matrix(K, N, "bf16", 8601)
    C0 = gi.random_matrix(M, N, "bf16", 8602)
    u, v = scales(M, 8603), scales(N, 8604)
    bias = gi.random_matrix(1, N, "bf16", 8605)[0].contiguous()
    note("bf16 large tiles, scaled with bias and ReLU")
    C, st = run_scaled("bf16", A, B, C0, u, v, bias, "relu", 0.5, 1.0)
    assert st == dg.GEMM_OK
    R, D = oracle_scaled("bf16", A, B, C0, u, v, bias, "relu", 0.5, 1.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


# Small tiles split over a workspace: 40 tiles in 6 K ranges, 16 tiles of a
# ragged product in 8 (more workgroups than the few-tile kernel would run).
@pytest.mark.parametrize("shape", [(640, 1000, 8192), (129, 1000, 8200)],
                         ids=lambda s: "x".join(map(str, s)))
def test_small_tiles_split(shape):
    M, N, K = shape
    assert dg.gemm_bf16_workspace_size(M, N, K) > 0
    check_op("bf16", 0, 0, M, N, K, 8700 + M, alpha=1.0, beta=1.0, ws=True)


# 2048 x 1500: 192 tiles of 128 x 128, each alone on its CU; 1500 x 1530:
# 144 of them and 576 of 64 x 64, so 64 x 64 tiles. Ragged M, N and K in
# every layout, 16-byte rows (leading dimensions rounded up to multiples of 8).
SMALL_TILE_SHAPES = [(2048, 1500, 300), (1500, 1530, 136)]


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape", SMALL_TILE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_tiles_ragged(shape, ops):
    from test_bf16_dword_gpu import inputs, run
    from test_transpose_gpu import oracle_op
    M, N, K = shape
    A, B, C0 = inputs(M, N, K, 8800 + 7 * ops[0] + ops[1] + M, 0.5)
    note(f"bf16 small tiles {ops} M={M} N={N} K={K}")
    C = run(ops, A, B, C0, 0.75, 0.5, four=False)
    R, D = oracle_op("bf16", A, B, C0, 0.75, 0.5)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


@pytest.mark.parametrize("shape", SMALL_TILE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_tiles_bias_gelu(shape):
    from test_bf16_dword_gpu import inputs, run
    from test_transpose_gpu import oracle_op
    M, N, K = shape
    A, B, C0 = inputs(M, N, K, 8900 + M, 1.0)
    bias = gi.random_matrix(1, N, "bf16", 8903)[0].contiguous()
    note(f"bf16 small tiles, bias + GELU, M={M} N={N} K={K}")
    C = run((1, 0), A, B, C0, 1.25, 1.0, four=False, bias=bias, act="gelu_tanh")
    R, D = oracle_op("bf16", A, B, C0, 1.25, 1.0, bias, "gelu_tanh")
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")
