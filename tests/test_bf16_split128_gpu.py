"""bf16 products with a single, partly full round of 256 x 256 tiles (129 ..
256 of them) that a workspace lets run on 128 x 128 tiles instead: one full
round of those, two per CU, and the tiles of the last round split over K,
their fp32 partial tiles added in range order by the last range to finish.
Through the C ABI with a workspace of gemm_bf16_workspace_size bytes.

* Against the oracle over every entry: row-major and transposed A (B stored
  N x K stays on 256 x 256 tiles and is checked too), 16-byte and 4-byte
  rows, ragged M, N and K (the K tail in the last range), alpha / beta, bias
  + GELU and quantisation scales.
* Exact small-integer products equal the exact result bit for bit (every
  range's partial sum and their total are exact: a lost or doubled range
  would show); repeated calls give the same bits and leave the workspace's
  counters at zero for the next call.
"""
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, to_f64, tol
from test_bf16_dword_gpu import inputs, run
from test_transpose_gpu import oracle_op

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (1, 0), (0, 1)]
OP_IDS = ["NN", "TN", "NT"]

# (M, N, K): 144 tiles of 256 x 256, or 552 of 128 x 128 (40 past one round
# of two per CU, each cut into 2 K ranges: 33 slabs of 64, the last 52 deep);
# 2048 x 4608: 144 large tiles, 576 small ones (64 past the round, 2 ranges
# of 16 slabs).
SHAPES = [(2900, 3000, 2100), (2048, 4608, 2048)]


def test_workspace_is_asked_for():
    for M, N, K in SHAPES:
        assert dg.gemm_bf16_workspace_size(M, N, K) > 0


@pytest.mark.parametrize("four", [False, True], ids=["16-byte", "4-byte"])
@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_parity(shape, ops, four):
    M, N, K = shape
    A, B, C0 = inputs(M, N, K, 9600 + M + 3 * ops[0] + ops[1], 0.5)
    note(f"bf16 128 x 128 split for one round {ops} M={M} N={N} K={K} four={four}")
    C = run(ops, A, B, C0, 0.75, 0.5, four=four, ws=True)
    R, D = oracle_op("bf16", A, B, C0, 0.75, 0.5)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


def test_bias_gelu_and_scales():
    from test_scale_gpu import oracle_scaled, scales
    M, N, K = SHAPES[0]
    A, B, C0 = inputs(M, N, K, 9650, 1.0)
    bias = gi.random_matrix(1, N, "bf16", 9653)[0].contiguous()
    note(f"bf16 128 x 128 split, bias + GELU, M={M} N={N} K={K}")
    C = run((0, 0), A, B, C0, 1.25, 1.0, four=False, bias=bias, act="gelu_tanh", ws=True)
    R, D = oracle_op("bf16", A, B, C0, 1.25, 1.0, bias, "gelu_tanh")
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")
    u, v = scales(M, 9655), scales(N, 9656)
    note(f"bf16 128 x 128 split, scales + bias + ReLU, M={M} N={N} K={K}")
    C = run((1, 0), A, B, C0, 0.5, 1.0, four=True, bias=bias, act="relu", scales=(u, v), ws=True)
    R, D = oracle_scaled("bf16", A, B, C0, u, v, bias, "relu", 0.5, 1.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


def test_exact_integers_repeats_and_counters():
    # Entries in -2 .. 2: every partial sum is an integer of magnitude at most
    # 4 K, exact in fp32, and alpha = 1/64 keeps the product exact: the one
    # rounding to bf16 must equal round-to-nearest-even of the exact result.
    M, N, K = SHAPES[0]
    g = torch.Generator().manual_seed(9660)
    A = torch.randint(-2, 3, (M, K), generator=g).to(torch.bfloat16)
    B = torch.randint(-2, 3, (K, N), generator=g).to(torch.bfloat16)
    exact = ((A.double() @ B.double()) / 64).to(torch.bfloat16)
    nbytes = dg.gemm_bf16_workspace_size(M, N, K)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    a, b = A.cuda(), B.cuda()
    results = []
    for rep in range(3):
        c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        note(f"bf16 128 x 128 split, exact integers M={M} N={N} K={K}, call {rep}")
        st = dg.gemm_bf16_ws(M, N, K, 1.0 / 64, a.data_ptr(), K, b.data_ptr(), N, 0.0,
                             c.data_ptr(), N, ws.data_ptr(), nbytes, 0)
        torch.cuda.synchronize()
        assert st == dg.GEMM_OK, dg.gemm_status_string(st)
        # One counter per split tile (40), padded to 256 bytes: all back to 0.
        assert int(ws[:256].view(torch.int32).abs().sum()) == 0
        results.append(c.cpu())
    assert torch.equal(results[0], exact)
    for r in results[1:]:
        assert torch.equal(r.view(torch.int16), results[0].view(torch.int16))
