"""bf16 products with at least one whole round of 256 x 256 tiles and a partly
full last one, through the C ABI: the trailing tile columns (or rows) that
hold the last round's tiles run as a second product on the same stream (on
the few-tile kernel when the strip is thin), the tiled kernel whole rounds
of 256 x 256 tiles on the rest.

* Against the oracle over every entry, in all four operand layouts, with
  ragged M, N and K, 4-byte rows, alpha / beta, bias + GELU and quantisation
  scales (the strip's operand, bias and scale pointers are offset).
* The call equals, bit for bit, the two products it is made of, each called
  on its own: the head (whole rounds of 256 x 256 tiles) and the strip.
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

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
OP_IDS = ["NN", "NT", "TN", "TT"]

# (M, N, K), strip: 4300 x 4096 has 17 x 16 = 272 tiles of 256 x 256, so rows
# 4096 .. 4299 (204 rows, 256 tiles of 64 x 64) go to the few-tile kernel;
# 4096 x 4200 the same by columns (104 columns); 4608^2 has 324 tiles and its
# last 4 tile columns (4608 x 1024) run on the tiled kernel's 128 x 128 tiles.
SHAPES = [((4300, 4096, 136), ("rows", 4096)), ((4096, 4200, 129), ("cols", 4096)),
          ((4608, 4608, 100), ("cols", 3584))]


def _sid(c):
    return "x".join(map(str, c[0]))


@pytest.mark.parametrize("four", [False, True], ids=["16-byte", "4-byte"])
@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("case", SHAPES, ids=_sid)
def test_parity(case, ops, four):
    (M, N, K), _ = case
    A, B, C0 = inputs(M, N, K, 9600 + M + 3 * ops[0] + ops[1], 0.5)
    note(f"bf16 partition {ops} M={M} N={N} K={K} four={four}")
    C = run(ops, A, B, C0, 0.75, 0.5, four=four)
    R, D = oracle_op("bf16", A, B, C0, 0.75, 0.5)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


@pytest.mark.parametrize("case", SHAPES, ids=_sid)
def test_bias_gelu_and_scales(case):
    from test_scale_gpu import oracle_scaled, scales
    (M, N, K), _ = case
    A, B, C0 = inputs(M, N, K, 9650 + M, 1.0)
    bias = gi.random_matrix(1, N, "bf16", 9653)[0].contiguous()
    note(f"bf16 partition, bias + GELU, M={M} N={N} K={K}")
    C = run((0, 0), A, B, C0, 1.25, 1.0, four=False, bias=bias, act="gelu_tanh")
    R, D = oracle_op("bf16", A, B, C0, 1.25, 1.0, bias, "gelu_tanh")
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")
    u, v = scales(M, 9655), scales(N, 9656)
    note(f"bf16 partition, scales + bias + ReLU, M={M} N={N} K={K}")
    C = run((1, 1), A, B, C0, 0.5, 1.0, four=True, bias=bias, act="relu", scales=(u, v))
    R, D = oracle_scaled("bf16", A, B, C0, u, v, bias, "relu", 0.5, 1.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


@pytest.mark.parametrize("case", SHAPES, ids=_sid)
def test_same_bits_as_its_two_products(case):
    (M, N, K), (by, start) = case
    A, B, C0 = inputs(M, N, K, 9670 + M, 1.0)
    note(f"bf16 partition against head and strip called alone, M={M} N={N} K={K}")
    C = run((0, 0), A, B, C0, 1.0, 1.0, four=False)
    if by == "rows":
        head = run((0, 0), A[:start], B, C0[:start], 1.0, 1.0, four=False)
        strip = run((0, 0), A[start:], B, C0[start:], 1.0, 1.0, four=False)
        both = torch.cat([head, strip], 0)
    else:
        head = run((0, 0), A, B[:, :start].contiguous(), C0[:, :start].contiguous(), 1.0, 1.0,
                   four=False)
        strip = run((0, 0), A, B[:, start:].contiguous(), C0[:, start:].contiguous(), 1.0, 1.0,
                    four=False)
        both = torch.cat([head, strip], 1)
    assert torch.equal(C.view(torch.int16), both.view(torch.int16))
