"""bf16 tiled kernel with 128 x 128 tiles whose K is split between two groups
of 8 waves in one workgroup (products with at most one such tile per CU and
an even number of at least 32 64-deep K slabs), through the C ABI.

* Against the oracle over every entry: all four operand layouts, 16-byte and
  4-byte rows, ragged M, N and K (the K tail in the second group's last
  slab), 129 .. 160 tiles (where the split replaces 64 x 64 tiles), alpha /
  beta, bias + GELU and quantisation scales.
* Exact small-integer products equal the exact result bit for bit (both
  groups' partial sums and their sum are exact: a lost or doubled half, or a
  slab taken twice, would show).
* Repeated calls give the same bits.
"""
import pytest
import torch

import gemm_inputs as gi
import oracle
from gpu_util import note, to_f64, tol
from test_bf16_dword_gpu import inputs, run
from test_transpose_gpu import oracle_op

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
OP_IDS = ["NN", "NT", "TN", "TT"]

# (M, N, K): 256 tiles of 128 x 128 and 32 slabs; 2000^2 (256 tiles, ragged
# edges) with K = 2150 (34 slabs, a 38-deep tail); 1536 x 1664 (156 tiles,
# 36 slabs).
SHAPES = [(2048, 2048, 2048), (2000, 2000, 2150), (1536, 1664, 2304)]


@pytest.mark.parametrize("four", [False, True], ids=["16-byte", "4-byte"])
@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_parity(shape, ops, four):
    M, N, K = shape
    A, B, C0 = inputs(M, N, K, 9500 + M + 3 * ops[0] + ops[1], 0.5)
    note(f"bf16 K split in the workgroup {ops} M={M} N={N} K={K} four={four}")
    C = run(ops, A, B, C0, 0.75, 0.5, four=four)
    R, D = oracle_op("bf16", A, B, C0, 0.75, 0.5)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


def test_bias_gelu_and_scales():
    from test_scale_gpu import oracle_scaled, scales
    M, N, K = 2000, 2000, 2150
    A, B, C0 = inputs(M, N, K, 9550, 1.0)
    bias = gi.random_matrix(1, N, "bf16", 9553)[0].contiguous()
    note(f"bf16 K split, bias + GELU, M={M} N={N} K={K}")
    C = run((0, 0), A, B, C0, 1.25, 1.0, four=False, bias=bias, act="gelu_tanh")
    R, D = oracle_op("bf16", A, B, C0, 1.25, 1.0, bias, "gelu_tanh")
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")
    u, v = scales(M, 9555), scales(N, 9556)
    note(f"bf16 K split, scales + bias + ReLU, M={M} N={N} K={K}")
    C = run((0, 1), A, B, C0, 0.5, 1.0, four=True, bias=bias, act="relu", scales=(u, v))
    R, D = oracle_scaled("bf16", A, B, C0, u, v, bias, "relu", 0.5, 1.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


def test_exact_integers_and_repeats():
    # Entries in -2 .. 2: every partial sum is an integer of magnitude at most
    # 4 K, exact in fp32, and alpha = 1/64 keeps the product exact: the one
    # rounding to bf16 must equal round-to-nearest-even of the exact result.
    M, N, K = 2000, 2048, 2150
    g = torch.Generator().manual_seed(9560)
    A = torch.randint(-2, 3, (M, K), generator=g).to(torch.bfloat16)
    B = torch.randint(-2, 3, (K, N), generator=g).to(torch.bfloat16)
    note(f"bf16 K split, exact integers M={M} N={N} K={K}")
    C = run((0, 0), A, B, None, 1.0 / 64, 0.0, four=False)
    exact = (A.double() @ B.double()) / 64
    assert torch.equal(C, exact.to(torch.bfloat16))
    A, B, C0 = inputs(M, N, K, 9562, 0.5)
    first = run((1, 0), A, B, C0, 1.0, 0.5, four=False)
    again = run((1, 0), A, B, C0, 1.0, 0.5, four=False)
    assert torch.equal(first.view(torch.int16), again.view(torch.int16))
