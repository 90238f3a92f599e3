"""The bf16 few-tile kernel (one 64 x 64 tile per workgroup, K split over its
4 waves, partials added in wave order), through the C ABI. It takes products
whose 64 x 64 tiles fit two rounds of workgroups (512 on a full MI355X), or
one round when a workspace split would run fewer workgroups.

* Against the oracle in every operand layout: ragged M, N and K, the ragged K
  tail in the last wave's last slab, K shorter than four slabs (idle waves),
  a single tile, two rounds of tiles, alpha / beta, bias + GELU, quantisation
  scales.
* Exact small-integer products equal the exact result bit for bit (every
  partial sum is exact, so a lost or doubled partial would show), with 16-byte
  and with 4-byte rows.
* Rows aligned to 4 bytes only (4-byte copies into the same LDS layouts) give
  the bits of 16-byte rows in every layout, on the shapes above whose tiles
  fit one round (the kernel takes no more with 4-byte rows).
* Repeated calls give the same bits; a call with a workspace on a shape the
  kernel takes gives the plain call's bits (the workspace is not used).
"""
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, padded, to_f64, tol
from test_bf16_dword_gpu import inputs, run
from test_transpose_gpu import oracle_op

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
OP_IDS = ["NN", "NT", "TN", "TT"]

# (M, N, K): 45 tiles, K of 3 slabs (the fourth wave idle, a 1-element K
# tail); a full round (256 tiles); 9 tiles and a single slab (three waves
# idle); 441 tiles (two rounds), K of 9 slabs (ranges of 3, 3, 3 and 0);
# 24 tiles, K of 16 slabs with a 40-element tail in the last wave's last slab.
SHAPES = [(300, 520, 129), (1024, 1024, 4096), (129, 136, 64), (1300, 1300, 520), (500, 150, 1000)]


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_parity(shape, ops):
    M, N, K = shape
    assert ((M + 63) // 64) * ((N + 63) // 64) <= 512
    for rep, (alpha, beta) in enumerate(((1.0, 0.0), (0.75, -1.5))):
        A, B, C0 = inputs(M, N, K, 9700 + 3 * M + rep, beta)
        note(f"bf16 few-tile {ops} M={M} N={N} K={K} alpha={alpha} beta={beta}")
        C = run(ops, A, B, C0, alpha, beta, four=False)
        R, D = oracle_op("bf16", A, B, C0, alpha, beta)
        assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16"), f"call {rep}"


# With 4-byte rows the kernel takes one round of tiles (256), not two.
ONE_ROUND = [s for s in SHAPES if ((s[0] + 63) // 64) * ((s[1] + 63) // 64) <= 256]


@pytest.mark.parametrize("ops", OPS, ids=OP_IDS)
@pytest.mark.parametrize("shape", ONE_ROUND, ids=lambda s: "x".join(map(str, s)))
def test_four_byte_rows_same_bits(shape, ops):
    M, N, K = shape
    for rep, (alpha, beta) in enumerate(((1.0, 0.0), (0.75, -1.5))):
        A, B, C0 = inputs(M, N, K, 9720 + 3 * M + rep, beta)
        note(f"bf16 few-tile, 4-byte rows {ops} M={M} N={N} K={K} alpha={alpha} beta={beta}")
        four = run(ops, A, B, C0, alpha, beta, four=True)
        wide = run(ops, A, B, C0, alpha, beta, four=False)
        assert torch.equal(four.view(torch.int16), wide.view(torch.int16)), f"call {rep}"


@pytest.mark.parametrize("four", [False, True], ids=["16-byte", "4-byte"])
@pytest.mark.parametrize("ops", [(0, 0), (1, 1)], ids=["NN", "TT"])
def test_bias_gelu(ops, four):
    M, N, K = 300, 520, 1000
    A, B, C0 = inputs(M, N, K, 9750 + ops[0], 1.0)
    bias = gi.random_matrix(1, N, "bf16", 9753)[0].contiguous()
    note(f"bf16 few-tile, bias + GELU {ops} M={M} N={N} K={K} four={four}")
    C = run(ops, A, B, C0, 1.25, 1.0, four=four, bias=bias, act="gelu_tanh")
    R, D = oracle_op("bf16", A, B, C0, 1.25, 1.0, bias, "gelu_tanh")
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


def test_scaled():
    from test_scale_gpu import oracle_scaled, scales
    M, N, K = 300, 520, 1000
    A, B, C0 = inputs(M, N, K, 9760, 1.0)
    u, v = scales(M, 9763), scales(N, 9764)
    bias = gi.random_matrix(1, N, "bf16", 9765)[0].contiguous()
    note(f"bf16 few-tile, scaled, M={M} N={N} K={K}")
    C = run((0, 1), A, B, C0, 0.5, 1.0, four=False, bias=bias, act="relu", scales=(u, v))
    R, D = oracle_scaled("bf16", A, B, C0, u, v, bias, "relu", 0.5, 1.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")


@pytest.mark.parametrize("four", [False, True], ids=["16-byte", "4-byte"])
def test_exact_integers(four):
    # Entries in -2 .. 2: every partial sum is an integer of magnitude at
    # most 4 K = 16000, exact in fp32, and so is alpha times it (alpha = 1/64):
    # the kernel's one rounding to bf16 must equal round-to-nearest-even of
    # the exact product.
    M, N, K = 200, 300, 4000
    g = torch.Generator().manual_seed(9770)
    A = torch.randint(-2, 3, (M, K), generator=g).to(torch.bfloat16)
    B = torch.randint(-2, 3, (K, N), generator=g).to(torch.bfloat16)
    note(f"bf16 few-tile, exact integers M={M} N={N} K={K} four={four}")
    C = run((0, 0), A, B, None, 1.0 / 64, 0.0, four=four)
    exact = (A.double() @ B.double()) / 64
    assert torch.equal(C, exact.to(torch.bfloat16))


@pytest.mark.parametrize("four", [False, True], ids=["16-byte", "4-byte"])
def test_repeatable_and_workspace_unused(four):
    # 1024^2 x 4096: the split would cut its 64 tiles of 128 x 128 into 4 K
    # ranges (16 MiB of workspace); the few-tile kernel's 256 tiles take it.
    M, N, K = 1024, 1024, 4096
    assert dg.gemm_bf16_workspace_size(M, N, K) == 0
    A, B, C0 = inputs(M, N, K, 9780, 0.5)
    note(f"bf16 few-tile, repeats and a workspace call, M={M} N={N} K={K} four={four}")
    first = run((0, 0), A, B, C0, 1.0, 0.5, four=four)
    again = run((0, 0), A, B, C0, 1.0, 0.5, four=four)
    assert torch.equal(first.view(torch.int16), again.view(torch.int16))
    # The same call through gemm_bf16_ws with a workspace, rows of
    # K + 4 and N + 4 elements for 4-byte rows.
    pad = 4 if four else 0
    _, a = padded(M, K, K + pad, "bf16", fill=float("nan"))
    a.copy_(A.cuda())
    _, b = padded(K, N, N + pad, "bf16", fill=float("nan"))
    b.copy_(B.cuda())
    _, c = padded(M, N, N + pad, "bf16", fill=float("nan"))
    c.copy_(C0.cuda())
    nbytes = (16 << 20) + 256
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    st = dg.gemm_bf16_ws(M, N, K, 1.0, a.data_ptr(), K + pad, b.data_ptr(), N + pad, 0.5,
                         c.data_ptr(), N + pad, ws.data_ptr(), nbytes, 0)
    torch.cuda.synchronize()
    assert st == dg.GEMM_OK
    assert torch.equal(first.view(torch.int16), c.cpu().view(torch.int16))
    assert int(ws.count_nonzero()) == 0


# Small M that the automatic choice gives this kernel rather than the small-M
# one: 65 .. 128 rows whose 64 x 64 tiles fit one round (with or without a
# workspace), and 33 .. 64 rows with N x K <= 2^25 (plain calls; with a
# workspace the small-M split runs, and must agree with the oracle too).
# Ragged M, N and K; B row-major or stored N x K.
SMALL_M_SHAPES = [(65, 520, 1000), (100, 8192, 300), (128, 1000, 4100), (48, 1000, 4100),
                  (33, 4096, 8192)]


@pytest.mark.parametrize("ops", [(0, 0), (0, 1)], ids=["NN", "NT"])
@pytest.mark.parametrize("shape", SMALL_M_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_m_rows_plain_and_with_workspace(shape, ops):
    M, N, K = shape
    if ops == (0, 0):
        # gemm_plan describes the row-major call.
        from test_bf16_dword_gpu import _ld
        plan = dg.gemm_plan(2, M, N, K, 1.0, 16, _ld(K, False), 16, _ld(N, False), 0.0, 16,
                            _ld(N, False), dg.VARIANT_AUTO)
        assert plan == dg.VARIANT_MFMA
    A, B, C0 = inputs(M, N, K, 9790 + M + ops[1], 0.5)
    R, D = oracle_op("bf16", A, B, C0, 0.75, 0.5)
    for ws in (False, True):
        note(f"bf16 {M} rows {ops} N={N} K={K} workspace={ws}")
        C = run(ops, A, B, C0, 0.75, 0.5, four=False, ws=ws)
        assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16"), f"workspace={ws}"
