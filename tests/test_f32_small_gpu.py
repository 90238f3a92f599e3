"""GPU parity of the fp32 few-tile kernel (GEMM_VARIANT_SMALL) against the
oracle, through the C ABI.

The kernel covers C with 16 x 16, 32 x 32 or 64 x 64 tiles and splits K over
the 4, 8 or 16 waves of each workgroup; the shapes below reach every tile
size and wave count the planner picks (noted per shape), with ragged M, N and
K, K shorter than one 16-k chunk and shorter than one chunk per wave, single
rows and columns, all four operand layouts (with NaN in every padding
element), unaligned rows and bases, the fused bias and activation, and a
workspace call that must run the same kernel as the plain one (same bits).
"""
import numpy as np
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, oracle_ref, run, to_f64, tol
from test_transpose_gpu import check as check_op

pytestmark = pytest.mark.gpu

# (M, N, K) -> tile x tile, waves (from the planner's cost model)
SHAPES = [
    (128, 128, 128),     # 16, 4 (64 tiles; K of 8 chunks)
    (256, 256, 256),     # 16, 8 (the 256^3 workload)
    (256, 256, 4096),    # 16, 16 (long K, one tile per CU)
    (512, 512, 512),     # 32, 8
    (512, 512, 2048),    # 32, 16
    (64, 4096, 100),     # 32, 4
    (1000, 1000, 1000),  # 64, 8 (ragged M, N and K)
    (300, 500, 77),      # 32, 4 (ragged everything)
    (1, 4097, 3000),     # 16, 8 (one row)
    (4097, 1, 3000),     # 16, 8 (one column)
    (33, 17, 5),         # K shorter than one chunk
    (70, 90, 40),        # K of 3 chunks over 4 waves: one wave idle
    (1, 1, 1),
]


def _sid(s):
    return "x".join(map(str, s))


@pytest.mark.parametrize("shape", SHAPES, ids=_sid)
def test_auto_runs_the_few_tile_kernel(shape):
    M, N, K = shape
    assert dg.gemm_plan(4, M, N, K, 1.0, 4096, K, 8192, N, 0.0, 16384, N,
                        dg.VARIANT_AUTO) == dg.VARIANT_SMALL


@pytest.mark.parametrize("shape", SHAPES, ids=_sid)
def test_small_parity(shape):
    M, N, K = shape
    for rep, (alpha, beta) in enumerate(((1.0, 0.0), (0.5, 2.0), (-1.5, 1.0))):
        seed = 7100 + 7 * M + N + rep
        A = gi.random_matrix(M, K, "f32", seed)
        B = gi.random_matrix(K, N, "f32", seed + 1)
        C0 = gi.random_matrix(M, N, "f32", seed + 2) if beta != 0 else None
        note(f"few-tile f32 M={M} N={N} K={K} alpha={alpha} beta={beta}")
        C, st, _ = run("f32", A, B, C0, alpha, beta, dg.VARIANT_AUTO)
        assert st == dg.GEMM_OK, dg.gemm_status_string(st)
        R, D = oracle_ref("f32", A, B, C0, alpha, beta)
        err = oracle.max_rel_err(to_f64(C), R, D)
        assert err <= tol("f32"), f"call {rep}: max error ratio {err:.3e}"


@pytest.mark.parametrize("pad,offset", [((1, 3, 5), 0), ((0, 0, 0), 1), ((2, 1, 7), 3)],
                         ids=["odd_ld", "base+1", "both"])
@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 500, 77), (1000, 1000, 1000)], ids=_sid)
def test_small_unaligned(shape, pad, offset):
    """Rows and bases aligned only to 4 bytes."""
    M, N, K = shape
    A = gi.random_matrix(M, K, "f32", 7300 + M)
    B = gi.random_matrix(K, N, "f32", 7301 + N)
    C0 = gi.random_matrix(M, N, "f32", 7302 + K)
    note(f"few-tile f32 unaligned M={M} N={N} K={K} pad={pad} offset={offset}")
    C, st, _ = run("f32", A, B, C0, 0.75, -0.5, dg.VARIANT_AUTO, pad, offset)
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    assert torch.isfinite(C).all()
    R, D = oracle_ref("f32", A, B, C0, 0.75, -0.5)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("f32")


@pytest.mark.parametrize("ops", [(0, 1), (1, 0), (1, 1)], ids=["ABt", "AtB", "AtBt"])
@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 500, 77), (1000, 1000, 1000),
                                   (64, 4096, 100), (33, 17, 5)], ids=_sid)
def test_small_transposed(shape, ops):
    M, N, K = shape
    check_op("f32", ops[0], ops[1], M, N, K, 7400 + M, alpha=1.25, beta=0.5, pad=(4, 1, 3))


@pytest.mark.parametrize("act", ["none", "relu", "gelu_tanh"])
@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 500, 77), (512, 512, 2048)], ids=_sid)
def test_small_bias_activation(shape, act):
    M, N, K = shape
    check_op("f32", 0, 0, M, N, K, 7500 + M, alpha=0.5, beta=1.0, bias=True, act=act)


def test_small_forced_on_a_large_shape():
    """GEMM_VARIANT_SMALL runs any shape: 2048 x 1536 x 300 (768 tiles of
    64 x 64 over 256 CUs)."""
    M, N, K = 2048, 1536, 300
    A = gi.random_matrix(M, K, "f32", 7600)
    B = gi.random_matrix(K, N, "f32", 7601)
    C0 = gi.random_matrix(M, N, "f32", 7602)
    note(f"few-tile forced M={M} N={N} K={K}")
    C, st, _ = run("f32", A, B, C0, 1.0, 1.0, dg.VARIANT_SMALL)
    assert st == dg.GEMM_OK
    R, D = oracle_ref("f32", A, B, C0, 1.0, 1.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("f32")


@pytest.mark.parametrize("shape", [(256, 256, 256), (1000, 1000, 1000), (512, 512, 2048)], ids=_sid)
def test_small_repeatable_and_workspace_call_identical(shape):
    """Fixed-order sums: repeated calls give the same bits, and gemm_f32_ws
    (which needs no workspace at these shapes) runs the same kernel."""
    M, N, K = shape
    assert dg.gemm_f32_workspace_size(M, N, K) == 0
    A = gi.random_matrix(M, K, "f32", 7700, dist="n").cuda()
    B = gi.random_matrix(K, N, "f32", 7701).cuda()
    C = torch.empty(M, N, device="cuda")
    note(f"few-tile repeat M={M} N={N} K={K}")
    outs = []
    for call in range(4):
        C.fill_(float("nan"))
        if call < 3:
            st = dg.gemm_f32(M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0, C.data_ptr(), N, 0)
        else:
            st = dg.gemm_f32_ws(M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0, C.data_ptr(),
                                N, None, 0, 0)
        assert st == dg.GEMM_OK
        torch.cuda.synchronize()
        outs.append(C.clone())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


def test_small_exact_integers():
    """Integer entries in [-4, 4]: every partial sum is exact, so the result
    equals the oracle bit for bit whatever the split."""
    M, N, K = 300, 500, 1000
    A = gi.small_int_matrix(M, K, "f32", 7800)
    B = gi.small_int_matrix(K, N, "f32", 7801)
    C0 = gi.small_int_matrix(M, N, "f32", 7802)
    note("few-tile small integers")
    C, st, _ = run("f32", A, B, C0, 1.0, -1.0, dg.VARIANT_SMALL)
    assert st == dg.GEMM_OK
    R, _ = oracle_ref("f32", A, B, C0, 1.0, -1.0)
    assert np.array_equal(to_f64(C), R)


# ---- partly full last rounds: a strip of C on the few-tile kernel ----------
#
# (M, N, K): 4096 x 2176 has 32 x 17 = 544 tiles of 128 x 128 on 512 slots;
# the 32 left over are tile column 16, so columns 2048 .. 2175 go to the
# few-tile kernel. 2176 x 4096 leaves tile row 16 (rows 2048 .. 2175). 4095 x
# 2177 x 129 leaves 64 tiles: its last two tile columns (129 columns of C,
# the last one ragged).
PARTITIONED = [(4096, 2176, 200), (2176, 4096, 200), (4095, 2177, 129)]


@pytest.mark.parametrize("shape", PARTITIONED, ids=_sid)
def test_partition_needs_no_workspace(shape):
    # The split-K tail would need a workspace here; the strip does not.
    assert dg.gemm_f32_workspace_size(*shape) == 0


@pytest.mark.parametrize("variant", range(4))
@pytest.mark.parametrize("shape", PARTITIONED, ids=_sid)
def test_partition_parity_full(shape, variant):
    """Every entry against the oracle, through gemm_f32_scaled, with the
    strip's pointers offset in each operand: (0) plain, alpha and beta;
    (1) both operands stored transposed, rows padded to odd lengths;
    (2) row and column scales with bias and GELU; (3) B stored N x K with
    column scales and ReLU, workspace given (and unused)."""
    _partition_parity(shape, variant)


def _partition_parity(shape, variant):
    from test_scale_gpu import oracle_scaled, run_scaled, scales
    M, N, K = shape
    ops, pad, ws = [((0, 0), (0, 0, 0), False), ((1, 1), (1, 3, 5), False),
                    ((0, 0), (4, 4, 4), False), ((0, 1), (0, 0, 0), True)][variant]
    alpha, beta = [(0.5, 2.0), (1.0, -1.0), (1.0, 0.5), (-0.75, 0.0)][variant]
    seed = 7900 + M + variant
    A = gi.random_matrix(M, K, "f32", seed)
    B = gi.random_matrix(K, N, "f32", seed + 1)
    C0 = gi.random_matrix(M, N, "f32", seed + 2) if beta != 0 else None
    u = scales(M, seed + 3) if variant == 2 else None
    v = scales(N, seed + 4) if variant in (2, 3) else None
    bias = gi.random_matrix(1, N, "f32", seed + 5)[0].contiguous() if variant == 2 else None
    act = {2: "gelu_tanh", 3: "relu"}.get(variant, "none")
    note(f"partition f32 M={M} N={N} K={K} ops={ops} pad={pad} ws={ws} variant={variant}")
    C, st = run_scaled("f32", A, B, C0, u, v, bias, act, alpha, beta, ops, pad, ws)
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    assert torch.isfinite(C).all()
    R, D = oracle_scaled("f32", A, B, C0, u, v, bias, act if (bias is not None or act != "none") else None,
                         alpha, beta)
    err = oracle.max_rel_err(to_f64(C), R, D)
    assert err <= tol("f32"), f"max error ratio {err:.3e}"


@pytest.mark.parametrize("shape", PARTITIONED, ids=_sid)
def test_partition_against_tiled_kernel_alone(shape):
    """The tiled kernel alone (forced) gives the same outputs outside the
    strip bit for bit: the partition leaves the tiled part's arithmetic as it
    was."""
    M, N, K = shape
    A = gi.random_matrix(M, K, "f32", 8000 + M)
    B = gi.random_matrix(K, N, "f32", 8001 + N)
    note(f"partition vs tiled alone M={M} N={N} K={K}")
    Ca, st, _ = run("f32", A, B, None, 1.0, 0.0, dg.VARIANT_AUTO)
    assert st == dg.GEMM_OK
    forced = dg.VARIANT_MFMA if K % 4 == 0 and N % 4 == 0 else dg.VARIANT_GENERAL
    Ct, st, _ = run("f32", A, B, None, 1.0, 0.0, forced)
    assert st == dg.GEMM_OK
    tm, tn = (M + 127) // 128, (N + 127) // 128
    tail = (tm * tn) % 512
    if M == 2176:            # row strip: tile rows from 16 on
        same = (slice(0, (tm - -(-tail // tn)) * 128), slice(None))
    else:                    # column strip
        same = (slice(None), slice(0, (tn - -(-tail // tm)) * 128))
    assert torch.equal(Ca[same].view(torch.int32), Ct[same].view(torch.int32))
    R, D = oracle_ref("f32", A, B, None, 1.0, 0.0)
    assert oracle.max_rel_err(to_f64(Ca), R, D) <= tol("f32")


# ---- one round with two tiles on some CUs: the tiles past one per CU ------
#
# With 257 .. 511 tiles of 128 x 128 the tiled kernel would run a single
# round with two tiles on some CUs. The trailing tile columns (or rows) that
# hold the tiles past one per CU go to the few-tile kernel instead, and the
# tiled kernel runs one tile per CU on the rest. (M, N, K, strip): 2048 x 2560
# (320 tiles): columns 2048 .. 2559; 2177 x 2300 (324 tiles, both edges
# ragged): rows 1792 .. 2176 (385 rows); 3072 x 2048 (384 tiles): rows
# 2048 .. 3071; 2304^2 (324 tiles): columns 1792 .. 2303.
ONE_ROUND = [((2048, 2560, 200), ("cols", 2048)), ((2177, 2300, 129), ("rows", 1792)),
             ((3072, 2048, 100), ("rows", 2048)), ((2304, 2304, 136), ("cols", 1792))]


@pytest.mark.parametrize("variant", range(4))
@pytest.mark.parametrize("case", ONE_ROUND, ids=lambda c: _sid(c[0]))
def test_one_round_partition_parity_full(case, variant):
    """As test_partition_parity_full, for the one-round partition."""
    _partition_parity(case[0], variant)


@pytest.mark.parametrize("case", ONE_ROUND, ids=lambda c: _sid(c[0]))
def test_one_round_partition_against_tiled_kernel_alone(case):
    """Outside the strip the outputs are the tiled kernel's alone (forced),
    bit for bit; inside, they match the oracle."""
    (M, N, K), (by, start) = case
    A = gi.random_matrix(M, K, "f32", 8100 + M)
    B = gi.random_matrix(K, N, "f32", 8101 + N)
    note(f"one-round partition vs tiled alone M={M} N={N} K={K}")
    Ca, st, _ = run("f32", A, B, None, 1.0, 0.0, dg.VARIANT_AUTO)
    assert st == dg.GEMM_OK
    forced = dg.VARIANT_MFMA if K % 4 == 0 and N % 4 == 0 else dg.VARIANT_GENERAL
    Ct, st, _ = run("f32", A, B, None, 1.0, 0.0, forced)
    assert st == dg.GEMM_OK
    same = (slice(0, start), slice(None)) if by == "rows" else (slice(None), slice(0, start))
    assert torch.equal(Ca[same].view(torch.int32), Ct[same].view(torch.int32))
    R, D = oracle_ref("f32", A, B, None, 1.0, 0.0)
    assert oracle.max_rel_err(to_f64(Ca), R, D) <= tol("f32")
