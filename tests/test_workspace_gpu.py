"""GPU parity of gemm_bf16_ws (split-K over a caller workspace) against the
CPU oracle, plus the workspace contract: repeated calls reuse it without
clearing (the counters are left at zero), results do not depend on timing
(partials are added in a fixed order), and shapes that do not split ignore it.
"""
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, oracle_ref, padded, to_f64, tol

pytestmark = pytest.mark.gpu


def workspace(M, N, K):
    n = dg.gemm_bf16_workspace_size(M, N, K)
    # torch's allocations are 256-byte aligned; zero-filled before first use.
    return torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda"), n


def run_ws(A, B, C0, alpha, beta, ws, nbytes, ld_pad=(0, 0, 0)):
    M, K = A.shape
    N = B.shape[1]
    lda, ldb, ldc = K + ld_pad[0], N + ld_pad[1], N + ld_pad[2]
    _, a = padded(M, K, lda, "bf16", fill=float("nan"))
    _, b = padded(K, N, ldb, "bf16", fill=float("nan"))
    _, c = padded(M, N, ldc, "bf16", fill=float("nan"))
    a.copy_(A.cuda())
    b.copy_(B.cuda())
    if C0 is not None:
        c.copy_(C0.cuda())
    st = dg.gemm_bf16_ws(M, N, K, alpha, a.data_ptr(), lda, b.data_ptr(), ldb, beta,
                         c.data_ptr(), ldc, ws.data_ptr() if nbytes else None, nbytes, 0)
    torch.cuda.synchronize()
    return c.cpu(), st


# Row-major B with 65 .. 128 rows reaches this kernel's split no more: such
# calls with fewer than 16 strips of 256 columns go to the few-tile kernel,
# and wider ones to the streaming split (STREAM_SHAPES below). 33 .. 64 rows
# split only with K > 4096 or N x K > 2^25. The split needs K >= 4096.
SHAPES = [(16, 264, 4100), (1, 1032, 4104), (17, 64, 4200), (32, 8, 4136), (5, 4096, 4104),
          (16, 128, 5000), (31, 520, 8192), (3, 1024, 8200), (33, 520, 4200), (64, 264, 4200)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_split_k_parity(shape):
    M, N, K = shape
    assert dg.gemm_bf16_workspace_size(M, N, K) > 0       # these shapes do split
    ws, n = workspace(M, N, K)
    for rep, (alpha, beta) in enumerate(((1.5, -0.5), (1.0, 0.0), (0.25, 1.0))):
        seed = 900 + 10 * M + rep
        A = gi.random_matrix(M, K, "bf16", seed, dist="n")
        B = gi.random_matrix(K, N, "bf16", seed + 1)
        C0 = gi.random_matrix(M, N, "bf16", seed + 2) if beta != 0 else None
        note(f"gemm_bf16_ws M={M} N={N} K={K} alpha={alpha} beta={beta} ws={n}")
        C, st = run_ws(A, B, C0, alpha, beta, ws, n)
        assert st == dg.GEMM_OK, dg.gemm_status_string(st)
        R, D = oracle_ref("bf16", A, B, C0, alpha, beta)
        err = oracle.max_rel_err(to_f64(C), R, D)
        assert err <= tol("bf16"), f"call {rep}: max error ratio {err:.3e}"
    # Every counter is back at zero after the calls.
    strips = (N + 63) // 64
    assert int(ws[:4 * strips].view(torch.int32).abs().sum()) == 0


# Shapes with at least 16 strips of 256 columns (N > 3840) and at least 8
# blocks of 32 rows of K: with a workspace and row-major B they run on the
# streaming kernel (K interleaved over 2 to 16 workgroups per strip in 32-row
# blocks), ragged in M, N and K.
STREAM_SHAPES = [(16, 3841, 4100), (1, 4100, 4104), (17, 5000, 4200), (128, 8256, 4104),
                 (33, 4352, 4200), (7, 4104, 4360), (64, 6000, 4133), (2, 8192, 4200),
                 (100, 8320, 4100), (65, 8256, 4104)]


@pytest.mark.parametrize("shape", STREAM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_stream_split_parity(shape):
    M, N, K = shape
    assert dg.gemm_bf16_workspace_size(M, N, K) > 0
    ws, n = workspace(M, N, K)
    for rep, (alpha, beta, pad) in enumerate(((1.5, -0.5, (0, 0, 0)), (1.0, 0.0, (8, 16, 24)),
                                              (0.25, 1.0, (0, 8, 0)))):
        seed = 7000 + 10 * M + rep
        A = gi.random_matrix(M, K, "bf16", seed, dist="n")
        B = gi.random_matrix(K, N, "bf16", seed + 1)
        C0 = gi.random_matrix(M, N, "bf16", seed + 2) if beta != 0 else None
        note(f"gemm_bf16_ws stream M={M} N={N} K={K} alpha={alpha} beta={beta} pad={pad}")
        C, st = run_ws(A, B, C0, alpha, beta, ws, n, ld_pad=pad)
        assert st == dg.GEMM_OK, dg.gemm_status_string(st)
        R, D = oracle_ref("bf16", A, B, C0, alpha, beta)
        err = oracle.max_rel_err(to_f64(C), R, D)
        assert err <= tol("bf16"), f"call {rep}: max error ratio {err:.3e}"
    # The counters (one int per 256-column strip) are back at zero.
    strips = (N + 255) // 256
    assert int(ws[:4 * strips].view(torch.int32).abs().sum()) == 0


def test_stream_split_is_deterministic():
    M, N, K = 16, 4352, 4104
    ws, n = workspace(M, N, K)
    A = gi.random_matrix(M, K, "bf16", 7990, dist="n")
    B = gi.random_matrix(K, N, "bf16", 7991)
    note(f"gemm_bf16_ws stream determinism M={M} N={N} K={K}")
    first, st = run_ws(A, B, None, 1.0, 0.0, ws, n)
    assert st == dg.GEMM_OK
    for _ in range(3):
        again, st = run_ws(A, B, None, 1.0, 0.0, ws, n)
        assert st == dg.GEMM_OK
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))


def test_split_k_is_deterministic():
    M, N, K = 16, 1032, 4104
    ws, n = workspace(M, N, K)
    A = gi.random_matrix(M, K, "bf16", 990, dist="n")
    B = gi.random_matrix(K, N, "bf16", 991)
    note(f"gemm_bf16_ws determinism M={M} N={N} K={K}")
    first, st = run_ws(A, B, None, 1.0, 0.0, ws, n)
    assert st == dg.GEMM_OK
    for _ in range(3):
        again, st = run_ws(A, B, None, 1.0, 0.0, ws, n)
        assert st == dg.GEMM_OK
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))


def test_padded_rows_and_no_split_shapes():
    # Padded 16-byte rows keep the split; a shape that fills the GPU ignores the workspace.
    M, N, K = 20, 264, 1000
    ws, n = workspace(M, N, K)
    A = gi.random_matrix(M, K, "bf16", 995, dist="n")
    B = gi.random_matrix(K, N, "bf16", 996)
    C0 = gi.random_matrix(M, N, "bf16", 997)
    note(f"gemm_bf16_ws padded M={M} N={N} K={K}")
    C, st = run_ws(A, B, C0, 1.0, 1.0, ws, n, ld_pad=(8, 16, 24))
    assert st == dg.GEMM_OK
    R, D = oracle_ref("bf16", A, B, C0, 1.0, 1.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol("bf16")
    # A NULL workspace is accepted (no split), here for a 64-row tile.
    M2 = 40
    A2 = gi.random_matrix(M2, K, "bf16", 998, dist="n")
    note(f"gemm_bf16_ws no-split M={M2} N={N} K={K}")
    C2, st = run_ws(A2, B, None, 1.0, 0.0, ws, 0)
    assert st == dg.GEMM_OK
    R2, D2 = oracle_ref("bf16", A2, B, None, 1.0, 0.0)
    assert oracle.max_rel_err(to_f64(C2), R2, D2) <= tol("bf16")


# ---- fp32: split K for the last round of tiles -------------------------------

def run_ws_f32(A, B, C0, alpha, beta, ws, nbytes, ld_pad=(0, 0, 0)):
    M, K = A.shape
    N = B.shape[1]
    lda, ldb, ldc = K + ld_pad[0], N + ld_pad[1], N + ld_pad[2]
    _, a = padded(M, K, lda, "f32", fill=float("nan"))
    _, b = padded(K, N, ldb, "f32", fill=float("nan"))
    _, c = padded(M, N, ldc, "f32", fill=float("nan"))
    a.copy_(A.cuda())
    b.copy_(B.cuda())
    if C0 is not None:
        c.copy_(C0.cuda())
    st = dg.gemm_f32_ws(M, N, K, alpha, a.data_ptr(), lda, b.data_ptr(), ldb, beta,
                        c.data_ptr(), ldc, ws.data_ptr() if nbytes else None, nbytes, 0)
    torch.cuda.synchronize()
    return c.cpu(), st


# Aligned (vector) and unaligned (element-wise) rows, ragged tiles, K ranges of
# one or several slabs. Shapes with few tiles split only with at least 2^18
# tile-k (fewer go to the few-tile kernel, which needs no workspace).
F32_SHAPES = [((1100, 1030, 4100), (0, 0, 0)),     # 81 tiles, 6 ranges of 22 slabs
              ((1700, 1300, 2100), (4, 8, 12)),    # 154 tiles, 3 ranges
              ((600, 4100, 300), (0, 0, 0)),       # 165 tiles, 3 ranges of 3-4 slabs
              ((4095, 1000, 1000), (1, 3, 5)),     # 256 tiles, unaligned, 2 ranges
              # a last round more than half full: 18 x 18 = 324 tiles on 512
              # slots, every tile cut into 3 K ranges (two rounds of units)
              ((2300, 2290, 2050), (0, 0, 0)), ((2300, 2290, 2050), (1, 3, 5))]


@pytest.mark.parametrize("case", F32_SHAPES, ids=lambda c: "x".join(map(str, c[0])) + f"_pad{c[1][0]}")
def test_f32_split_k_parity(case):
    (M, N, K), pad = case
    nbytes = dg.gemm_f32_workspace_size(M, N, K)
    assert nbytes > 0                                      # these shapes do split
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for rep, (alpha, beta) in enumerate(((0.5, 2.0), (1.0, 0.0))):
        seed = 1700 + M + rep
        A = gi.random_matrix(M, K, "f32", seed)
        B = gi.random_matrix(K, N, "f32", seed + 1)
        C0 = gi.random_matrix(M, N, "f32", seed + 2) if beta != 0 else None
        note(f"gemm_f32_ws M={M} N={N} K={K} pad={pad} alpha={alpha} beta={beta} ws={nbytes}")
        C, st = run_ws_f32(A, B, C0, alpha, beta, ws, nbytes, pad)
        assert st == dg.GEMM_OK, dg.gemm_status_string(st)
        R, D = oracle_ref("f32", A, B, C0, alpha, beta)
        err = oracle.max_rel_err(to_f64(C), R, D)
        assert err <= tol("f32"), f"call {rep}: max error ratio {err:.3e}"
    tiles = ((M + 127) // 128) * ((N + 127) // 128)
    assert int(ws[:4 * tiles].view(torch.int32).abs().sum()) == 0


def test_f32_split_k_deterministic():
    M, N, K = 600, 4100, 300
    nbytes = dg.gemm_f32_workspace_size(M, N, K)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    A = gi.random_matrix(M, K, "f32", 1790)
    B = gi.random_matrix(K, N, "f32", 1791)
    note(f"gemm_f32_ws determinism M={M} N={N} K={K}")
    first, st = run_ws_f32(A, B, None, 1.0, 0.0, ws, nbytes)
    assert st == dg.GEMM_OK
    for _ in range(3):
        again, st = run_ws_f32(A, B, None, 1.0, 0.0, ws, nbytes)
        assert st == dg.GEMM_OK
        assert torch.equal(first.view(torch.int32), again.view(torch.int32))


# ---- bf16 tiled kernel: split K when few tiles leave most CUs idle -----------

# (shape, ld padding): ragged M, N and K, K ranges of one or several slabs,
# the ragged K tail in the last range, padded 16-byte rows.
# Long K against few tiles, so that the split beats the few-tile kernel.
TILED_SHAPES = [((300, 520, 8200), (0, 0, 0)), ((257, 264, 4100), (0, 0, 0)),
                ((512, 512, 16384), (0, 0, 0)), ((640, 1000, 8192), (8, 16, 24)),
                ((129, 1000, 8200), (0, 0, 0))]


@pytest.mark.parametrize("case", TILED_SHAPES,
                         ids=lambda c: "x".join(map(str, c[0])) + f"_pad{c[1][0]}")
@pytest.mark.parametrize("ops", [(0, 0), (0, 1), (1, 0), (1, 1)], ids=["NN", "NT", "TN", "TT"])
def test_bf16_tiled_split_k_parity(case, ops):
    from test_transpose_gpu import check
    (M, N, K), pad = case
    assert dg.gemm_bf16_workspace_size(M, N, K) > 0          # these shapes do split
    for rep, (alpha, beta) in enumerate(((1.0, 0.0), (0.5, 2.0))):
        check("bf16", ops[0], ops[1], M, N, K, 5100 + M + rep, alpha, beta, pad, ws=True)
    check("bf16", ops[0], ops[1], M, N, K, 5150 + M, 1.0, 1.0, pad, bias=True, act="gelu_tanh",
          ws=True)


def test_bf16_tiled_split_k_deterministic_and_counters_reset():
    from test_transpose_gpu import run_op
    M, N, K = 512, 512, 16384
    A = gi.random_matrix(M, K, "bf16", 5200, dist="n")
    B = gi.random_matrix(K, N, "bf16", 5201)
    nbytes = dg.gemm_bf16_workspace_size(M, N, K)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    a, b = A.cuda(), B.cuda()
    outs = []
    for _ in range(3):
        note(f"gemm_bf16_ws tiled split determinism M={M} N={N} K={K}")
        c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        st = dg.gemm_bf16_ws(M, N, K, 1.0, a.data_ptr(), K, b.data_ptr(), N, 0.0, c.data_ptr(), N,
                             ws.data_ptr(), nbytes, 0)
        torch.cuda.synchronize()
        assert st == dg.GEMM_OK
        outs.append(c.cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))
    assert int(ws[:16 * 4].view(torch.int32).abs().sum()) == 0         # 16 tiles' counters
    R, D = oracle_ref("bf16", A, B, None, 1.0, 0.0)
    assert oracle.max_rel_err(to_f64(outs[0]), R, D) <= tol("bf16")

