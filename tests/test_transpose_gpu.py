"""GPU parity of the transposed-operand entry points (gemm_f32_op,
gemm_bf16_op) against the oracle.

The oracle computes C = act(alpha * A B + bias) + beta * C0 on the logical
operands; the tests store op(A) = A^T as a K x M row-major array (and op(B) =
B^T as N x K) and hand the logical matrices to the oracle. Every layout
combination runs through the vector kernels (16-byte rows), the unaligned
kernels, padded leading dimensions, small M, tiny and ragged shapes, the fp32
split-K tail and the fused epilogue.
"""
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import full_max_err, note, padded, to_f64, tol, workload_reference

pytestmark = pytest.mark.gpu

OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
OP_ID = {0: "N", 1: "T"}
ACTS = {"none": dg.ACT_NONE, "relu": dg.ACT_RELU, "gelu_tanh": dg.ACT_GELU_TANH}


def _store(X, trans, ld_pad, dtype, fill=float("nan")):
    """Device storage of the logical matrix X (rows x cols): X itself, or X^T
    when `trans`, with `ld_pad` extra elements per row."""
    S = X.t().contiguous() if trans else X
    rows, cols = S.shape
    ld = max(cols, 1) + ld_pad
    buf, view = padded(rows, cols, ld, dtype, fill=fill)
    if rows and cols:
        view.copy_(S.cuda())
    return buf, view, ld


def run_op(dtype, opa, opb, A, B, C0, alpha, beta, ld_pad=(0, 0, 0), bias=None, act="none",
           ws=False):
    M, K = A.shape
    N = B.shape[1]
    _, a, lda = _store(A, opa, ld_pad[0], dtype)
    _, b, ldb = _store(B, opb, ld_pad[1], dtype)
    ldc = max(N, 1) + ld_pad[2]
    _, c = padded(M, N, ldc, dtype, fill=float("nan"))
    if C0 is not None:
        c.copy_(C0.cuda())
    bb = bias.cuda() if bias is not None else None
    size_fn = dg.gemm_f32_workspace_size if dtype == "f32" else dg.gemm_bf16_workspace_size
    nbytes = size_fn(M, N, K) if ws else 0
    wbuf = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    fn = dg.gemm_f32_op if dtype == "f32" else dg.gemm_bf16_op
    st = fn(opa, opb, M, N, K, float(alpha), a.data_ptr(), lda, b.data_ptr(), ldb, float(beta),
            c.data_ptr(), ldc, None if bb is None else bb.data_ptr(), ACTS[act],
            wbuf.data_ptr() if nbytes else None, nbytes, 0)
    torch.cuda.synchronize()
    return c.cpu(), st, nbytes


def oracle_op(dtype, A, B, C0, alpha, beta, bias=None, act=None, rows=None, cols=None):
    return oracle.gemm(gi.as_numpy(A), gi.as_numpy(B),
                       None if (C0 is None or beta == 0) else gi.as_numpy(C0),
                       float(alpha), float(beta), dtype, rows=rows, cols=cols,
                       bias=None if bias is None else gi.as_numpy(bias), act=act)


def check(dtype, opa, opb, M, N, K, seed, alpha=1.0, beta=0.0, pad=(0, 0, 0), bias=False,
          act="none", ws=False):
    A = gi.random_matrix(M, K, dtype, seed, dist="n")
    B = gi.random_matrix(K, N, dtype, seed + 1)
    C0 = gi.random_matrix(M, N, dtype, seed + 2) if beta != 0 else None
    bv = gi.random_matrix(1, N, dtype, seed + 3)[0].contiguous() if bias else None
    note(f"gemm_{dtype}_op {OP_ID[opa]}{OP_ID[opb]} M={M} N={N} K={K} pad={pad} "
         f"alpha={alpha} beta={beta} bias={bias} act={act} ws={ws}")
    C, st, nbytes = run_op(dtype, opa, opb, A, B, C0, alpha, beta, pad, bv, act, ws)
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    R, D = oracle_op(dtype, A, B, C0, alpha, beta, bv,
                     act if (bias or act != "none") else None)
    err = oracle.max_rel_err(to_f64(C), R, D)
    assert err <= tol(dtype), f"max error ratio {err:.3e}"
    return nbytes


SHAPES = [
    ((300, 520, 200), (0, 0, 0)),     # vector kernels, ragged M, N and K
    ((257, 264, 136), (8, 8, 8)),     # padded 16-byte rows
    ((130, 200, 129), (1, 3, 5)),     # unaligned rows
    ((16, 264, 300), (0, 0, 0)),      # small M (bf16: small-M kernel for A B and A B^T)
    ((1, 1, 1), (0, 0, 0)),
    ((3, 5, 7), (0, 0, 0)),
    ((64, 1, 65), (0, 0, 0)),
    ((513, 33, 64), (0, 0, 0)),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ops", OPS, ids=lambda o: OP_ID[o[0]] + OP_ID[o[1]])
@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "x".join(map(str, c[0])) + f"_pad{c[1][0]}")
def test_op_parity(dtype, ops, case):
    (M, N, K), pad = case
    for rep, (alpha, beta) in enumerate(((1.0, 0.0), (0.5, 2.0))):
        check(dtype, ops[0], ops[1], M, N, K, 4100 + 13 * M + N + rep, alpha, beta, pad)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ops", OPS[1:], ids=lambda o: OP_ID[o[0]] + OP_ID[o[1]])
def test_op_with_epilogue(dtype, ops):
    check(dtype, ops[0], ops[1], 300, 264, 130, 4400, 1.0, 1.0, bias=True, act="gelu_tanh")
    check(dtype, ops[0], ops[1], 130, 72, 77, 4410, -0.5, 0.0, (1, 1, 1), bias=True, act="relu")


@pytest.mark.parametrize("ops", OPS[1:], ids=lambda o: OP_ID[o[0]] + OP_ID[o[1]])
def test_f32_op_split_k(ops):
    # 165 tiles in 3 K ranges; 256 unaligned tiles in 2.
    nbytes = check("f32", ops[0], ops[1], 600, 4100, 300, 4500, 0.5, 2.0, ws=True)
    assert nbytes > 0
    nbytes = check("f32", ops[0], ops[1], 4095, 1000, 1000, 4510, 1.0, 0.0, (1, 3, 5), ws=True)
    assert nbytes > 0


@pytest.mark.parametrize("ops", OPS, ids=lambda o: OP_ID[o[0]] + OP_ID[o[1]])
def test_nn_op_is_bit_identical_to_plain(ops):
    """op(A) op(B) with transposed storage equals the plain call on the
    materialised transposes, bit for bit (same kernel family, same k order).
    Every stored row is 16 bytes long in every layout (M, N, K multiples of
    8), so that all of them take the same kernel (the few-tile kernel here,
    whose order of K differs from the tiled kernels')."""
    if ops == (0, 0):
        pytest.skip("the plain call itself")
    M, N, K = 264, 264, 200
    A = gi.random_matrix(M, K, "bf16", 4600, dist="n")
    B = gi.random_matrix(K, N, "bf16", 4601)
    note(f"gemm_bf16_op {OP_ID[ops[0]]}{OP_ID[ops[1]]} vs NN, bitwise")
    C1, st1, _ = run_op("bf16", ops[0], ops[1], A, B, None, 1.0, 0.0)
    C2, st2, _ = run_op("bf16", 0, 0, A, B, None, 1.0, 0.0)
    assert st1 == st2 == dg.GEMM_OK
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


def test_op_argument_checks():
    note("gemm_op argument checks")
    M, N, K = 64, 48, 32
    a = torch.zeros(K, M, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(N, K, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    bad = dg.GEMM_ERR_INVALID_VALUE
    args = (1.0, a.data_ptr(), M, b.data_ptr(), K, 0.0, c.data_ptr(), N)
    assert dg.gemm_bf16_op(2, 0, M, N, K, *args) == bad
    assert dg.gemm_bf16_op(0, -1, M, N, K, *args) == bad
    # lda must cover the stored row length: M for op T, K for op N.
    assert dg.gemm_bf16_op(1, 1, M, N, K, 1.0, a.data_ptr(), M - 1, b.data_ptr(), K, 0.0,
                           c.data_ptr(), N) == bad
    assert dg.gemm_bf16_op(1, 1, M, N, K, 1.0, a.data_ptr(), M, b.data_ptr(), K - 1, 0.0,
                           c.data_ptr(), N) == bad
    assert dg.gemm_bf16_op(1, 1, M, N, K, *args) == dg.GEMM_OK
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,ops", [(d, o) for d in ("bf16", "f32") for o in OPS[1:]],
                         ids=lambda v: v if isinstance(v, str) else OP_ID[v[0]] + OP_ID[v[1]])
def test_op_full_size(dtype, ops):
    """4096^3 with transposed storage, in the launch configuration the
    benchmark times, against the oracle over every entry of C (the logical
    operands are those of the 4096^3 workloads, so their reference is too)."""
    wid = 3 if dtype == "bf16" else 2
    w = gi.WORKLOADS[wid]
    d = gi.make(w)
    note(f"gemm_{dtype}_op {OP_ID[ops[0]]}{OP_ID[ops[1]]} 4096^3 full size")
    C, st, _ = run_op(dtype, ops[0], ops[1], d["A"], d["B"], None, 1.0, 0.0)
    assert st == dg.GEMM_OK
    R, D = workload_reference(wid)
    err = full_max_err(C, R, D)
    note(f"all {w.M}x{w.N} entries, max error ratio {err:.3e}")
    assert err <= tol(dtype)


# Small M with B stored N x K (x W^T with W kept as [out][in]): the small-M
# vector kernel reads the transposed B directly; unaligned rows fall back to
# the tiled kernels.
SMALL_M_TB = [((16, 520, 300), (0, 0, 0), False), ((32, 72, 130), (0, 0, 0), False),
              ((1, 1032, 4104), (0, 0, 0), True), ((17, 64, 4200), (0, 0, 0), True),
              ((5, 200, 77), (8, 8, 8), False), ((5, 100, 77), (1, 1, 1), False),
              ((3, 1024, 8200), (0, 0, 0), True)]


@pytest.mark.parametrize("case", SMALL_M_TB,
                         ids=lambda c: "x".join(map(str, c[0])) + f"_pad{c[1][0]}" + ("_ws" if c[2] else ""))
def test_small_m_transposed_b(case):
    (M, N, K), pad, ws = case
    for rep, (alpha, beta) in enumerate(((1.0, 0.0), (0.5, 2.0))):
        nbytes = check("bf16", 0, 1, M, N, K, 4800 + M + rep, alpha, beta, pad, ws=ws)
        assert nbytes > 0 or not ws
    check("bf16", 0, 1, M, N, K, 4850 + M, 1.0, 1.0, pad, bias=True, act="gelu_tanh", ws=ws)


def test_small_m_transposed_b_is_deterministic():
    """Repeated calls give the same bits, with and without split K (partials
    are added in a fixed order; each strip's chunk order is fixed)."""
    M, N, K = 16, 1032, 4104
    A = gi.random_matrix(M, K, "bf16", 4900, dist="n")
    B = gi.random_matrix(K, N, "bf16", 4901)
    for ws in (False, True):
        note(f"gemm_bf16_op NT small M determinism ws={ws}")
        first, st, _ = run_op("bf16", 0, 1, A, B, None, 1.0, 0.0, ws=ws)
        assert st == dg.GEMM_OK
        for _ in range(2):
            again, st, _ = run_op("bf16", 0, 1, A, B, None, 1.0, 0.0, ws=ws)
            assert st == dg.GEMM_OK
            assert torch.equal(first.view(torch.int16), again.view(torch.int16))


def test_small_m_transposed_b_full_size():
    """16 x 8192 x 8192 with B stored N x K, split-K, as the benchmark times it,
    against the oracle over every entry."""
    w = gi.WORKLOADS[52]
    d = gi.make(w)
    note("gemm_bf16_op NT 16x8192x8192 full size, split-K")
    C, st, nbytes = run_op("bf16", 0, 1, d["A"], d["B"], None, 1.0, 0.0, ws=True)
    assert st == dg.GEMM_OK and nbytes > 0
    R, D = workload_reference(52)
    err = full_max_err(C, R, D)
    note(f"all {w.M}x{w.N} entries, max error ratio {err:.3e}")
    assert err <= tol("bf16")
