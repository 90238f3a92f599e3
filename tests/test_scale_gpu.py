"""GPU parity of the quantisation-scale entry points (gemm_f32_scaled,
gemm_bf16_scaled) against the oracle's scaled form,

    C = act(alpha * u_i * v_j * sum_k op(A)_ik op(B)_kj + bias_j) + beta * C0,

through every kernel family the plain calls use (bf16 tiled, unaligned,
small-M vector, 64-column and streaming split-K, element-wise small M, the
tiled split for M > 128, fp32 tiled aligned, unaligned and split-K tail, the
fp32 few-tile kernel, and transposed operands). Two bit-identity checks pin the placement of the
factors: all-ones scales give exactly the unscaled epilogue, and power-of-two
scales give exactly the plain product of pre-scaled operands (scaling by a
power of two commutes with every rounding)."""
import numpy as np
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import full_max_err, note, padded, to_f64, tol

pytestmark = pytest.mark.gpu

ACTS = {"none": dg.ACT_NONE, "relu": dg.ACT_RELU, "gelu_tanh": dg.ACT_GELU_TANH}


def scales(n: int, seed: int, pow2: bool = False) -> torch.Tensor:
    """n seeded fp32 factors: +-U[0.25, 4), or +-2^e with e in -3 .. 3."""
    rng = np.random.default_rng(seed)
    sign = rng.choice([-1.0, 1.0], n)
    mag = np.exp2(rng.integers(-3, 4, n)) if pow2 else rng.uniform(0.25, 4.0, n)
    return torch.from_numpy((sign * mag).astype(np.float32))


def _store(X, trans, ld_pad, dtype):
    S = X.t().contiguous() if trans else X
    rows, cols = S.shape
    ld = max(cols, 1) + ld_pad
    buf, view = padded(rows, cols, ld, dtype, fill=float("nan"))
    if rows and cols:
        view.copy_(S.cuda())
    return buf, view, ld


def run_scaled(dtype, A, B, C0, u, v, bias, act, alpha, beta, ops=(0, 0), pad=(0, 0, 0),
               ws=False, entry="scaled"):
    """One call through the C ABI; entry "scaled" (gemm_*_scaled) or "op"
    (gemm_*_op, which takes no scales). Returns (C on the host, status)."""
    M, K = A.shape
    N = B.shape[1]
    _, a, lda = _store(A, ops[0], pad[0], dtype)
    _, b, ldb = _store(B, ops[1], pad[1], dtype)
    ldc = max(N, 1) + pad[2]
    _, c = padded(M, N, ldc, dtype, fill=float("nan"))
    if C0 is not None:
        c.copy_(C0.cuda())
    keep = []

    def dev(t):
        if t is None:
            return None
        d = t.cuda()
        keep.append(d)
        return d.data_ptr()
    size_fn = dg.gemm_f32_workspace_size if dtype == "f32" else dg.gemm_bf16_workspace_size
    nbytes = size_fn(M, N, K) if ws else 0
    wbuf = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    wsp = wbuf.data_ptr() if nbytes else None
    if entry == "scaled":
        fn = dg.gemm_f32_scaled if dtype == "f32" else dg.gemm_bf16_scaled
        st = fn(ops[0], ops[1], M, N, K, float(alpha), a.data_ptr(), lda, b.data_ptr(), ldb,
                float(beta), c.data_ptr(), ldc, dev(u), dev(v), dev(bias), ACTS[act], wsp,
                nbytes, 0)
    else:
        fn = dg.gemm_f32_op if dtype == "f32" else dg.gemm_bf16_op
        st = fn(ops[0], ops[1], M, N, K, float(alpha), a.data_ptr(), lda, b.data_ptr(), ldb,
                float(beta), c.data_ptr(), ldc, dev(bias), ACTS[act], wsp, nbytes, 0)
    torch.cuda.synchronize()
    return c.cpu(), st


def oracle_scaled(dtype, A, B, C0, u, v, bias, act, alpha, beta):
    return oracle.gemm(gi.as_numpy(A), gi.as_numpy(B),
                       None if (C0 is None or beta == 0) else gi.as_numpy(C0),
                       float(np.float32(alpha)), float(np.float32(beta)), dtype,
                       bias=None if bias is None else gi.as_numpy(bias), act=act,
                       row_scale=None if u is None else u.numpy(),
                       col_scale=None if v is None else v.numpy())


# (dtype, (M, N, K), ld_pad, ops, workspace): one case per kernel family and edge.
CASES = [
    ("bf16", (300, 520, 200), (0, 0, 0), (0, 0), False),     # tiled, ragged M and K
    ("bf16", (257, 264, 130), (8, 8, 8), (0, 0), False),     # tiled, padded rows
    ("bf16", (130, 200, 129), (1, 3, 5), (0, 0), False),     # unaligned rows: general kernel
    ("bf16", (16, 520, 300), (0, 0, 0), (0, 0), False),      # small-M vector
    ("bf16", (32, 72, 130), (0, 0, 0), (0, 0), False),       # small-M vector, two row blocks
    ("bf16", (16, 1032, 4100), (0, 0, 0), (0, 0), True),     # small-M 64-column split
    ("bf16", (16, 4352, 4100), (0, 0, 0), (0, 0), True),     # small-M streaming split
    ("bf16", (100, 4160, 1500), (8, 8, 8), (0, 0), True),    # streaming split, 7 row blocks, padded
    ("bf16", (5, 100, 77), (1, 1, 1), (0, 0), False),        # small-M element-wise
    ("bf16", (512, 512, 16384), (0, 0, 0), (0, 0), True),    # tiled split-K (M > 128)
    ("bf16", (512, 512, 4096), (0, 0, 0), (0, 0), True),     # few-tile kernel (the workspace unused)
    ("bf16", (300, 264, 200), (0, 0, 0), (1, 0), False),     # tiled, A stored K x M
    ("bf16", (200, 136, 264), (0, 0, 0), (1, 1), False),     # tiled, both transposed
    ("bf16", (16, 520, 4100), (0, 0, 0), (0, 1), True),      # small M, B stored N x K, split
    ("f32", (2100, 2000, 100), (0, 0, 0), (0, 0), False),    # fp32 tiled copy path
    ("f32", (2100, 2000, 65), (1, 3, 5), (0, 0), False),     # fp32 tiled, unaligned rows
    ("f32", (600, 4100, 300), (4, 8, 12), (0, 0), True),     # fp32 tiled split-K tail, padded
    ("f32", (2100, 2000, 100), (0, 0, 0), (1, 1), False),    # fp32 tiled, both transposed
    ("f32", (300, 264, 100), (0, 0, 0), (0, 0), False),      # fp32 few-tile kernel
    ("f32", (257, 130, 65), (1, 3, 5), (0, 0), False),       # few-tile, unaligned rows
    ("f32", (513, 384, 1000), (4, 8, 12), (0, 0), True),     # few-tile (needs no workspace)
    ("f32", (200, 136, 264), (0, 0, 0), (0, 1), False),      # few-tile, B stored N x K
    ("f32", (136, 200, 264), (0, 0, 0), (1, 0), False),      # few-tile, A stored K x M
]


def _case_id(c):
    return (f"{c[0]}_{'x'.join(map(str, c[1]))}_pad{c[2][0]}_{'NT'[c[3][0]]}{'NT'[c[3][1]]}"
            + ("_ws" if c[4] else ""))


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_scaled_parity(case):
    dtype, (M, N, K), pad, ops, ws = case
    # (alpha, beta, row scales, column scales, bias, activation)
    variants = [(1.0, 0.0, True, True, True, "gelu_tanh"), (0.5, 2.0, True, False, False, "none"),
                (-1.25, 1.0, False, True, True, "relu"), (1.0, 0.0, True, True, False, "none")]
    for rep, (alpha, beta, ru, rv, rb, act) in enumerate(variants):
        seed = 9700 + 13 * M + N + rep
        A = gi.random_matrix(M, K, dtype, seed, dist="n")
        B = gi.random_matrix(K, N, dtype, seed + 1)
        C0 = gi.random_matrix(M, N, dtype, seed + 2) if beta != 0 else None
        bias = gi.random_matrix(1, N, dtype, seed + 3)[0].contiguous() if rb else None
        u = scales(M, seed + 4) if ru else None
        v = scales(N, seed + 5) if rv else None
        note(f"scaled {dtype} M={M} N={N} K={K} ops={ops} pad={pad} ws={ws} alpha={alpha} "
             f"beta={beta} u={ru} v={rv} bias={rb} act={act}")
        C, st = run_scaled(dtype, A, B, C0, u, v, bias, act, alpha, beta, ops, pad, ws)
        assert st == dg.GEMM_OK, dg.gemm_status_string(st)
        R, D = oracle_scaled(dtype, A, B, C0, u, v, bias, act, alpha, beta)
        err = oracle.max_rel_err(to_f64(C), R, D)
        assert err <= tol(dtype), f"variant {rep}: max error ratio {err:.3e}"


@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[6], CASES[13], CASES[15]],
                         ids=_case_id)
def test_unit_scales_are_the_unscaled_epilogue(case):
    dtype, (M, N, K), pad, ops, ws = case
    A = gi.random_matrix(M, K, dtype, 9800, dist="n")
    B = gi.random_matrix(K, N, dtype, 9801)
    C0 = gi.random_matrix(M, N, dtype, 9802)
    bias = gi.random_matrix(1, N, dtype, 9803)[0].contiguous()
    note(f"scaled unit scales {dtype} M={M} N={N} K={K}")
    C1, st1 = run_scaled(dtype, A, B, C0, torch.ones(M), torch.ones(N), bias, "gelu_tanh",
                         0.75, -0.5, ops, pad, ws)
    C2, st2 = run_scaled(dtype, A, B, C0, None, None, bias, "gelu_tanh", 0.75, -0.5, ops, pad, ws,
                         entry="op")
    assert st1 == st2 == dg.GEMM_OK
    iv = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(C1.view(iv), C2.view(iv))


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[5], CASES[6], CASES[8], CASES[13],
                                  CASES[14]], ids=_case_id)
def test_power_of_two_scales_match_prescaled_operands(case):
    """diag(u) (A B) diag(v) = (diag(u) A)(B diag(v)) holds bit for bit when
    the factors are powers of two (no over- or underflow here), since scaling
    by 2^e commutes with every rounding of the sums."""
    dtype, (M, N, K), pad, ops, ws = case
    A = gi.random_matrix(M, K, dtype, 9900, dist="n")
    B = gi.random_matrix(K, N, dtype, 9901)
    u, v = scales(M, 9902, pow2=True), scales(N, 9903, pow2=True)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    As = (A.to(torch.float32) * u[:, None]).to(tdt)
    Bs = (B.to(torch.float32) * v[None, :]).to(tdt)
    note(f"scaled power-of-two {dtype} M={M} N={N} K={K}")
    C1, st1 = run_scaled(dtype, A, B, None, u, v, None, "none", 1.0, 0.0, ops, pad, ws)
    C2, st2 = run_scaled(dtype, As, Bs, None, None, None, None, "none", 1.0, 0.0, ops, pad, ws,
                         entry="op")
    assert st1 == st2 == dg.GEMM_OK
    iv = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(C1.view(iv), C2.view(iv))


def test_misaligned_scales_rejected():
    M, N, K = 64, 64, 64
    a = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(K, N, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    s = torch.ones(N + 1, dtype=torch.float32, device="cuda")
    note("scaled argument checks")
    bad = dg.GEMM_ERR_INVALID_VALUE
    args = (M, N, K, 1.0, a.data_ptr(), K, b.data_ptr(), N, 0.0, c.data_ptr(), N)
    assert dg.gemm_bf16_scaled(0, 0, *args, s.data_ptr() + 2, None) == bad
    assert dg.gemm_bf16_scaled(0, 0, *args, None, s.data_ptr() + 1) == bad
    assert dg.gemm_bf16_scaled(2, 0, *args, None, None) == bad
    torch.cuda.synchronize()
    assert int(c.view(torch.int16).abs().sum()) == 0          # nothing was launched


def test_small_m_streaming_scaled_full_size():
    """16 x 8192 x 8192 (the small-M workload's operands) with per-row and
    per-column scales, bias and GELU through the streaming split, against the
    oracle over every entry."""
    w = gi.WORKLOADS[52]
    d = gi.make(w)
    u, v = scales(w.M, 9950), scales(w.N, 9951)
    bias = gi.random_matrix(1, w.N, "bf16", 9952)[0].contiguous()
    note("scaled bf16 16x8192x8192 full size, streaming split")
    C, st = run_scaled("bf16", d["A"], d["B"], None, u, v, bias, "gelu_tanh", 1.0, 0.0, ws=True)
    assert st == dg.GEMM_OK
    R, D = oracle_scaled("bf16", d["A"], d["B"], None, u, v, bias, "gelu_tanh", 1.0, 0.0)
    assert full_max_err(C, R, D) <= tol("bf16")
