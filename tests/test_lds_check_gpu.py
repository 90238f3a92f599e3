"""Race checks for the hand-written LDS pipelines (the RTX 3090 SGEMM article,
sections 5.3 and 6.3, checks its double buffer with a race detector; this is
the substitute on gfx950, where the copies are explicit LDS-destined loads
ordered only by the kernels' own waits and barriers).

Two checking builds of the library (dense_gemm_04_amd/build.py) must give the
normal build's results bit for bit, through the C ABI, on every pipeline:
  * poison: each LDS stage is filled with NaN right after the barrier that
    retires it, so a read of a retired stage, or of a stage whose copy has
    not landed, turns into NaN in C;
  * sync: every batch of copies completes before any wave reads LDS again,
    the order one staging buffer would impose.
Cases cover the bf16 tiled kernel (all three tile sizes, several rounds of tiles,
split-K tail, transposed layouts, 16-byte and 4-byte copies), the small-M copy rings (64-column and streaming, split
and not), the element-wise and unaligned kernels, and the fp32 copy path
(16-byte and 4-byte copies: tiles walked, transposed layouts, split-K
tail), its register-staged path and the vector-FMA kernel, at ragged shapes. A second test repeats each
split-K path 100 times and requires identical bits every time.
"""
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, oracle_ref, padded, to_f64, tol

pytestmark = pytest.mark.gpu

_LIBS = {}


def libs():
    if not _LIBS:
        _LIBS["normal"] = dg.load()
        _LIBS["poison"] = dg.load_check_build("poison")
        _LIBS["sync"] = dg.load_check_build("sync")
    return _LIBS


def _store(X, trans, ld_pad, dtype):
    S = X.t().contiguous() if trans else X
    rows, cols = S.shape
    ld = max(cols, 1) + ld_pad
    buf, view = padded(rows, cols, ld, dtype, fill=float("nan"))
    view.copy_(S.cuda())
    return buf, view, ld


def run(lib, dtype, A, B, C0, alpha, beta, ops=(0, 0), pad=(0, 0, 0), ws=False, variant=None):
    """One call on library handle `lib`: gemm_*_op (or gemm_*_ex with a forced
    variant). Returns C on the host."""
    M, K = A.shape
    N = B.shape[1]
    _, a, lda = _store(A, ops[0], pad[0], dtype)
    _, b, ldb = _store(B, ops[1], pad[1], dtype)
    ldc = N + pad[2]
    _, c = padded(M, N, ldc, dtype, fill=float("nan"))
    if C0 is not None:
        c.copy_(C0.cuda())
    size_fn = dg.gemm_f32_workspace_size if dtype == "f32" else dg.gemm_bf16_workspace_size
    nbytes = size_fn(M, N, K) if ws else 0
    wbuf = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    if variant is not None:
        fn = lib.gemm_f32_ex if dtype == "f32" else lib.gemm_bf16_ex
        st = fn(M, N, K, float(alpha), a.data_ptr(), lda, b.data_ptr(), ldb, float(beta),
                c.data_ptr(), ldc, None, variant)
    else:
        fn = lib.gemm_f32_op if dtype == "f32" else lib.gemm_bf16_op
        st = fn(ops[0], ops[1], M, N, K, float(alpha), a.data_ptr(), lda, b.data_ptr(), ldb,
                float(beta), c.data_ptr(), ldc, None, 0, wbuf.data_ptr() if nbytes else None,
                nbytes, None)
    torch.cuda.synchronize()
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    return c.cpu()


# (dtype, (M, N, K), ld_pad, ops, workspace, forced variant)
CASES = [
    ("bf16", (4360, 4104, 200), (0, 0, 0), (0, 0), False, None),   # tiled, 1155 small tiles: three rounds
    ("bf16", (4000, 4000, 200), (0, 0, 0), (0, 0), False, None),   # tiled, 256 large tiles, ragged
    ("bf16", (4000, 4000, 136), (8, 8, 8), (1, 1), False, None),   # large tiles, both transposed, padded
    ("bf16", (520, 520, 4100), (0, 0, 0), (0, 0), True, None),     # tiled split-K tail, ragged K
    ("bf16", (520, 520, 4100), (0, 0, 0), (0, 0), False, None),    # same without a workspace: few-tile kernel
    ("bf16", (2900, 3000, 2100), (2, 2, 2), (1, 0), True, None),   # one round of large tiles as small ones + split tail
    ("bf16", (256, 264, 200), (0, 0, 0), (1, 1), False, None),     # few-tile kernel, both transposed
    ("bf16", (1500, 1528, 136), (8, 0, 0), (0, 0), False, None),   # 64 x 64 tiles (576), 16-byte rows
    ("bf16", (2048, 1500, 300), (0, 0, 0), (0, 0), False, None),   # 192 small tiles, one per CU
    ("bf16", (2048, 2048, 2048), (0, 0, 0), (0, 0), False, None),  # 128 x 128 tiles, K split in the workgroup
    ("bf16", (2000, 2000, 2150), (2, 2, 2), (1, 1), False, None),  # the same, ragged, K tail, 4-byte copies, both transposed
    ("bf16", (2048, 1500, 300), (8, 8, 8), (1, 1), False, None),   # the same, both transposed
    ("bf16", (2048, 1500, 300), (2, 2, 2), (0, 1), False, None),   # the same, 4-byte copies, B stored N x K
    ("bf16", (300, 264, 200), (0, 0, 0), (1, 0), False, None),     # tiled, A stored K x M
    ("bf16", (300, 264, 200), (0, 0, 0), (0, 1), False, None),     # tiled, B stored N x K (M > 128)
    ("bf16", (300, 264, 200), (8, 8, 8), (1, 1), False, None),     # tiled, both, padded rows
    ("bf16", (16, 520, 300), (0, 0, 0), (0, 0), False, None),      # small-M 64-column ring
    ("bf16", (17, 64, 4200), (0, 0, 0), (0, 0), True, None),       # small-M ring, split-K
    ("bf16", (100, 8256, 300), (0, 0, 0), (0, 0), False, None),    # small-M ring, 3 stages (N past one round of 64 x 64 tiles)
    ("bf16", (16, 520, 4100), (0, 0, 0), (0, 1), True, None),      # small-M ring, B stored N x K, split
    ("bf16", (16, 4352, 4100), (0, 0, 0), (0, 0), True, None),     # streaming split
    ("bf16", (33, 4104, 4200), (8, 8, 8), (0, 0), True, None),     # streaming split, padded
    ("bf16", (5, 100, 77), (1, 1, 1), (0, 0), False, None),        # small-M element-wise
    ("bf16", (130, 200, 129), (1, 3, 5), (0, 0), False, None),     # unaligned rows
    ("bf16", (4000, 4000, 200), (2, 2, 2), (0, 0), False, None),   # 4-byte copies, large tiles
    ("bf16", (300, 264, 200), (2, 2, 2), (1, 1), False, None),     # few-tile, 4-byte copies, both transposed
    ("bf16", (300, 264, 129), (2, 2, 2), (1, 0), False, None),     # few-tile, 4-byte copies, A stored K x M
    ("bf16", (300, 264, 129), (1, 3, 2), (0, 1), False, None),     # few-tile, 4-byte copies, B stored N x K
    ("bf16", (520, 520, 4100), (2, 2, 2), (0, 0), False, None),    # few-tile, 4-byte copies, ragged K
    ("bf16", (1500, 1530, 136), (2, 2, 2), (0, 0), False, None),   # 64 x 64 tiles (576), 4-byte copies
    ("bf16", (1500, 1530, 136), (2, 2, 2), (1, 1), False, None),   # the same, both transposed
    ("bf16", (520, 522, 4100), (2, 0, 0), (0, 0), True, None),     # 4-byte copies, split K
    ("f32", (3000, 2900, 72), (0, 0, 0), (0, 0), False, None),     # copy path, 552 tiles walked
    ("f32", (2100, 2000, 100), (0, 0, 0), (1, 0), False, None),    # copy path, A stored K x M
    ("f32", (2100, 2000, 100), (0, 0, 0), (0, 1), False, None),    # copy path, B stored N x K
    ("f32", (2100, 2000, 100), (4, 4, 4), (1, 1), False, None),    # copy path, both, padded
    ("f32", (1100, 1030, 4100), (0, 0, 0), (0, 0), True, None),    # copy path, few tiles split
    ("f32", (600, 4100, 300), (4, 8, 12), (0, 0), True, None),     # split-K tail, padded
    ("f32", (2300, 2290, 2050), (0, 0, 0), (0, 0), True, None),    # fuller last round split: 3 ranges
    ("f32", (2100, 2000, 65), (1, 3, 5), (0, 0), False, None),     # 4-byte copies (unaligned rows)
    ("f32", (2100, 2000, 100), (1, 3, 5), (1, 1), False, None),    # 4-byte copies, both transposed
    ("f32", (2100, 2000, 100), (3, 1, 5), (0, 1), False, None),    # 4-byte copies, B stored N x K
    ("f32", (1100, 1030, 4100), (1, 3, 5), (0, 0), True, None),    # 4-byte copies, split K
    ("f32", (3, 40, 50), (4_199_950, 0, 0), (0, 0), False, 2),     # register-staged (lda past the copy range)
    ("f32", (300, 264, 100), (0, 0, 0), (0, 0), False, 3),         # vector-FMA kernel
]


def _case_id(c):
    return (f"{c[0]}_{'x'.join(map(str, c[1]))}_pad{c[2][0]}_{'NT'[c[3][0]]}{'NT'[c[3][1]]}"
            + ("_ws" if c[4] else "") + {None: "", 2: "_general", 3: "_valu"}[c[5]])


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_checking_builds_match_normal_build(case):
    dtype, (M, N, K), pad, ops, ws, variant = case
    L = libs()
    for rep, (alpha, beta) in enumerate(((1.0, 0.0), (0.5, 2.0))):
        seed = 9400 + 11 * M + N + rep
        A = gi.random_matrix(M, K, dtype, seed, dist="n")
        B = gi.random_matrix(K, N, dtype, seed + 1)
        C0 = gi.random_matrix(M, N, dtype, seed + 2) if beta != 0 else None
        out = {}
        for name, lib in L.items():
            note(f"lds check [{name}] {dtype} M={M} N={N} K={K} ops={ops} pad={pad} ws={ws} "
                 f"variant={variant} alpha={alpha} beta={beta}")
            out[name] = run(lib, dtype, A, B, C0, alpha, beta, ops, pad, ws, variant)
        iv = torch.int32 if dtype == "f32" else torch.int16
        for name in ("poison", "sync"):
            assert torch.equal(out[name].view(iv), out["normal"].view(iv)), \
                f"{name} build differs from the normal build (call {rep})"
        R, D = oracle_ref(dtype, A, B, C0, alpha, beta)
        err = oracle.max_rel_err(to_f64(out["normal"]), R, D)
        assert err <= tol(dtype), f"call {rep}: max error ratio {err:.3e}"


# Split-K paths: repeated calls on one workspace must give identical bits
# every time (fixed-order sums; counters left at zero by every call).
REPEAT = [("bf16", (16, 8192, 8192)), ("bf16", (16, 1032, 4104)), ("bf16", (512, 512, 16384)),
          ("f32", (2300, 2290, 2050)), ("f32", (1024, 1024, 4096))]


@pytest.mark.parametrize("case", REPEAT, ids=lambda c: f"{c[0]}_{'x'.join(map(str, c[1]))}")
def test_split_k_repeats_bitwise(case):
    dtype, (M, N, K) = case
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    A = gi.random_matrix(M, K, dtype, 9600, dist="n").cuda()
    B = gi.random_matrix(K, N, dtype, 9601).cuda()
    size_fn = dg.gemm_f32_workspace_size if dtype == "f32" else dg.gemm_bf16_workspace_size
    ws_fn = dg.gemm_f32_ws if dtype == "f32" else dg.gemm_bf16_ws
    nbytes = size_fn(M, N, K)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    C = torch.empty(M, N, dtype=tdt, device="cuda")
    ref = None
    note(f"split-K repeat {dtype} M={M} N={N} K={K}: 100 calls")
    for call in range(100):
        C.fill_(float("nan"))
        st = ws_fn(M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0, C.data_ptr(), N,
                   ws.data_ptr(), nbytes, 0)
        assert st == dg.GEMM_OK
        if ref is None:
            torch.cuda.synchronize()
            ref = C.clone()
            assert bool(torch.isfinite(ref.float()).all())
        elif not torch.equal(C, ref):
            raise AssertionError(f"call {call} differs from call 0")
    torch.cuda.synchronize()
