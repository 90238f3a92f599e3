"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Bar (error relative to |alpha| sum_k |a||b| + |beta||c0|, computed by the
oracle): <= 1e-5 for fp32 output, <= 8e-3 for bf16 output (oracle run on the
same bf16 inputs). Exact-arithmetic cases must match bit for bit.
"""
import numpy as np
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, oracle_ref, run, to_f64, tol

pytestmark = pytest.mark.gpu

F32_VARIANTS = [dg.VARIANT_AUTO, dg.VARIANT_MFMA, dg.VARIANT_GENERAL, dg.VARIANT_VALU,
                dg.VARIANT_SMALL]
BF16_VARIANTS = [dg.VARIANT_AUTO, dg.VARIANT_MFMA, dg.VARIANT_GENERAL]

# Shapes that span several tiles in each direction and end in ragged tails
# (the 256x256 bf16 tile, the 128x128 fp32 tile, K slabs of 32/64).
RAGGED = [(1, 1, 1), (3, 5, 7), (17, 33, 65), (129, 257, 63), (300, 200, 100),
          (257, 520, 129), (513, 384, 1000), (640, 136, 72),
          # 16-byte-aligned rows in both dtypes (vector path) with ragged tiles:
          (64, 64, 8), (520, 264, 40), (256, 256, 64), (1000, 1032, 136), (264, 776, 200)]


def check(dtype, M, N, K, alpha, beta, variant, seed, ld_pad=(0, 0, 0), offset=0):
    A = gi.random_matrix(M, K, dtype, seed, dist="n")
    B = gi.random_matrix(K, N, dtype, seed + 1)
    C0 = gi.random_matrix(M, N, dtype, seed + 2) if beta != 0 else None
    note(f"{dtype} M={M} N={N} K={K} alpha={alpha} beta={beta} variant={variant} "
         f"ld_pad={ld_pad} offset={offset}")
    per = 4 if dtype == "f32" else 8
    lds = (max(K, 1) + ld_pad[0], max(N, 1) + ld_pad[1], max(N, 1) + ld_pad[2])
    if variant == dg.VARIANT_MFMA and (offset % per or any(x % per for x in lds)):
        # The 128-bit path must refuse rows that are not 16-byte aligned.
        _, st, _ = run(dtype, A, B, C0, alpha, beta, variant, ld_pad, offset)
        assert st == dg.GEMM_ERR_INVALID_VALUE
        return None
    C, st, _ = run(dtype, A, B, C0, alpha, beta, variant, ld_pad, offset)
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    R, D = oracle_ref(dtype, A, B, C0, alpha, beta)
    err = oracle.max_rel_err(to_f64(C), R, D)
    assert err <= tol(dtype), f"max error ratio {err:.3e}"
    return err


@pytest.mark.parametrize("variant", F32_VARIANTS, ids=lambda v: dg.VARIANT_NAMES[v])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_f32_ragged(shape, variant):
    M, N, K = shape
    check("f32", M, N, K, 0.5, 2.0, variant, seed=100 + M)
    check("f32", M, N, K, 1.0, 0.0, variant, seed=200 + N)


@pytest.mark.parametrize("variant", BF16_VARIANTS, ids=lambda v: dg.VARIANT_NAMES[v])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_bf16_ragged(shape, variant):
    M, N, K = shape
    check("bf16", M, N, K, 0.5, 2.0, variant, seed=300 + M)
    check("bf16", M, N, K, 1.0, 0.0, variant, seed=400 + N)


# (N, K) for the small-M kernels: element-wise rows (N or K not a multiple of
# 8) and 16-byte rows (the copy-ring path) with ragged K tails, K spanning
# more 256-row chunks than the ring holds, and N ending in a partial strip.
SKINNY_NK = [(1, 1), (31, 33), (200, 1100), (1000, 520), (8, 8), (40, 264),
             (264, 2000), (1032, 4104), (96, 1536)]


@pytest.mark.parametrize("M", [1, 2, 5, 15, 16, 17, 31, 32])
@pytest.mark.parametrize("NK", SKINNY_NK, ids=lambda s: "x".join(map(str, s)))
def test_bf16_skinny(M, NK):
    N, K = NK
    check("bf16", M, N, K, 1.5, -0.5, dg.VARIANT_SKINNY, seed=500 + M + N)
    check("bf16", M, N, K, 1.0, 0.0, dg.VARIANT_AUTO, seed=600 + M + K)


# The vector small-M kernel also takes 33..128 rows (64- and 128-row tiles of A).
SKINNY_WIDE_NK = [(264, 2000), (1032, 4104), (96, 1536), (40, 264), (8, 8), (1000, 520)]


@pytest.mark.parametrize("M", [33, 48, 64, 65, 100, 128])
@pytest.mark.parametrize("NK", SKINNY_WIDE_NK, ids=lambda s: "x".join(map(str, s)))
def test_bf16_small_m_up_to_128(M, NK):
    N, K = NK
    check("bf16", M, N, K, 1.5, -0.5, dg.VARIANT_SKINNY, seed=800 + M + N)
    check("bf16", M, N, K, 1.0, 0.0, dg.VARIANT_AUTO, seed=900 + M + K)


@pytest.mark.parametrize("M", [33, 64, 128])
def test_bf16_small_m_wide_unaligned_falls_back(M):
    # Rows that are not 16-byte aligned: the element-wise small-M kernel stops
    # at 32 rows, so these run on the tiled kernels (4-byte copies for even
    # leading dimensions, the unaligned kernel for odd ones).
    assert dg.gemm_plan(2, M, 200, 1100, 1.0, 4096, 1100, 8192, 200, 0.0, 16384, 200,
                        dg.VARIANT_AUTO) == dg.VARIANT_GENERAL
    check("bf16", M, 200, 1100, 1.0, 1.0, dg.VARIANT_AUTO, 950 + M)
    check("bf16", M, 264, 1000, 1.0, 1.0, dg.VARIANT_AUTO, 960 + M, ld_pad=(1, 3, 5))


@pytest.mark.parametrize("M", [7, 16, 29])
def test_bf16_skinny_padded(M):
    # 16-byte padded rows keep the copy-ring path; odd padding takes the other.
    check("bf16", M, 264, 1000, 1.0, 1.0, dg.VARIANT_SKINNY, 720 + M, ld_pad=(8, 16, 24))
    check("bf16", M, 264, 1000, 1.0, 1.0, dg.VARIANT_SKINNY, 730 + M, ld_pad=(1, 3, 5))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_padded_leading_dimensions(dtype):
    # lda/ldb/ldc larger than the row length; multiples of 16 bytes keep the vector path.
    per = 4 if dtype == "f32" else 8
    check(dtype, 300, 264, 136, 1.0, 1.0, dg.VARIANT_MFMA, 700, ld_pad=(per, 2 * per, 3 * per))
    check(dtype, 300, 264, 136, 1.0, 1.0, dg.VARIANT_AUTO, 701, ld_pad=(1, 3, 5))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_base_pointers(dtype):
    # Bases shifted by one element: only the element-wise path may run.
    M, N, K = 200, 136, 264
    assert dg.gemm_plan(4 if dtype == "f32" else 2, M, N, K, 1.0, 4096 + 4, K, 8192, N, 0.0,
                        16384, N, dg.VARIANT_MFMA) in (-1, dg.VARIANT_SKINNY)
    check(dtype, M, N, K, 1.0, 0.5, dg.VARIANT_AUTO, 800, offset=1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", [0, 2, 5])
def test_guard_bands_untouched(dtype, variant):
    """Nothing outside the M x N window of C is written (ldc > N, extra rows)."""
    if variant == dg.VARIANT_SMALL and dtype != "f32":
        pytest.skip("variant does not apply")
    M, N, K = 129, 250, 70
    A = gi.random_matrix(M, K, dtype, 900)
    B = gi.random_matrix(K, N, dtype, 901)
    C0 = gi.random_matrix(M, N, dtype, 902)
    sentinel = -12288.0          # exactly representable in fp32 and bf16
    note(f"guard bands {dtype} variant={variant}")
    C, st, buf = run(dtype, A, B, C0, 1.0, 1.0, variant, ld_pad=(0, 0, 11), c_fill=sentinel)
    assert st == dg.GEMM_OK
    ldc = N + 11
    host = buf.cpu().to(torch.float64).numpy()
    mask = np.ones(host.shape, bool)
    for i in range(M):
        mask[i * ldc:i * ldc + N] = False
    assert np.all(host[mask] == sentinel)
    R, D = oracle_ref(dtype, A, B, C0, 1.0, 1.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5])
def test_beta_zero_ignores_nan_in_c(dtype, variant):
    if (variant in (dg.VARIANT_VALU, dg.VARIANT_SMALL) and dtype != "f32") or \
       (variant == dg.VARIANT_SKINNY and dtype != "bf16"):
        pytest.skip("variant does not apply")
    M = 16 if variant == dg.VARIANT_SKINNY else 130
    A = gi.random_matrix(M, 96, dtype, 1000)
    B = gi.random_matrix(96, 136, dtype, 1001)
    note(f"nan-c {dtype} variant={variant}")
    C, st, _ = run(dtype, A, B, None, 1.0, 0.0, variant)   # C buffer is NaN-filled
    assert st == dg.GEMM_OK
    assert torch.isfinite(C.float()).all()
    R, D = oracle_ref(dtype, A, B, None, 1.0, 0.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= tol(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_k_zero_and_alpha_zero_scale_c(dtype):
    M, N = 70, 90
    C0 = gi.random_matrix(M, N, dtype, 1100)
    for K, alpha, beta in [(0, 1.0, 0.5), (0, 1.0, 0.0), (40, 0.0, -2.0), (40, 0.0, 1.0)]:
        A = gi.random_matrix(M, K, dtype, 1101)
        B = gi.random_matrix(K, N, dtype, 1102)
        note(f"scale {dtype} K={K} alpha={alpha} beta={beta}")
        C, st, _ = run(dtype, A, B, C0, alpha, beta)
        assert st == dg.GEMM_OK
        want = oracle.bf16_round(beta * to_f64(C0)) if dtype == "bf16" else beta * to_f64(C0)
        assert np.array_equal(to_f64(C), want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", [0, 2, 3, 4, 5])
def test_identity_gives_b_bitwise(dtype, variant):
    if (variant in (dg.VARIANT_VALU, dg.VARIANT_SMALL) and dtype != "f32") or \
       (variant == dg.VARIANT_SKINNY and dtype != "bf16"):
        pytest.skip("variant does not apply")
    K = 32 if variant == dg.VARIANT_SKINNY else 300
    N = 520
    A = torch.eye(K, dtype=torch.float32).to(gi.random_matrix(1, 1, dtype, 0).dtype)
    B = gi.random_matrix(K, N, dtype, 1200, dist="n")
    note(f"identity {dtype} variant={variant}")
    C, st, _ = run(dtype, A, B, None, 1.0, 0.0, variant)
    assert st == dg.GEMM_OK
    assert torch.equal(C, B)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", [0, 2, 3, 4, 5])
def test_all_ones_exact(dtype, variant):
    """A = B = 1: every entry is K*alpha + beta*c0 exactly (c0 on a quarter grid)."""
    if (variant in (dg.VARIANT_VALU, dg.VARIANT_SMALL) and dtype != "f32") or \
       (variant == dg.VARIANT_SKINNY and dtype != "bf16"):
        pytest.skip("variant does not apply")
    M = 20 if variant == dg.VARIANT_SKINNY else 260
    N, K, alpha, beta = 136, 1000, 2.0, 0.5
    tdt = gi.random_matrix(1, 1, dtype, 0).dtype
    A = torch.ones(M, K).to(tdt)
    B = torch.ones(K, N).to(tdt)
    C0 = (gi.small_int_matrix(M, N, "f32", 1300) / 4).to(tdt)
    note(f"all-ones {dtype} variant={variant}")
    C, st, _ = run(dtype, A, B, C0, alpha, beta, variant)
    assert st == dg.GEMM_OK
    want = K * alpha + beta * to_f64(C0)
    if dtype == "bf16":
        want = oracle.bf16_round(want)
    assert np.array_equal(to_f64(C), want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", [0, 2, 3, 4, 5])
def test_small_integers_exact(dtype, variant):
    """Integer entries in [-4, 4]: fp32 accumulation is exact in any order, so
    fp32 output equals the oracle and bf16 output equals its rounding."""
    if (variant in (dg.VARIANT_VALU, dg.VARIANT_SMALL) and dtype != "f32") or \
       (variant == dg.VARIANT_SKINNY and dtype != "bf16"):
        pytest.skip("variant does not apply")
    M = 31 if variant == dg.VARIANT_SKINNY else 333
    N, K = 264, 777
    A = gi.small_int_matrix(M, K, dtype, 1400)
    B = gi.small_int_matrix(K, N, dtype, 1401)
    C0 = gi.small_int_matrix(M, N, dtype, 1402)
    note(f"small-int {dtype} variant={variant}")
    C, st, _ = run(dtype, A, B, C0, 1.0, -1.0, variant)
    assert st == dg.GEMM_OK
    R, _ = oracle_ref(dtype, A, B, C0, 1.0, -1.0)
    want = oracle.bf16_round(R) if dtype == "bf16" else R
    assert np.array_equal(to_f64(C), want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_repeatable_bitwise(dtype):
    M, N, K = 520, 392, 610
    A = gi.random_matrix(M, K, dtype, 1500)
    B = gi.random_matrix(K, N, dtype, 1501)
    note(f"repeat {dtype}")
    C1, _, _ = run(dtype, A, B, None, 1.0, 0.0)
    C2, _, _ = run(dtype, A, B, None, 1.0, 0.0)
    assert torch.equal(C1, C2)


def test_non_default_stream():
    s = torch.cuda.Stream()
    A = gi.random_matrix(256, 128, "bf16", 1600)
    B = gi.random_matrix(128, 264, "bf16", 1601)
    note("stream")
    C, st, _ = run("bf16", A, B, None, 1.0, 0.0, stream=s)
    assert st == dg.GEMM_OK
    R, D = oracle_ref("bf16", A, B, None, 1.0, 0.0)
    assert oracle.max_rel_err(to_f64(C), R, D) <= oracle.TOL_BF16


def test_torch_tensor_wrappers():
    A = gi.random_matrix(300, 200, "f32", 1700).cuda()
    B = gi.random_matrix(200, 100, "f32", 1701).cuda()
    C = torch.empty(300, 100, device="cuda")
    note("wrappers")
    dg.matmul_f32(A, B, C)
    torch.cuda.synchronize()
    R, D = oracle_ref("f32", A.cpu(), B.cpu(), None, 1.0, 0.0)
    assert oracle.max_rel_err(to_f64(C.cpu()), R, D) <= oracle.TOL_F32
    with pytest.raises(dg.GemmError):
        dg.matmul_f32(A, B, C, variant=9)
