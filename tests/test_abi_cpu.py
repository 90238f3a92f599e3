"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, validates its arguments before touching HIP, and plans the kernel
family from shape and alignment alone."""
import ctypes
import os
import re

import pytest

import dense_gemm_04_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dg.LIB_PATH):
        from dense_gemm_04_amd import build
        build.build()
    return dg.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert header_functions() == sorted(dg.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


@pytest.mark.parametrize("check", ["poison", "sync"])
def test_checking_builds_load_and_export_every_symbol(check):
    from dense_gemm_04_amd import build
    if not os.path.exists(build.lib_path(check)):
        build.build(check=check)
    chk = dg.load_check_build(check)
    for name in header_functions():
        assert hasattr(chk, name), name
    # Validation is the same code in every build.
    assert chk.gemm_f32(-1, 4, 4, 1.0, 0x10000, 4, 0x20000, 4, 0.0, 0x30000, 4,
                        None) == dg.GEMM_ERR_INVALID_VALUE


def test_status_strings(lib):
    assert dg.gemm_status_string(0) == "success"
    assert dg.gemm_status_string(1) == "invalid argument"
    assert "gfx950" in dg.gemm_status_string(2)
    assert dg.gemm_status_string(3) == "kernel launch failed"
    assert "scratch" in dg.gemm_status_string(4)
    assert dg.gemm_status_string(99) == "unknown status"


# Fake, suitably aligned device addresses: planning only inspects alignment.
A, B, C = 0x10000, 0x20000, 0x30000


def plan(esz=4, M=64, N=64, K=64, alpha=1.0, a=A, lda=None, b=B, ldb=None, beta=0.0, c=C,
         ldc=None, variant=0):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return dg.gemm_plan(esz, M, N, K, alpha, a, lda, b, ldb, beta, c, ldc, variant)


def test_plan_rejects_invalid_arguments(lib):
    assert plan(M=-1) == -1
    assert plan(N=-1) == -1
    assert plan(K=-1) == -1
    assert plan(lda=63) == -1                 # lda < K
    assert plan(ldb=63) == -1                 # ldb < N
    assert plan(ldc=63) == -1                 # ldc < N
    assert plan(K=0, lda=0) == -1             # lda < max(1, K)
    assert plan(a=None) == -1
    assert plan(b=None) == -1
    assert plan(c=None) == -1
    assert plan(a=A + 2) == -1                # fp32 pointer not 4-byte aligned
    assert plan(esz=2, a=A + 1) == -1         # bf16 pointer not 2-byte aligned
    assert plan(esz=3) == -1
    assert plan(variant=9) == -1
    assert plan(M=1 << 31) == -1
    # Extents of 2^60 bytes or more: leading dimensions that would overflow offsets.
    assert plan(M=1 << 20, lda=1 << 40) == -1                   # A spans ~2^62 bytes
    assert plan(K=1 << 20, lda=1 << 20, ldb=1 << 40) == -1      # B
    assert plan(M=1 << 20, ldc=1 << 40) == -1                   # C
    assert plan(M=1 << 20, lda=1 << 30) == dg.VARIANT_MFMA       # 2^52 bytes: fine


def test_plan_quick_paths(lib):
    # Nothing to do: M or N empty, or C <- 1 * C.
    assert plan(M=0, c=None) == dg.VARIANT_AUTO
    assert plan(N=0, c=None, ldb=1, ldc=1) == dg.VARIANT_AUTO
    assert plan(K=0, lda=1, a=None, b=None, beta=1.0, c=None) == dg.VARIANT_AUTO
    # alpha == 0 or K == 0: A and B may be NULL, C is scaled.
    assert plan(alpha=0.0, a=None, b=None, beta=0.5) == dg.VARIANT_AUTO
    assert plan(K=0, lda=1, a=None, b=None, beta=0.0) == dg.VARIANT_AUTO
    assert plan(K=0, lda=1, a=None, b=None, beta=0.0, c=None) == -1


def test_plan_chooses_family(lib):
    big = dict(M=4096, N=4096, K=4096)
    assert plan(**big) == dg.VARIANT_MFMA
    # fp32 with few 128 x 128 tiles: the few-tile kernel, whatever the alignment.
    assert plan() == dg.VARIANT_SMALL                          # 64^3
    assert plan(M=256, N=256, K=256) == dg.VARIANT_SMALL
    assert plan(M=1536, N=1536, K=1024) == dg.VARIANT_SMALL    # 144 tiles: 32 x 32 tiles win
    assert plan(M=1792, N=1792, K=1024) == dg.VARIANT_MFMA     # 196 tiles: one tiled round wins
    assert plan(M=2048, N=2048, K=2048) == dg.VARIANT_MFMA
    assert plan(a=A + 4) == dg.VARIANT_SMALL
    assert plan(lda=66) == dg.VARIANT_SMALL
    assert plan(variant=dg.VARIANT_SMALL, **big) == dg.VARIANT_SMALL
    assert plan(esz=2, variant=dg.VARIANT_SMALL) == -1
    assert plan(variant=dg.VARIANT_MFMA) == dg.VARIANT_MFMA
    assert plan(esz=2, M=16) == dg.VARIANT_SKINNY             # bf16, M <= 128 (16-byte rows)
    assert plan(esz=2, M=32) == dg.VARIANT_SKINNY
    # 33 .. 64 rows: the tiled kernels when N x K <= 2^25 (plain calls), else
    # the small-M kernel.
    assert plan(esz=2, M=33) == dg.VARIANT_MFMA
    assert plan(esz=2, M=33, N=8192, K=8192) == dg.VARIANT_SKINNY
    assert plan(esz=2, M=64, N=8192, K=8192) == dg.VARIANT_SKINNY
    # 65 .. 128 rows: the tiled kernels when their 64 x 64 tiles fit one round
    # (at most 256; here 2), else the small-M kernel (2 x 129 tiles).
    assert plan(esz=2, M=128) == dg.VARIANT_MFMA
    assert plan(esz=2, M=65, N=8192) == dg.VARIANT_MFMA
    assert plan(esz=2, M=128, N=8256) == dg.VARIANT_SKINNY
    assert plan(esz=2, M=129) == dg.VARIANT_MFMA
    assert plan(esz=2, M=32, lda=66) == dg.VARIANT_SKINNY      # unaligned: element-wise, M <= 32
    assert plan(esz=2, M=33, lda=66) == dg.VARIANT_GENERAL
    assert plan(M=4095, N=4097, K=1023) == dg.VARIANT_GENERAL  # ld not a multiple of 4 floats
    assert plan(a=A + 4, **big) == dg.VARIANT_GENERAL          # base not 16-byte aligned
    assert plan(M=4096, N=4096, K=64, lda=68) == dg.VARIANT_MFMA
    assert plan(M=4096, N=4096, K=64, lda=66) == dg.VARIANT_GENERAL
    assert plan(variant=dg.VARIANT_VALU) == dg.VARIANT_VALU
    assert plan(esz=2, variant=dg.VARIANT_VALU) == -1
    assert plan(M=16, variant=dg.VARIANT_SKINNY) == -1
    assert plan(esz=2, M=129, variant=dg.VARIANT_SKINNY) == -1
    assert plan(esz=2, M=33, lda=66, variant=dg.VARIANT_SKINNY) == -1
    assert plan(a=A + 4, variant=dg.VARIANT_MFMA) == -1
    assert plan(variant=dg.VARIANT_GENERAL) == dg.VARIANT_GENERAL


def test_invalid_calls_return_before_any_hip_call(lib):
    # These return from validation; no device is touched.
    assert dg.gemm_f32(-1, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, 0) == dg.GEMM_ERR_INVALID_VALUE
    assert dg.gemm_bf16(4, 4, 4, 1.0, A, 3, B, 4, 0.0, C, 4, 0) == dg.GEMM_ERR_INVALID_VALUE
    assert dg.gemm_f32_ex(4, 4, 4, 1.0, A, 4, B, 4, 0.0, C, 4, 0, 7) == dg.GEMM_ERR_INVALID_VALUE
    assert dg.gemm_bf16_ex(64, 64, 64, 1.0, A, 64, B, 64, 0.0, C, 64, 0,
                           dg.VARIANT_VALU) == dg.GEMM_ERR_INVALID_VALUE
    # Empty problems succeed without touching the device either.
    assert dg.gemm_f32(0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, 0) == dg.GEMM_OK


def test_noalloc_checks_before_any_hip_call(lib):
    # Invalid arguments, then shapes whose split-K workspace exceeds the static
    # scratch, are refused on the host; a shape that fits goes on to the
    # device check (no GPU here).
    noalloc = dg.gemm_bf16_ws_noalloc
    assert noalloc(4, 4, 4, 1.0, A, 3, B, 4, 0.0, C, 4, 0) == dg.GEMM_ERR_INVALID_VALUE
    assert noalloc(4, 4, 4, 1.0, A + 1, 4, B, 4, 0.0, C, 4, 0) == dg.GEMM_ERR_INVALID_VALUE
    assert noalloc(0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, 0) == dg.GEMM_OK
    # 128 x 8256 x 8192: 33 strips x 8 phases of 128 x 256 fp32 partials.
    assert dg.gemm_bf16_workspace_size(128, 8256, 8192) > dg.NOALLOC_SCRATCH_BYTES
    assert noalloc(128, 8256, 8192, 1.0, A, 8192, B, 8256, 0.0, C, 8256,
                   0) == dg.GEMM_ERR_SCRATCH_LIMIT
    import torch
    if not torch.cuda.is_available():
        assert dg.gemm_bf16_workspace_size(128, 8192, 8192) <= dg.NOALLOC_SCRATCH_BYTES
        assert noalloc(128, 8192, 8192, 1.0, A, 8192, B, 8192, 0.0, C, 8192,
                       0) == dg.GEMM_ERR_UNSUPPORTED_DEVICE
        assert noalloc(16, 64, 64, 1.0, A, 64, B, 64, 0.0, C, 64,
                       0) == dg.GEMM_ERR_UNSUPPORTED_DEVICE


def test_valid_call_without_gpu_reports_unsupported_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = dg.gemm_f32(64, 64, 64, 1.0, A, 64, B, 64, 0.0, C, 64, 0)
    assert st == dg.GEMM_ERR_UNSUPPORTED_DEVICE


def test_oracle_and_library_share_nothing():
    """The oracle and the HIP sources must not include, import or link each other."""
    csrc = os.path.join(ROOT, "dense_gemm_04_amd")
    for dirpath, _, files in os.walk(csrc):
        for f in files:
            if f.endswith((".hip", ".hpp", ".py", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".c", ".py")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "dense_gemm_04_amd" not in text and "gemm.h" not in text, f


def test_workspace_size(lib):
    # 16 x 8192 x 8192 runs on the streaming kernel: 32 strips of 256 columns,
    # K interleaved over 8 phases (256 workgroups): a 256-byte counter block,
    # then 32 x 8 fp32 partial tiles of 16 x 256.
    assert dg.gemm_bf16_workspace_size(16, 8192, 8192) == 256 + 32 * 8 * 16 * 256 * 4
    # 17..32 rows use 32-row tiles, 33..64 64-row and 65..128 128-row tiles.
    assert dg.gemm_bf16_workspace_size(32, 8192, 8192) == 256 + 32 * 8 * 32 * 256 * 4
    assert dg.gemm_bf16_workspace_size(33, 8192, 8192) == 256 + 32 * 8 * 64 * 256 * 4
    assert dg.gemm_bf16_workspace_size(128, 16384, 8192) == 256 + 64 * 4 * 128 * 256 * 4
    # 65 .. 128 rows whose 64 x 64 tiles fit one round run on the tiled
    # kernels (the few-tile kernel here: no workspace; 128 x 4352: the split
    # of 34 tiles of 128 x 128 into 7 K ranges).
    assert dg.gemm_bf16_workspace_size(128, 8192, 8192) == 0
    assert dg.gemm_bf16_workspace_size(128, 4352, 8192) == 256 + 34 * 7 * 128 * 128 * 4
    # 64 strips of 256 columns: 4 phases fill the chip.
    assert dg.gemm_bf16_workspace_size(16, 16384, 8192) == 256 + 64 * 4 * 16 * 256 * 4
    # 16 strips (N = 3841) would take 16 phases, the most; K = 4104 has 129
    # blocks of 32 rows.
    assert dg.gemm_bf16_workspace_size(16, 3841, 4104) == 256 + 16 * 16 * 16 * 256 * 4
    # The small-M splits need K >= 4096: shorter K runs unsplit, faster.
    assert dg.gemm_bf16_workspace_size(16, 3841, 700) == 0
    assert dg.gemm_bf16_workspace_size(7, 4104, 260) == 0
    assert dg.gemm_bf16_workspace_size(16, 8192, 4095) == 0
    assert dg.gemm_bf16_workspace_size(16, 8192, 4096) > 0
    assert dg.gemm_bf16_workspace_size(7, 4104, 40) == 0
    # N = 3840 is 15 strips: the 64-column kernel's split (60 strips of 64
    # columns; K = 8192 has 64 chunks of 128: 5 segments of 13 chunks).
    assert dg.gemm_bf16_workspace_size(16, 3840, 8192) == 256 + 5 * 60 * 16 * 64 * 4
    # M > 128 is sized for the tiled kernel instead (see the next test); no
    # small-M split when strips already fill the GPU, one K chunk, empty or
    # invalid sizes.
    assert dg.gemm_bf16_workspace_size(129, 8192, 8192) == 512 + 128 * 2 * 128 * 128 * 4
    # 4352 x 4096 would take 128 x 128 tiles whose last round (64 of 1088) a
    # workspace could split; it runs one round of 256 x 256 tiles and a
    # 256-row strip on the few-tile kernel instead, with no workspace.
    assert dg.gemm_bf16_workspace_size(4352, 4096, 4096) == 0
    # 3072^2 takes one round of 144 256 x 256 tiles; with a workspace it runs
    # 576 tiles of 128 x 128 instead: 512 in one round, the last 64 cut into
    # 3 K ranges of 16 slabs (at K = 3072). 4000^2 (256 large tiles, a full
    # round) needs none.
    assert dg.gemm_bf16_workspace_size(3072, 3072, 3072) == 256 + 64 * 3 * 128 * 128 * 4
    assert dg.gemm_bf16_workspace_size(2900, 3000, 2100) == 256 + 40 * 2 * 128 * 128 * 4
    assert dg.gemm_bf16_workspace_size(4000, 4000, 2048) == 0
    assert dg.gemm_bf16_workspace_size(16, 2048, 8192) > 0
    assert dg.gemm_bf16_workspace_size(16, 16384, 128) == 0
    assert dg.gemm_bf16_workspace_size(16, 64, 128) == 0
    assert dg.gemm_bf16_workspace_size(0, 64, 1024) == 0
    assert dg.gemm_bf16_workspace_size(16, 0, 1024) == 0
    assert dg.gemm_bf16_workspace_size(16, 64, 0) == 0
    assert dg.gemm_bf16_workspace_size(-1, 64, 1024) == 0
    # Segments are capped at 64 (N = 64, K = 2^20: 64 segments of 128 chunks).
    assert dg.gemm_bf16_workspace_size(16, 64, 1 << 20) == 256 + 64 * 1 * 16 * 64 * 4
    # K = 300 (3 chunks) would give 3 segments, but below K = 4096 nothing splits.
    assert dg.gemm_bf16_workspace_size(16, 64, 300) == 0
    # 17 strips want 16 segments; K = 4104 has 33 chunks: 11 segments of 3.
    assert dg.gemm_bf16_workspace_size(16, 1032, 4104) == 256 + 11 * 17 * 16 * 64 * 4


def test_tiled_workspace_size(lib):
    # M > 128: the bf16 tiled kernel's split, for 128 x 128 tiles that leave
    # most CUs idle: fewer than half as many tiles as CUs (256), cut into up to
    # 8 K ranges of at least 16 slabs of 64, each with a 64 KB fp32 partial.
    tile = 128 * 128 * 4
    # 129 x 8192 x 8192: 128 tiles, 128 slabs -> 2 ranges.
    assert dg.gemm_bf16_workspace_size(129, 8192, 8192) == 512 + 128 * 2 * tile
    # 512^2 x 16384: 16 tiles, 256 slabs -> 8 ranges; 640 x 1000 x 8192: 40
    # tiles -> 6 ranges (240 workgroups, more than its 160 tiles of 64 x 64).
    assert dg.gemm_bf16_workspace_size(512, 512, 16384) == 256 + 16 * 8 * tile
    assert dg.gemm_bf16_workspace_size(640, 1000, 8192) == 256 + 40 * 6 * tile
    # The few-tile kernel instead, when its 64 x 64 tiles fit one round and
    # are at least as many as the split's workgroups: 1024^2 x 4096 (256
    # against 64 x 4), 512^2 x 4096 (64 against 16 x 4), 1024^2 x 2048.
    assert dg.gemm_bf16_workspace_size(1024, 1024, 4096) == 0
    assert dg.gemm_bf16_workspace_size(512, 512, 4096) == 0
    assert dg.gemm_bf16_workspace_size(1024, 1024, 2048) == 0
    # 129 x 1000 x 8200: 16 tiles, 129 slabs -> 8 ranges of 17 (the last 10).
    assert dg.gemm_bf16_workspace_size(129, 1000, 8200) == 256 + 16 * 8 * tile
    # One partly full round of 256 x 256 tiles (3072^2 and 3000^2: 144) runs
    # 576 small tiles with a workspace, the last 64 split: 3072^2 x 8192 in 4
    # ranges of 32 slabs, 3000^3 (47 slabs) in 2 of 24.
    assert dg.gemm_bf16_workspace_size(3072, 3072, 8192) == 256 + 64 * 4 * tile
    assert dg.gemm_bf16_workspace_size(3000, 3000, 3000) == 256 + 64 * 2 * tile
    # No split: one tile per CU already (512 x 8192 and 2048^2: 256 small
    # tiles), a full round of 256 x 256 tiles (4096^2), fewer than 32 slabs.
    assert dg.gemm_bf16_workspace_size(512, 8192, 8192) == 0
    assert dg.gemm_bf16_workspace_size(2048, 2048, 2048) == 0
    assert dg.gemm_bf16_workspace_size(4096, 4096, 4096) == 0
    assert dg.gemm_bf16_workspace_size(1024, 1024, 1024) == 0
    assert dg.gemm_bf16_workspace_size(300, 520, 1984) == 0


def test_workspace_validation(lib):
    # Rejected before any HIP call, so these run without a GPU.
    args = (16, 8192, 8192, 1.0, A, 8192, B, 8192, 0.0, C, 8192)
    need = dg.gemm_bf16_workspace_size(16, 8192, 8192)
    ws = 0x400000
    assert dg.gemm_bf16_ws(*args, None, 64, 0) == dg.GEMM_ERR_INVALID_VALUE       # NULL, size > 0
    assert dg.gemm_bf16_ws(*args, ws + 128, need, 0) == dg.GEMM_ERR_INVALID_VALUE  # misaligned
    assert dg.gemm_bf16_ws(*args, ws, need - 1, 0) == dg.GEMM_ERR_INVALID_VALUE    # too small
    bad = (16, 64, 64, 1.0, A, 63, B, 64, 0.0, C, 64)                                # lda < K
    assert dg.gemm_bf16_ws(*bad, ws, 1 << 20, 0) == dg.GEMM_ERR_INVALID_VALUE


def test_f32_workspace_size(lib):
    # 4095 x 4097: 32 x 33 = 1056 tiles of 128 x 128 on 512 slots (256 compute
    # units, 2 workgroups each): 1024 in two full rounds and 32 left, which are
    # C's last column; the few-tile kernel takes that column, so no workspace.
    assert dg.gemm_f32_workspace_size(4095, 4097, 1023) == 0
    # A last round more than half full: 2304^2 has 18 x 18 = 324 tiles on 512
    # slots; K = 2048 is 64 slabs, and 3 ranges give 2 rounds of 22 slabs +
    # 3 x 0.25 = 44.75 against 64 unsplit.
    assert dg.gemm_f32_workspace_size(2304, 2304, 2048) == 1536 + 324 * 3 * 128 * 128 * 4
    # Few tiles with long K: 1024^2 is 64 tiles (64 x 4096 = 2^18 tile-k), cut
    # into 8 ranges of 16 slabs.
    assert dg.gemm_f32_workspace_size(1024, 1024, 4096) == 256 + 64 * 8 * 128 * 128 * 4
    # Few tiles with fewer tile-k go to the few-tile kernel, which needs no
    # workspace: 300 x 200 (6 tiles), 1024^3 (64 tiles x 1024), 256^3.
    assert dg.gemm_f32_workspace_size(300, 200, 100) == 0
    assert dg.gemm_f32_workspace_size(1024, 1024, 1024) == 0
    assert dg.gemm_f32_workspace_size(256, 256, 256) == 0
    # 257 .. 511 tiles: one round, two tiles on some CUs. 2048 x 2560 (320
    # tiles) puts its last 4 tile columns (64 tiles) on the few-tile kernel and
    # runs one tile per CU on the rest, which beats the split given a
    # workspace too, so it needs none; so does 2048 x 2304 (288 tiles). For
    # 2304^2 (above) the split wins when a workspace is given.
    assert dg.gemm_f32_workspace_size(128 * 16, 128 * 20, 4096) == 0
    assert dg.gemm_f32_workspace_size(2048, 2304, 4096) == 0
    # No split: whole rounds (4096^2 is 1024 tiles), a fuller last round whose
    # ranges would be shorter than 16 slabs (3072 x 2048 x 1024: 384 tiles of
    # 32 slabs), K of one slab, empty or invalid sizes.
    assert dg.gemm_f32_workspace_size(4096, 4096, 4096) == 0
    assert dg.gemm_f32_workspace_size(3072, 2048, 1024) == 0
    assert dg.gemm_f32_workspace_size(300, 200, 32) == 0
    assert dg.gemm_f32_workspace_size(0, 200, 100) == 0
    assert dg.gemm_f32_workspace_size(-1, 200, 100) == 0


def test_f32_workspace_validation(lib):
    args = (1024, 1024, 4096, 1.0, A, 4096, B, 1024, 0.0, C, 1024)
    need = dg.gemm_f32_workspace_size(1024, 1024, 4096)
    assert need > 0
    ws = 0x400000
    assert dg.gemm_f32_ws(*args, None, 64, 0) == dg.GEMM_ERR_INVALID_VALUE
    assert dg.gemm_f32_ws(*args, ws + 64, need, 0) == dg.GEMM_ERR_INVALID_VALUE
    assert dg.gemm_f32_ws(*args, ws, need - 1, 0) == dg.GEMM_ERR_INVALID_VALUE


def test_bias_act_validation(lib):
    """Bias alignment, activation code and workspace are checked before any HIP call."""
    f32 = (300, 200, 100, 1.0, A, 100, B, 200, 0.0, C, 200)
    bf = (300, 200, 100, 1.0, A, 100, B, 200, 0.0, C, 200)
    bias = 0x500000
    bad = dg.GEMM_ERR_INVALID_VALUE
    assert dg.gemm_f32_bias_act(*f32, bias, 3, None, 0, 0) == bad
    assert dg.gemm_f32_bias_act(*f32, bias, -1, None, 0, 0) == bad
    assert dg.gemm_f32_bias_act(*f32, bias + 2, dg.ACT_RELU, None, 0, 0) == bad
    assert dg.gemm_bf16_bias_act(*bf, bias + 1, dg.ACT_RELU, None, 0, 0) == bad
    big = (1024, 1024, 4096, 1.0, A, 4096, B, 1024, 0.0, C, 1024)
    need = dg.gemm_f32_workspace_size(1024, 1024, 4096)
    assert need > 0
    assert dg.gemm_f32_bias_act(*big, bias, dg.ACT_RELU, 0x400000, need - 1, 0) == bad
    assert dg.gemm_f32_bias_act(*f32, bias, dg.ACT_RELU, None, 64, 0) == bad
    # Product-free calls: with no bias and beta == 1 nothing runs; a bias needs C.
    assert dg.gemm_f32_bias_act(4, 4, 0, 1.0, None, 4, None, 4, 1.0, None, 4, None,
                                dg.ACT_GELU_TANH, None, 0, 0) == dg.GEMM_OK
    assert dg.gemm_f32_bias_act(4, 4, 0, 1.0, None, 4, None, 4, 1.0, None, 4, bias,
                                dg.ACT_GELU_TANH, None, 0, 0) == bad
    assert dg.gemm_bf16_bias_act(0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, None,
                                 dg.ACT_RELU, None, 0, 0) == dg.GEMM_OK


def test_bias_act_without_gpu_reports_unsupported_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = dg.gemm_bf16_bias_act(64, 64, 64, 1.0, A, 64, B, 64, 0.0, C, 64, 0x500000,
                               dg.ACT_GELU_TANH, None, 0, 0)
    assert st == dg.GEMM_ERR_UNSUPPORTED_DEVICE


def test_op_validation(lib):
    """Operation codes and the transposed leading-dimension rules are checked
    before any HIP call."""
    bad = dg.GEMM_ERR_INVALID_VALUE
    M, N, K = 300, 200, 100
    # op(A) = A^T: A stored K x M needs lda >= M; op(B) = B^T: B stored N x K needs ldb >= K.
    assert dg.gemm_f32_op(1, 0, M, N, K, 1.0, A, M - 1, B, N, 0.0, C, N) == bad
    assert dg.gemm_f32_op(0, 1, M, N, K, 1.0, A, K, B, K - 1, 0.0, C, N) == bad
    assert dg.gemm_bf16_op(3, 0, M, N, K, 1.0, A, K, B, N, 0.0, C, N) == bad
    assert dg.gemm_bf16_op(0, -1, M, N, K, 1.0, A, K, B, N, 0.0, C, N) == bad
    # A K x M storage may have lda < K (e.g. a wide, short A^T).
    st = dg.gemm_f32_op(1, 1, 8, 4, 1000, 1.0, A, 8, B, 1000, 0.0, C, 4)
    assert st in (dg.GEMM_OK, dg.GEMM_ERR_UNSUPPORTED_DEVICE)
    assert dg.gemm_f32_op(1, 1, 8, 4, 1000, 1.0, A, 7, B, 1000, 0.0, C, 4) == bad
    assert dg.gemm_bf16_op(1, 1, 0, 4, 4, 1.0, None, 1, None, 4, 0.0, None, 4) == dg.GEMM_OK


def test_op_without_gpu_reports_unsupported_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    for opa, opb in ((0, 0), (0, 1), (1, 0), (1, 1)):
        st = dg.gemm_bf16_op(opa, opb, 64, 64, 64, 1.0, A, 64, B, 64, 0.0, C, 64)
        assert st == dg.GEMM_ERR_UNSUPPORTED_DEVICE
