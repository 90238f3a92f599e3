"""The six workloads at full size, in the launch configuration the benchmark
times (default kernel choice, packed leading dimensions), checked against the
oracle over EVERY entry of C: the RTX 3090 SGEMM article (section 2.2) keeps
the plain kernel as the baseline that each optimised version is compared
against in full. The oracle runs once per workload (all host cores, tens of
seconds at most) and is shared by the calls that compute the same C: the
plain call and the split-K call through a workspace."""
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
from gpu_util import full_max_err, note, tol, workload_reference

pytestmark = pytest.mark.gpu


def _operands(w):
    inp = gi.make(w)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    A = inp["A"].cuda()
    B = inp["B"].cuda()
    # With beta == 0 C starts as NaN: C must be write-only then.
    C = inp["C0"].cuda() if inp["C0"] is not None else torch.full((w.M, w.N), float("nan"),
                                                                    dtype=tdt, device="cuda")
    return A, B, C


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 51, 52])
def test_workload_full_size(wid):
    w = gi.WORKLOADS[wid]
    note(f"workload {w.name}")
    A, B, C = _operands(w)
    fn = dg.gemm_f32 if w.dtype == "f32" else dg.gemm_bf16
    st = fn(w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, B.data_ptr(), w.N, w.beta,
            C.data_ptr(), w.N, int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    R, D = workload_reference(wid)
    err = full_max_err(C, R, D)
    note(f"workload {w.name}: all {w.M}x{w.N} entries, max error ratio {err:.3e}")
    assert err <= tol(w.dtype)


def test_workload_small_m_split_k():
    # The small-M workload through gemm_bf16_ws, as the benchmark times it;
    # two calls in a row on one workspace (the second relies on the counters
    # the first left at zero).
    w = gi.WORKLOADS[52]
    note(f"workload {w.name} via gemm_bf16_ws")
    A, B, _ = _operands(w)
    nbytes = dg.gemm_bf16_workspace_size(w.M, w.N, w.K)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    R, D = workload_reference(52)
    for call in range(2):
        C = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda")
        st = dg.gemm_bf16_ws(w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, B.data_ptr(), w.N,
                             w.beta, C.data_ptr(), w.N, ws.data_ptr(), nbytes,
                             int(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert st == dg.GEMM_OK, dg.gemm_status_string(st)
        err = full_max_err(C, R, D)
        note(f"call {call}: all {w.M}x{w.N} entries, max error ratio {err:.3e}")
        assert err <= tol(w.dtype)


def test_workload_edge_tiled_kernel_alone():
    # 4095 x 4097 x 1023 on the tiled kernel alone (gemm_f32_ex, forced
    # element-wise variant): 1056 tiles in three rounds, the ragged last tile
    # column (one column of C) included. The automatic choice puts that
    # column on the few-tile kernel instead (test_workload_full_size[51]).
    w = gi.WORKLOADS[51]
    note(f"workload {w.name} on the tiled kernel alone")
    A, B, C = _operands(w)
    st = dg.gemm_f32_ex(w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, B.data_ptr(), w.N, w.beta,
                        C.data_ptr(), w.N, int(torch.cuda.current_stream().cuda_stream),
                        dg.VARIANT_GENERAL)
    torch.cuda.synchronize()
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    R, D = workload_reference(51)
    err = full_max_err(C, R, D)
    note(f"all {w.M}x{w.N} entries, max error ratio {err:.3e}")
    assert err <= tol(w.dtype)


def test_workload_edge_workspace_call_is_the_plain_call():
    # gemm_f32_ws needs no workspace for 4095 x 4097 x 1023 (the partly full
    # last round goes to the few-tile kernel as a strip, which beats splitting
    # it) and gives the plain call's bits.
    w = gi.WORKLOADS[51]
    assert dg.gemm_f32_workspace_size(w.M, w.N, w.K) == 0
    A, B, C = _operands(w)
    C2 = C.clone()
    h = int(torch.cuda.current_stream().cuda_stream)
    note(f"workload {w.name} via gemm_f32 and gemm_f32_ws")
    st = dg.gemm_f32(w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, B.data_ptr(), w.N, w.beta,
                     C.data_ptr(), w.N, h)
    st2 = dg.gemm_f32_ws(w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, B.data_ptr(), w.N, w.beta,
                         C2.data_ptr(), w.N, None, 0, h)
    torch.cuda.synchronize()
    assert st == st2 == dg.GEMM_OK
    assert torch.equal(C.view(torch.int32), C2.view(torch.int32))
