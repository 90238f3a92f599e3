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


def test_workload_edge_split_k():
    # 4095 x 4097 x 1023 through gemm_f32_ws: 1024 whole tiles, then the last
    # 32 tiles (the ragged ones among them) split into 8 K ranges each.
    w = gi.WORKLOADS[51]
    note(f"workload {w.name} via gemm_f32_ws")
    A, B, C = _operands(w)
    nbytes = dg.gemm_f32_workspace_size(w.M, w.N, w.K)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    st = dg.gemm_f32_ws(w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, B.data_ptr(), w.N, w.beta,
                        C.data_ptr(), w.N, ws.data_ptr(), nbytes,
                        int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    R, D = workload_reference(51)
    err = full_max_err(C, R, D)
    note(f"all {w.M}x{w.N} entries, max error ratio {err:.3e}")
    assert err <= tol(w.dtype)
