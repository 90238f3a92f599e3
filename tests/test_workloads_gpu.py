"""The six workloads at full size, in the launch configuration the benchmark
times (default kernel choice, packed leading dimensions), checked against the
oracle on sampled entries that cover every 128-row and 128-column tile band
(first, last and one random row/column of each), plus every entry finite."""
import numpy as np
import pytest
import torch

import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, tol

pytestmark = pytest.mark.gpu


def sample(n: int, band: int, seed: int):
    rng = np.random.default_rng(seed)
    idx = set()
    for s in range(0, n, band):
        e = min(s + band, n)
        idx.update({s, e - 1, int(rng.integers(s, e))})
    return sorted(idx)


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 51, 52])
def test_workload_full_size(wid):
    w = gi.WORKLOADS[wid]
    note(f"workload {w.name}")
    inp = gi.make(w)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    A = inp["A"].cuda()
    B = inp["B"].cuda()
    C = inp["C0"].cuda() if inp["C0"] is not None else torch.full((w.M, w.N), float("nan"),
                                                                    dtype=tdt, device="cuda")
    fn = dg.gemm_f32 if w.dtype == "f32" else dg.gemm_bf16
    st = fn(w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, B.data_ptr(), w.N, w.beta,
            C.data_ptr(), w.N, int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    assert bool(torch.isfinite(C.float()).all())
    rows = sample(w.M, 128, wid)
    cols = sample(w.N, 128, wid + 1)
    got = C[rows][:, cols].cpu().to(torch.float64).numpy()
    R, D = oracle.gemm(gi.as_numpy(inp["A"]), gi.as_numpy(inp["B"]),
                       gi.as_numpy(inp["C0"]) if inp["C0"] is not None else None,
                       w.alpha, w.beta, w.dtype, rows=rows, cols=cols)
    err = oracle.max_rel_err(got, R, D)
    note(f"workload {w.name}: {len(rows)}x{len(cols)} sampled entries, max error ratio {err:.3e}")
    assert err <= tol(w.dtype)


def test_workload_small_m_split_k():
    # The small-M workload through gemm_bf16_ws, as the benchmark times it:
    # 128 strips x 2 K segments; two calls in a row on one workspace (the
    # second relies on the counters the first left at zero).
    w = gi.WORKLOADS[52]
    note(f"workload {w.name} via gemm_bf16_ws")
    inp = gi.make(w)
    A, B = inp["A"].cuda(), inp["B"].cuda()
    nbytes = dg.gemm_bf16_workspace_size(w.M, w.N, w.K)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    rows = list(range(w.M))
    cols = sample(w.N, 64, 520)
    R, D = oracle.gemm(gi.as_numpy(inp["A"]), gi.as_numpy(inp["B"]), None, w.alpha, w.beta,
                       w.dtype, rows=rows, cols=cols)
    for call in range(2):
        C = torch.full((w.M, w.N), float("nan"), dtype=torch.bfloat16, device="cuda")
        st = dg.gemm_bf16_ws(w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, B.data_ptr(), w.N,
                             w.beta, C.data_ptr(), w.N, ws.data_ptr(), nbytes,
                             int(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert st == dg.GEMM_OK, dg.gemm_status_string(st)
        assert bool(torch.isfinite(C.float()).all())
        got = C[:, cols].cpu().to(torch.float64).numpy()
        err = oracle.max_rel_err(got, R, D)
        note(f"call {call}: max error ratio {err:.3e}")
        assert err <= tol(w.dtype)


def test_workload_edge_split_k():
    # 4095 x 4097 x 1023 through gemm_f32_ws: 1024 whole tiles, then the last
    # 32 tiles (the ragged ones among them) split into 8 K ranges each.
    w = gi.WORKLOADS[51]
    note(f"workload {w.name} via gemm_f32_ws")
    inp = gi.make(w)
    A, B, C = inp["A"].cuda(), inp["B"].cuda(), inp["C0"].cuda()
    nbytes = dg.gemm_f32_workspace_size(w.M, w.N, w.K)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    st = dg.gemm_f32_ws(w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, B.data_ptr(), w.N, w.beta,
                        C.data_ptr(), w.N, ws.data_ptr(), nbytes,
                        int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == dg.GEMM_OK, dg.gemm_status_string(st)
    assert bool(torch.isfinite(C).all())
    rows = sample(w.M, 128, 610)
    cols = sample(w.N, 128, 611)
    got = C[rows][:, cols].cpu().to(torch.float64).numpy()
    R, D = oracle.gemm(gi.as_numpy(inp["A"]), gi.as_numpy(inp["B"]), gi.as_numpy(inp["C0"]),
                       w.alpha, w.beta, w.dtype, rows=rows, cols=cols)
    err = oracle.max_rel_err(got, R, D)
    note(f"max error ratio {err:.3e}")
    assert err <= tol(w.dtype)
