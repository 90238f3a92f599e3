"""The five workloads at full size, in the launch configuration the benchmark
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
