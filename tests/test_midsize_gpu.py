"""The mid-size shapes that the benchmark's --all run times, at their full
sizes and in the launch configuration it times (default kernel choice, packed
leading dimensions): the plain call, and the split-K call through a workspace
when the size query asks for one. Between them they run the bf16 tiled kernel
on 128 x 128 tiles (K split between two groups of waves) and on a round of
256 x 256 tiles beside a strip, the small-M kernel at 128 rows, the fp32
kernel with a last round more than half full (one tile per CU beside a strip,
or split over K) and the bf16 few-tile kernel.

Compared with the oracle on sampled rows and columns of C that touch every
64-row and every 64-column band (the first, the last and one random row of
each band, over all N columns; the same for columns, over all M rows): every
output tile of every kernel is checked, while the oracle does a few percent
of the full product (the full oracle for these shapes takes minutes).
"""
import numpy as np
import pytest
import torch

import bench
import dense_gemm_04_amd as dg
import gemm_inputs as gi
import oracle
from gpu_util import note, to_f64, tol

pytestmark = pytest.mark.gpu

MIDSIZE = {w.wid: w for w in bench.midsize_workloads()}


def _sample(n, seed):
    rng = np.random.default_rng(seed)
    idx = set()
    for b0 in range(0, n, 64):
        b1 = min(n, b0 + 64)
        idx.update((b0, b1 - 1, int(rng.integers(b0, b1))))
    return sorted(idx)


@pytest.mark.parametrize("wid", sorted(MIDSIZE))
def test_midsize_sampled(wid):
    w = MIDSIZE[wid]
    d = gi.make(w)
    A, B = d["A"].cuda(), d["B"].cuda()
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    rows, cols = _sample(w.M, 7000 + wid), _sample(w.N, 7100 + wid)
    a_np, b_np = gi.as_numpy(d["A"]), gi.as_numpy(d["B"])
    c0_np = gi.as_numpy(d["C0"]) if d["C0"] is not None else None
    R_rows, D_rows = oracle.gemm(a_np, b_np, c0_np, w.alpha, w.beta, w.dtype, rows=rows)
    R_cols, D_cols = oracle.gemm(a_np, b_np, c0_np, w.alpha, w.beta, w.dtype, cols=cols)
    size_fn = dg.gemm_f32_workspace_size if w.dtype == "f32" else dg.gemm_bf16_workspace_size
    nbytes = size_fn(w.M, w.N, w.K)
    calls = [("plain", 0)] + ([("workspace", nbytes)] if nbytes else [])
    for label, nb in calls:
        note(f"workload {w.name}, {label} call ({nb} workspace bytes)")
        C = (d["C0"].cuda() if d["C0"] is not None
             else torch.full((w.M, w.N), float("nan"), dtype=tdt, device="cuda"))
        ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device="cuda")
        if w.dtype == "f32":
            fn = dg.gemm_f32_ws if nb else dg.gemm_f32
        else:
            fn = dg.gemm_bf16_ws if nb else dg.gemm_bf16
        args = (w.M, w.N, w.K, w.alpha, A.data_ptr(), w.K, B.data_ptr(), w.N, w.beta,
                C.data_ptr(), w.N)
        st = fn(*args, ws.data_ptr(), nb, 0) if nb else fn(*args, 0)
        torch.cuda.synchronize()
        assert st == dg.GEMM_OK, dg.gemm_status_string(st)
        Ch = C.cpu()
        e_rows = oracle.max_rel_err(to_f64(Ch[rows]), R_rows, D_rows)
        e_cols = oracle.max_rel_err(to_f64(Ch[:, cols]), R_cols, D_cols)
        note(f"workload {w.name}, {label}: {len(rows)} rows and {len(cols)} columns, "
             f"max error ratio {max(e_rows, e_cols):.3e}")
        assert e_rows <= tol(w.dtype) and e_cols <= tol(w.dtype), (label, e_rows, e_cols)
