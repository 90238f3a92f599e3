"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random matrices. It holds none of the GEMM arithmetic,
so both the CPU oracle and the HIP library can be fed from it without sharing
any code with each other.

Every matrix comes from its own CPU ``torch.Generator`` seeded with
``1000 * workload_id + {A: 1, B: 2, C0: 3}``. Uniform[-1, 1] is
``rand * 2 - 1`` in fp32, normal is ``randn`` in fp32, and a bf16 matrix is
the fp32 sample rounded to bf16 by torch (round to nearest, ties to even).

The workloads follow the shapes the pages discuss: the 4096-cubed SGEMM of the
RTX 3090 SGEMM article (section 1.1, "why 4096"), the BF16 GEMM of the
Blackwell BF16 notes (section 1.2 for the format, section 5.2 for the small-M
inference shapes) and a transformer projection shape (same notes, section 1.1,
QKV / MLP projections are GEMMs).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int                 # seed family: 1000 * wid + {1, 2, 3}
    name: str
    dtype: str               # "f32" or "bf16" (storage type of A, B, C)
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dist_a: str              # "u" = U[-1,1], "n" = N(0,1)
    dist_b: str
    b_scale: float = 1.0     # multiplies the B sample before rounding
    dist_c: Optional[str] = None   # C0 distribution, None when beta == 0

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """Each operand read once, C written once, C0 read once if beta != 0."""
        c_passes = 1 + (1 if self.beta != 0.0 else 0)
        return self.elem_bytes * (self.M * self.K + self.K * self.N + c_passes * self.M * self.N)


WORKLOADS = {
    1: Workload(1, "sgemm_f32_256", "f32", 256, 256, 256, 1.0, 0.0, "u", "u"),
    2: Workload(2, "sgemm_f32_4096", "f32", 4096, 4096, 4096, 1.0, 0.0, "u", "u"),
    3: Workload(3, "gemm_bf16_4096", "bf16", 4096, 4096, 4096, 1.0, 0.0, "n", "n"),
    4: Workload(4, "gemm_bf16_proj_8192x12288x4096", "bf16", 8192, 12288, 4096, 1.0, 1.0,
                "n", "n", b_scale=1.0 / math.sqrt(4096), dist_c="n"),
    51: Workload(51, "sgemm_f32_edge_4095x4097x1023", "f32", 4095, 4097, 1023, 0.5, 2.0,
                 "u", "u", dist_c="u"),
    52: Workload(52, "gemm_bf16_skinny_16x8192x8192", "bf16", 16, 8192, 8192, 1.0, 0.0, "u", "u"),
}


def _draw(rows: int, cols: int, dist: str, seed: int, scale: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    if dist == "u":
        x = torch.rand(rows, cols, generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif dist == "n":
        x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if scale != 1.0:
        x = x * scale
    return x


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x.contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def make(w: Workload, M: Optional[int] = None, N: Optional[int] = None,
         K: Optional[int] = None) -> dict:
    """Draw A (MxK), B (KxN) and C0 (MxN, or None) as contiguous CPU tensors.

    ``M``, ``N`` and ``K`` override the workload's shape while keeping its
    seeds and distributions (used for smaller parity cases).
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    base = 1000 * w.wid
    A = _store(_draw(M, K, w.dist_a, base + 1), w.dtype)
    B = _store(_draw(K, N, w.dist_b, base + 2, w.b_scale), w.dtype)
    C0 = None
    if w.dist_c is not None:
        C0 = _store(_draw(M, N, w.dist_c, base + 3), w.dtype)
    return {"A": A, "B": B, "C0": C0, "alpha": w.alpha, "beta": w.beta,
            "M": M, "N": N, "K": K, "dtype": w.dtype}


def random_matrix(rows: int, cols: int, dtype: str, seed: int, dist: str = "u",
                  scale: float = 1.0) -> torch.Tensor:
    """One seeded matrix, for the shape sweeps in the tests."""
    return _store(_draw(rows, cols, dist, seed, scale), dtype)


def small_int_matrix(rows: int, cols: int, dtype: str, seed: int, lo: int = -4,
                     hi: int = 4) -> torch.Tensor:
    """Seeded integers in [lo, hi], stored exactly in fp32 or bf16."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randint(lo, hi + 1, (rows, cols), generator=g).to(torch.float32)
    return _store(x, dtype)


def as_numpy(t: torch.Tensor) -> np.ndarray:
    """fp32 tensors as float32 arrays; bf16 tensors as their uint16 bit patterns."""
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)
