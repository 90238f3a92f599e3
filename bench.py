"""Benchmark: GEMM TFLOPS (2MNK/t) on one MI355X.

Default run: the 4096^3 fp32 SGEMM (the pages' headline shape) is the timed
step; `value` is its rate. Inputs are seeded synthetic matrices already
resident in HBM. A step is one library call (one kernel launch) on torch's
current stream, timed with HIP events over exactly --steps calls after
--warmup untimed calls (each leg first runs its call untimed for a quarter
second so the GPU clock has settled).

Also reported:
  roofline      the timed kernel against MI355X's published fp32 matrix peak;
  cpu_baseline  the CPU oracle (fp64, OpenMP over all host threads) on the
                whole 4096^3 product, as TFLOPS = 2MNK / seconds;
  workloads     every workload the parity tests cover, each timed as 7
                repetitions of n back-to-back calls (n >= 20 and a repetition
                >= 20 ms) after 10 warm-up calls, reported as the median and
                the minimum time per call; the split-K call (gemm_bf16_ws)
                beside the plain one for small M (the ragged fp32 shape needs no
                workspace: its partly full last round runs as a strip on the
                few-tile kernel); the small-M lines rotate 4 operand sets (512 MiB of B, more than
                the 256 MB Infinity Cache). Each carries its fraction of the
                bounding roofline, its HBM traffic ratio when a current
                counter summary exists, and its own oracle timing (config 1
                also on one thread). The 256^3 line, whose kernel takes less
                time than a caller needs to issue a call, also carries
                `graph`: 200 of the same calls captured in one HIP graph and
                replayed, each replay checked bit for bit against the eager
                result.

``--all`` prints one JSON line per workload instead (for the design notes).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}
PEAK_HBM_GBS = 8000.0
METRIC = "GEMM TFLOPS (2MNK/t) fp32 & bf16 at 4096³ + % of MI355X matrix peak"


def gemm_flops(M: int, N: int, K: int) -> int:
    """2*M*N*K: one multiply and one add per (i, j, k), as the SGEMM article counts."""
    return 2 * M * N * K


def tflops(flops: float, seconds: float) -> float:
    return flops / seconds / 1e12


SETTLE_SECONDS = 0.25

# Workloads also timed with the fused bias + GELU epilogue (--only, --all):
# the fp32 4096^3 SGEMM and the bf16 projection with its beta = 1 residual.
EPILOGUE_WORKLOADS = (2, 4)
# Mid-size shapes whose last round of tiles leaves compute units idle, timed
# by --all and --only with and without a split-K workspace (seed families
# 61..68).
def midsize_workloads():
    import gemm_inputs as gi
    return [gi.Workload(61, "gemm_bf16_512x8192x8192", "bf16", 512, 8192, 8192, 1.0, 0.0, "n", "n"),
            gi.Workload(62, "gemm_bf16_2048x2048x8192", "bf16", 2048, 2048, 8192, 1.0, 0.0, "n", "n"),
            gi.Workload(63, "gemm_bf16_128x8192x8192", "bf16", 128, 8192, 8192, 1.0, 0.0, "n", "n"),
            # last rounds more than half full: 324 and 320 tiles of 128 x 128
            # on 512 fp32 slots
            gi.Workload(64, "sgemm_f32_2048x2560x4096", "f32", 2048, 2560, 4096, 1.0, 0.0, "u", "u"),
            gi.Workload(65, "sgemm_f32_2304x2304x2048", "f32", 2304, 2304, 2048, 1.0, 0.0, "u", "u"),
            # 256 tiles of 64 x 64: the bf16 few-tile kernel
            gi.Workload(66, "gemm_bf16_1024x1024x4096", "bf16", 1024, 1024, 4096, 1.0, 0.0, "n", "n"),
            # 272 tiles of 256 x 256: one round of them and a 256-row strip
            gi.Workload(67, "gemm_bf16_4352x4096x4096", "bf16", 4352, 4096, 4096, 1.0, 0.0, "n", "n"),
            # one round of 144 tiles of 256 x 256; with a workspace 576 of
            # 128 x 128, the last 64 split over K
            gi.Workload(68, "gemm_bf16_3072x3072x8192", "bf16", 3072, 3072, 8192, 1.0, 0.0, "n", "n")]


# Workloads also timed with transposed operand storage (A^T B, A B^T, A^T B^T);
# the small-M workload with B stored N x K (a weight kept as [out][in]), split-K.
LAYOUT_WORKLOADS = {2: ((0, 1), (1, 0), (1, 1)), 3: ((0, 1), (1, 0), (1, 1)), 52: ((0, 1),)}


def _time_calls(call, steps: int, warmup: int, stream, settle: float = SETTLE_SECONDS):
    """Seconds per call over `steps` calls, after the GPU has settled and
    `warmup` untimed calls. Settling runs the call untimed for `settle`
    seconds first: from idle the GPU takes tens of milliseconds to reach its
    steady clock under load, and a 4096^3 bf16 GEMM measured right away runs
    about 20% slow."""
    import torch
    t_end = time.perf_counter() + settle
    while time.perf_counter() < t_end:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps     # seconds per call


def _device_call(w, sets: int = 1, use_ws: bool = False, act=None, ops=None, variant=None,
                 stream=None):
    """Allocate `sets` independent operand sets on the GPU and return a callable
    that runs the library on the next set each time (through gemm_*_ws with a
    zeroed workspace when `use_ws`; through gemm_*_bias_act with a seeded bias
    vector and activation `act` when `act` is given; through gemm_*_op with A
    stored K x M and/or B stored N x K when `ops` = (opa, opb) is given; through
    gemm_*_ex with `variant` when given), launching on `stream` (default: the
    current one). Each set's argument tuple is built once, and the call goes
    straight to the ctypes function, so that a call costs the caller as little
    as the binding allows (about 3 us, of which the HIP launch is 2.4)."""
    import itertools
    import torch
    import dense_gemm_04_amd as dg
    import gemm_inputs as gi
    lib = dg.load()
    f32 = w.dtype == "f32"
    inp = gi.make(w)
    bufs = []
    opa, opb = ops if ops is not None else (0, 0)
    for _ in range(sets):
        A = (inp["A"].t().contiguous() if opa else inp["A"]).cuda()
        B = (inp["B"].t().contiguous() if opb else inp["B"]).cuda()
        C = inp["C0"].cuda() if inp["C0"] is not None else torch.zeros(
            w.M, w.N, dtype=A.dtype, device="cuda")
        bufs.append((A, B, C))
    stream = stream if stream is not None else torch.cuda.current_stream()
    h = int(stream.cuda_stream)
    lda, ldb = (w.M if opa else w.K), (w.K if opb else w.N)
    size_fn = dg.gemm_f32_workspace_size if f32 else dg.gemm_bf16_workspace_size
    nbytes = size_fn(w.M, w.N, w.K) if use_ws else 0
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    wsp = ws.data_ptr() if nbytes else None
    # arguments: pre + (M, N, K, alpha, A, lda, B, ldb, beta, C, ldc) + mid + (stream,) + post
    pre, mid, post = (), (), ()
    if ops is not None:
        raw = lib.gemm_f32_op if f32 else lib.gemm_bf16_op
        pre, mid = (opa, opb), (None, 0, wsp, nbytes)
    elif act is not None:
        bias = gi.random_matrix(1, w.N, w.dtype, 1000 * w.wid + 4)[0].cuda()
        bufs.append(bias)
        raw = lib.gemm_f32_bias_act if f32 else lib.gemm_bf16_bias_act
        code = {v: k for k, v in dg.ACT_NAMES.items()}[act]
        mid = (bias.data_ptr(), code, wsp, nbytes)
    elif variant is not None:
        raw = lib.gemm_f32_ex if f32 else lib.gemm_bf16_ex
        post = (variant,)
    elif use_ws:
        raw = lib.gemm_f32_ws if f32 else lib.gemm_bf16_ws
        mid = (wsp, nbytes)
    else:
        raw = lib.gemm_f32 if f32 else lib.gemm_bf16
    argsets = [pre + (w.M, w.N, w.K, w.alpha, A.data_ptr(), lda, B.data_ptr(), ldb, w.beta,
                      C.data_ptr(), w.N) + mid + (h,) + post for A, B, C in bufs[:sets]]
    nxt = itertools.cycle(argsets).__next__

    def call():
        st = raw(*nxt())
        if st:
            raise RuntimeError(f"gemm returned {st}: {dg.gemm_status_string(st)}")
    call.keep = (bufs, ws)          # the buffers the argument tuples point into
    call.outputs = [b[2] for b in bufs[:sets]]
    return call, stream, inp


REPS = 7
MIN_REP_SECONDS = 0.02
MIN_REP_CALLS = 20


def _time_reps(call, stream, reps: int = REPS, warmup: int = 10):
    """(median, min) seconds per call and the calls per repetition: after the
    settling run and `warmup` calls, `reps` repetitions of n back-to-back
    calls, each bracketed by HIP events on the launch stream, with n chosen so
    that a repetition lasts at least MIN_REP_SECONDS and has at least
    MIN_REP_CALLS calls."""
    import statistics
    import torch
    probe = _time_calls(call, 10, warmup, stream)
    n = max(MIN_REP_CALLS, int(MIN_REP_SECONDS / max(probe, 1e-9)) + 1)
    per = []
    for _ in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(n):
            call()
        end.record(stream)
        torch.cuda.synchronize()
        per.append(start.elapsed_time(end) / 1e3 / n)
    return statistics.median(per), min(per), n


# Committed counter summary and kernel source behind each line of the
# `workloads` report (the traffic ratio is reported only while the summary's
# source hash matches the kernel built now).
PROFILE_OF = {
    "1": ("gemm_f32_small_256.md", "gemm_f32_small.hip"),
    "2": ("gemm_f32_mfma_4096.md", "gemm_f32_mfma.hip"),
    "3": ("gemm_bf16_tiled_4096.md", "gemm_bf16_tiled.hip"),
    "4": ("gemm_bf16_tiled_proj_8192x12288x4096.md", "gemm_bf16_tiled.hip"),
    "51": (("gemm_f32_mfma_edge_4095x4097x1023.md", "gemm_f32_mfma.hip"),
           ("gemm_f32_small_edge_strip_4095x1x1023.md", "gemm_f32_small.hip")),
    "52": ("gemm_bf16_smallm_16x8192x8192.md", "gemm_bf16_skinny.hip"),
    "52_ws": ("gemm_bf16_stream_splitk_16x8192x8192.md", "gemm_bf16_stream.hip"),
}

# The kernel each line runs.
KERNEL_OF = {
    "1": "gemm_f32_small (16x16 tiles, K over 8 waves)",
    "2": "gemm_f32_mfma (copy path, 128x128 tiles, tiles walked)",
    "3": "gemm_bf16_tiled (256x256 tiles)",
    "4": "gemm_bf16_tiled (256x256 tiles, beta = 1 residual)",
    "51": ("gemm_f32_mfma on C columns 0-4095 (two whole rounds, unaligned rows: 4-byte "
           "copies), then gemm_f32_small on column 4096"),
    "52": "gemm_bf16_smallm (64-column strips, 128 workgroups)",
    "52_ws": "gemm_bf16_stream (256-column strips, K interleaved over 8 phases)",
}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_timing(w, threads: int = 0) -> dict:
    """The oracle over every entry of the workload's C, timed by wall clock
    (`threads` = 0: all host threads)."""
    import oracle
    import gemm_inputs as gi
    inp = gi.make(w)
    A, B = gi.as_numpy(inp["A"]), gi.as_numpy(inp["B"])
    C0 = gi.as_numpy(inp["C0"]) if inp["C0"] is not None else None
    t0 = time.perf_counter()
    oracle.gemm(A, B, C0, w.alpha, w.beta, w.dtype, threads=threads)
    sec = time.perf_counter() - t0
    return {"seconds": round(sec, 3), "tflops": tflops(gemm_flops(w.M, w.N, w.K), sec),
            "gflops_fp64": gemm_flops(w.M, w.N, w.K) / sec / 1e9,
            "threads": threads if threads > 0 else oracle.max_threads(),
            "sample": f"all {w.M}x{w.N} entries"}


def workload_report(w, key: str, sets: int = 1, use_ws: bool = False) -> dict:
    """One line of the `workloads` report (see the module docstring)."""
    call, stream, _ = _device_call(w, sets, use_ws)
    med, mn, n = _time_reps(call, stream)
    peak = PEAK_TFLOPS[w.dtype]
    out = {"workload": w.name, "call": ("gemm_f32_ws" if w.dtype == "f32" else "gemm_bf16_ws")
           if use_ws else ("gemm_f32" if w.dtype == "f32" else "gemm_bf16"),
           "kernel": KERNEL_OF.get(key), "dtype": w.dtype, "M": w.M, "N": w.N, "K": w.K,
           "alpha": w.alpha, "beta": w.beta, "operand_sets": sets,
           "ms_median": round(med * 1e3, 5), "ms_min": round(mn * 1e3, 5),
           "reps": REPS, "calls_per_rep": n,
           "tflops": round(tflops(gemm_flops(w.M, w.N, w.K), med), 3),
           "peak_tflops": peak, "frac_matrix_peak": round(tflops(gemm_flops(w.M, w.N, w.K), med) / peak, 4),
           "algorithmic_bytes": w.algorithmic_bytes,
           "gbs": round(w.algorithmic_bytes / med / 1e9, 1),
           "frac_hbm": round(w.algorithmic_bytes / med / 1e9 / PEAK_HBM_GBS, 4)}
    traffic = workload_traffic(key)
    out["traffic_ratio"] = round(traffic / w.algorithmic_bytes, 2) if traffic else None
    out["bound"] = "hbm" if key.startswith("52") else "mfma"
    if key in GRAPH_KEYS:
        out["graph"] = graph_report(w, sets, use_ws)
    return out


# Workloads whose kernel runs in less time than a caller needs to issue one
# call: also timed as calls replayed from a captured HIP graph.
GRAPH_KEYS = ("1",)
GRAPH_CALLS = 200


def graph_report(w, sets: int = 1, use_ws: bool = False) -> dict:
    """GRAPH_CALLS calls captured once into a HIP graph (torch.cuda.CUDAGraph)
    on a stream of their own, then replayed: the GPU's own rate for
    back-to-back calls, without the per-call launch cost on the host. Each
    replay must leave C bit-identical to the eager call's result."""
    import statistics
    import torch
    s = torch.cuda.Stream()
    call, _, _ = _device_call(w, sets, use_ws, stream=s)
    with torch.cuda.stream(s):
        for _ in range(20):
            call()
    torch.cuda.synchronize()
    eager = [c.clone() for c in call.outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(GRAPH_CALLS):
            call()
    torch.cuda.synchronize()
    per = []
    same = True
    with torch.cuda.stream(s):
        t_end = time.perf_counter() + SETTLE_SECONDS
        while time.perf_counter() < t_end:
            g.replay()
            torch.cuda.synchronize()
        for _ in range(REPS):
            for c in call.outputs:
                c.fill_(float("nan"))
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            start.record(s)
            g.replay()
            end.record(s)
            torch.cuda.synchronize()
            per.append(start.elapsed_time(end) / 1e3 / GRAPH_CALLS)
            same = same and all(torch.equal(c, e) for c, e in zip(call.outputs, eager))
    med = statistics.median(per)
    return {"calls_per_graph": GRAPH_CALLS, "replays": REPS,
            "ms_median": round(med * 1e3, 5), "ms_min": round(min(per) * 1e3, 5),
            "tflops": round(tflops(gemm_flops(w.M, w.N, w.K), med), 3),
            "matches_eager": bool(same)}


def measure(w, steps: int, warmup: int, sets: int = 1, use_ws: bool = False, act=None,
            ops=None, variant=None) -> dict:
    call, stream, _ = _device_call(w, sets, use_ws, act, ops, variant)
    sec = _time_calls(call, steps, warmup, stream)
    ws_name = "gemm_f32_ws" if w.dtype == "f32" else "gemm_bf16_ws"
    epi_name = "gemm_f32_bias_act" if w.dtype == "f32" else "gemm_bf16_bias_act"
    label = f" ({ws_name}, split-K)" if use_ws else ""
    if act is not None:
        label = f" ({epi_name}, bias + {act})"
    if variant is not None:
        import dense_gemm_04_amd as dg
        label = f" (gemm_{w.dtype}_ex, {dg.VARIANT_NAMES[variant]} kernel)"
    if ops is not None:
        op_name = "gemm_f32_op" if w.dtype == "f32" else "gemm_bf16_op"
        label = (f" ({op_name}, {'A^T' if ops[0] else 'A'} {'B^T' if ops[1] else 'B'}"
                 + (", split-K)" if use_ws else ")"))
    out = {"workload": w.name + label,
           "dtype": w.dtype, "M": w.M, "N": w.N, "K": w.K,
           "alpha": w.alpha, "beta": w.beta, "ms": sec * 1e3,
           "tflops": tflops(gemm_flops(w.M, w.N, w.K), sec),
           "gbs": w.algorithmic_bytes / sec / 1e9}
    out["frac_matrix_peak"] = out["tflops"] / PEAK_TFLOPS[w.dtype]
    out["frac_hbm"] = out["gbs"] / PEAK_HBM_GBS
    return out


def vendor_lines(steps: int, warmup: int):
    """torch's own GEMM (the platform BLAS behind torch.mm / torch.addmm) on the
    headline workloads' operands, timed like this library's calls. Context only:
    it is not part of the path and not the benchmark's value."""
    import torch
    import gemm_inputs as gi
    torch.backends.cuda.matmul.allow_tf32 = False
    for wid, opb in ((1, 0), (2, 0), (3, 0), (4, 0), (51, 0), (52, 0), (52, 1)):
        w = gi.WORKLOADS[wid]
        inp = gi.make(w)
        # As for this library's small-M lines, 4 operand sets (512 MiB of B)
        # rotate so that the Infinity Cache cannot serve B.
        sets = 4 if wid == 52 else 1
        A = inp["A"].cuda()
        Bs = [(inp["B"].t().contiguous() if opb else inp["B"]).cuda() for _ in range(sets)]
        Bops = [B.t() if opb else B for B in Bs]
        C0 = inp["C0"].cuda() if inp["C0"] is not None else None
        out = torch.empty(w.M, w.N, dtype=A.dtype, device="cuda")
        state = {"i": 0}

        def call():
            Bop = Bops[state["i"] % sets]
            state["i"] += 1
            if C0 is None or w.beta == 0:
                torch.mm(A, Bop, out=out)
                if w.alpha != 1:
                    out.mul_(w.alpha)
            else:
                torch.addmm(C0, A, Bop, beta=w.beta, alpha=w.alpha, out=out)
        sec = _time_calls(call, steps, warmup, torch.cuda.current_stream())
        yield {"workload": w.name + (" (B stored N x K)" if opb else ""),
               "library": "torch.mm / torch.addmm " + torch.__version__,
               "ms": sec * 1e3, "tflops": tflops(gemm_flops(w.M, w.N, w.K), sec),
               "gbs": w.algorithmic_bytes / sec / 1e9}
        del A, Bs, Bops, C0, out


def kernel_source_sha(path: str) -> str:
    """First 16 hex digits of the sha256 of a kernel source's code and of the
    local headers it includes (`#include "..."`, followed through the headers
    they include): `//` comments, trailing blanks and empty lines removed, so
    that editing a comment leaves a counter summary current while any code
    change, in the kernel file or in shared device code, does not."""
    import hashlib
    import re
    code, seen, todo = [], set(), [os.path.abspath(path)]
    while todo:
        f = todo.pop(0)
        if f in seen or not os.path.exists(f):
            continue
        seen.add(f)
        for line in open(f, encoding="utf-8"):
            m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
            if m:
                todo.append(os.path.join(os.path.dirname(f), m.group(1)))
            line = re.sub(r"//.*", "", line).rstrip()
            if line:
                code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def workload_traffic(key: str):
    """HBM bytes per call of a `workloads` line: the sum over the kernels the
    call launches (PROFILE_OF holds one (summary, source) pair, or one pair
    per kernel), or None when any summary is missing or stale."""
    prof = PROFILE_OF.get(key)
    if not prof:
        return None
    pairs = (prof,) if isinstance(prof[0], str) else prof
    parts = [measured_traffic(*p) for p in pairs]
    return None if any(x is None for x in parts) else sum(parts)


def measured_traffic(summary: str, source: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary.

    The summary holds `source_sha: <hash>`, `fetch_bytes_per_launch: <n>` and
    `write_bytes_per_launch: <n>` lines (FETCH_SIZE and WRITE_SIZE already
    scaled by the copy-kernel calibration). Returns None when the summary is
    missing or was taken on a different kernel source than the one built now.
    """
    path = os.path.join(ROOT, "profiles", summary)
    src = os.path.join(ROOT, "dense_gemm_04_amd", "csrc", source)
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip().strip("-* `")] = v.strip().strip("`")
    if fields.get("source_sha") != kernel_source_sha(src):
        return None
    try:
        return int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--all", action="store_true", help="one JSON line per workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", type=int, default=None,
                    help="time one workload id (1, 2, 3, 4, 51, 52; 61-68 mid-size) and print its line "
                         "(with the split-K line for 52, the bias + GELU line for 2 and 4, "
                         "the transposed-layout lines for 2, 3 and 52)")
    ap.add_argument("--vendor", action="store_true",
                    help="time torch's own GEMM (torch.mm / torch.addmm, the platform BLAS) on the "
                         "headline workloads, for context beside this library's lines")
    ap.add_argument("--copy-mib", type=int, default=None,
                    help="time a plain device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the GEMM path runs on a single device and "
              "the library has no multi-GPU leg (run with --gpus 1).", file=sys.stderr)
        return 2

    import torch
    import gemm_inputs as gi
    import dense_gemm_04_amd as dg
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    dg.load()

    if args.copy_mib is not None:
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        stream = torch.cuda.current_stream()
        sec = _time_calls(lambda: dst.copy_(src), args.steps, args.warmup, stream, settle=0.0)
        print(json.dumps({"copy_bytes": n, "ms": sec * 1e3, "gbs": 2 * n / sec / 1e9}), flush=True)
        return 0

    if args.vendor:
        for line in vendor_lines(args.steps, args.warmup):
            print(json.dumps(line), flush=True)
        return 0

    if args.only is not None:
        extra = {m.wid: m for m in midsize_workloads()}
        w = gi.WORKLOADS[args.only] if args.only in gi.WORKLOADS else extra[args.only]
        if args.only in extra:
            for use_ws in (False, True):
                print(json.dumps(measure(w, args.steps, args.warmup, use_ws=use_ws)), flush=True)
            return 0
        r = measure(w, args.steps, args.warmup, 4 if args.only == 52 else 1)
        print(json.dumps(r), flush=True)
        if args.only == 52:
            print(json.dumps(measure(w, args.steps, args.warmup, 4 if args.only == 52 else 1,
                                     use_ws=True)), flush=True)
        if args.only in EPILOGUE_WORKLOADS:
            print(json.dumps(measure(w, args.steps, args.warmup, act="gelu_tanh")), flush=True)
        if args.only == 2:
            print(json.dumps(measure(w, args.steps, args.warmup, variant=dg.VARIANT_VALU)), flush=True)
        if args.only in LAYOUT_WORKLOADS:
            for ops in LAYOUT_WORKLOADS[args.only]:
                print(json.dumps(measure(w, args.steps, args.warmup, 4 if args.only == 52 else 1,
                                         use_ws=args.only == 52, ops=ops)), flush=True)
        return 0

    if args.all:
        for wid in (1, 2, 3, 4, 51, 52):
            w = gi.WORKLOADS[wid]
            # The small-M workload streams 128 MiB of B: rotate 4 sets (512 MiB)
            # so the 256 MB Infinity Cache cannot serve it.
            sets = 4 if wid == 52 else 1
            r = measure(w, args.steps, args.warmup, sets)
            print(json.dumps(r), flush=True)
            if wid in (51, 52):
                print(json.dumps(measure(w, args.steps, args.warmup, sets, use_ws=True)),
                      flush=True)
            if wid in EPILOGUE_WORKLOADS:
                print(json.dumps(measure(w, args.steps, args.warmup, sets, act="gelu_tanh")),
                      flush=True)
            if wid == 2:
                # The vector-FMA comparison kernel at the same shape.
                print(json.dumps(measure(w, args.steps, args.warmup, variant=dg.VARIANT_VALU)),
                      flush=True)
            if wid in LAYOUT_WORKLOADS:
                for ops in LAYOUT_WORKLOADS[wid]:
                    print(json.dumps(measure(w, args.steps, args.warmup, sets, use_ws=wid == 52,
                                             ops=ops)), flush=True)
        for w in midsize_workloads():
            for use_ws in (False, True):
                print(json.dumps(measure(w, args.steps, args.warmup, use_ws=use_ws)), flush=True)
        return 0

    w = gi.WORKLOADS[2]
    main_r = measure(w, args.steps, args.warmup)
    bf = measure(gi.WORKLOADS[3], args.steps, args.warmup)
    workloads = {}
    for key, wid, sets, use_ws in (("1", 1, 1, False), ("2", 2, 1, False), ("3", 3, 1, False),
                                   ("4", 4, 1, False), ("51", 51, 1, False),
                                   ("52", 52, 4, False), ("52_ws", 52, 4, True)):
        workloads[key] = workload_report(gi.WORKLOADS[wid], key, sets, use_ws)
    line = {
        "metric": METRIC,
        "value": round(main_r["tflops"], 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded U[-1,1] fp32 A and B, resident in HBM)",
        "config": {"workload": "SGEMM fp32 row-major M=N=K=4096, alpha=1, beta=0",
                   "M": w.M, "N": w.N, "K": w.K, "kernel": "gemm_f32 (MFMA 16x16x4 f32)"},
        "frac_of_matrix_peak": round(main_r["frac_matrix_peak"], 4),
        "roofline": {"bound": "mfma", "achieved": round(main_r["tflops"], 3),
                     "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s",
                     "frac": round(main_r["frac_matrix_peak"], 4),
                     "traffic": measured_traffic("gemm_f32_mfma_4096.md", "gemm_f32_mfma.hip")},
        "bf16_4096": {"workload": "BF16 GEMM M=N=K=4096, fp32 accumulate, bf16 out",
                      "tflops": round(bf["tflops"], 3), "ms": round(bf["ms"], 4),
                      "peak": PEAK_TFLOPS["bf16"], "frac": round(bf["frac_matrix_peak"], 4)},
    }
    line["workloads"] = workloads
    if not args.no_cpu:
        # The whole 4096^3 product on all host threads (3-4 s on 16 cores), and
        # every other workload's oracle beside its line.
        t = oracle_timing(w)
        line["cpu_baseline"] = {"value": t["tflops"], "unit": "TFLOPS", "cores": t["threads"],
                                "kind": "oracle", "cpu_model": cpu_model(),
                                "sample": f"all 4096x4096 entries of C (fp64 accumulate) in "
                                          f"{t['seconds']:.1f} s"}
        for key, rep in workloads.items():
            wid = int(key.split("_")[0])
            if key.endswith("_ws"):
                rep["cpu_oracle"] = workloads[str(wid)].get("cpu_oracle")
                continue
            rep["cpu_oracle"] = t if wid == 2 else oracle_timing(gi.WORKLOADS[wid])
        workloads["1"]["cpu_oracle_1_thread"] = oracle_timing(gi.WORKLOADS[1], threads=1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
