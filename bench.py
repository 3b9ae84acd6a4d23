"""Throughput of batch-invariant RMSNorm forward + backward on one MI355X.

A step is one pass of the whole path over one batch: rmsnorm_fwd (y, rstd),
then the backward's two kernels, rmsnorm_bwd_rows (dx and the dgamma chunk
partials) and rmsnorm_bwd_finish (dgamma). Inputs are resident in HBM before
timing starts. The default workload is the token norm at T=32768, D=4096
(bf16 activations with 1% outlier rows, fp32 gamma, eps=1e-6); --workload
selects the other synthetic workloads (`residual`: the same inputs through
rmsnorm_residual_fwd, which also writes a byte copy of x, then the backward,
with --gres also the residual copy's gradient).

Prints one JSON line. `value` is algorithmic bytes per step (each input
element read once, each output written once; formulas in algo_bytes) over
the mean step time of the K timed steps, each step timed with HIP events and
preceded, outside its events, by a read of a buffer four times the 256 MB
Infinity Cache, so no step finds the previous step's tensors there. `warm`
is the same K steps back to back (wall clock), where part of x is still in
the Infinity Cache from the step before. `kernels` and `kernels_cold` are
per-kernel times from passes whose steps bracket every kernel with events;
in `kernels_cold` the cache is also flushed between the forward and the
backward, so the rows kernel reads x from HBM as it does in training, where
other layers run between a norm's forward and its backward. `roofline` is
the dominant kernel (the backward rows kernel; the gated kernel for the
gated workload) from that pass against MI355X's 8 TB/s HBM peak;
`roofline_cache_assisted` the same kernel back to back. `copy_ceiling` times
the runtime's own 2 GiB device copy in the same run, a practical ceiling for
one read and one write stream. `cpu_baseline` times the CPU oracle on the
host cores for the same workload (16 threads, the host's share per GPU, and
one thread).

--workload gemm times the batch-invariant BF16 GEMM Y = X @ W.T instead
(bigemm_bf16_xwt, M = N = K = 4096 unless --m/--n/--k say otherwise): a
step is one GEMM, `value` is 2MNK flops per step / wall time in TFLOP/s, and
`roofline` compares the kernel with the 2.5 PFLOP/s dense bf16 matrix-core
peak; torch.matmul (the library GEMM, which is not batch-invariant) is timed
beside it for context.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "RMSNorm fwd+bwd GB/s and % HBM peak, T=32768 D=4096 bf16, 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of one MI355X
TRAFFIC_FILE = ROOT / "profiles" / "traffic_bwd_rows_T32768_D4096.json"
# sources of the rows kernel: a committed counter figure is used only while
# these are unchanged
BWD_SOURCES = ["bwd.hip", "bwd_kernel.hpp", "device_common.hpp", "geometry.hpp", "launch.hpp",
               "plan.hpp"]
GEMM_TRAFFIC_FILE = ROOT / "profiles" / "traffic_bigemm_M4096_N4096_K4096.json"
GEMM_SOURCES = ["gemm.hip", "device_common.hpp", "geometry.hpp", "launch.hpp"]


def algo_bytes(kind: str, T: int, D: int) -> int:
    """Algorithmic bytes (each input read once, each output written once)."""
    return {
        "fwd": T * (4 * D + 4) + 4 * D,            # x in, y out, rstd out, gamma in
        "residual_fwd": T * (6 * D + 4) + 4 * D,   # + residual copy out
        "gated_fwd": T * 6 * D + 4 * D,            # x, z in, out out, gamma in
        "bwd_rows": T * (6 * D + 4) + 4 * D,       # g, x in, rstd in, dx out, gamma in
        "bwd_rows_gres": T * (8 * D + 4) + 4 * D,  # + residual gradient in
        "bwd_finish": 4 * D,                       # dgamma out
        "add_fwd": T * (8 * D + 4) + 4 * D,        # x, residual in; y, residual_out, rstd out
        "add_bwd_rows": T * (8 * D + 4) + 4 * D,   # g, x, residual, rstd in; dh out
        "add_bwd_rows_gres": T * (10 * D + 4) + 4 * D,  # + gradient of residual_out in
    }[kind]


def source_hash(names=BWD_SOURCES) -> str:
    h = hashlib.sha256()
    for name in names:
        h.update((ROOT / "invariant_rmsnorm_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE, names=BWD_SOURCES):
    """HBM bytes per launch of a kernel from committed rocprofv3 counter
    runs, or None if absent or taken on a different kernel source."""
    try:
        rec = json.loads(path.read_text())
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash(names):
        return None
    return rec.get("hbm_bytes_per_launch")


def make_inputs(workload: str, torch, dev, rows: int = 0, dim: int = 0, gres: bool = False):
    import numpy as np
    from synth import workloads as wl

    def d_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if workload in ("token", "token_gres", "residual"):
        with_gres = workload == "token_gres" or (workload == "residual" and gres)
        p = wl.residual(T=rows or 32768, D=dim or 4096, with_gres=with_gres)
        desc = (f"token RMSNorm fwd+bwd with dgamma, T={p.T}, D={p.D}, bf16 x ~N(0,1) with 1% "
                "outlier rows x50, g ~N(0,1), fp32 gamma=1+N(0,0.1), eps=1e-6")
        if workload == "residual":
            desc = ("rmsnorm_residual fwd (y, rstd and a byte copy of x) + bwd with dgamma"
                    + (" and the residual copy's gradient g_res ~N(0,1) added to dx"
                       if with_gres else "")
                    + desc[len("token RMSNorm fwd+bwd with dgamma"):])
        elif workload == "token_gres":
            desc = desc.replace("with dgamma", "with dgamma and a residual gradient g_res ~N(0,1) "
                                "added to dx (plain forward)")
    elif workload == "large":
        p = wl.large()
        desc = ("RMSNorm fwd+bwd with dgamma, T=262144, D=4096, zero-centred gamma, "
                "g ~0.01 N(0,1), eps=1e-6")
    elif workload == "add":
        p = wl.fused_add(T=rows or 32768, D=dim or 4096)
        desc = (f"fused add-RMSNorm fwd+bwd with dgamma, T={p.T}, D={p.D}: h = x + residual "
                "(fp32), bf16 x, residual, g, residual-output gradient ~N(0,1), fp32 "
                "gamma=1+N(0,0.1), eps=1e-6")
    elif workload == "gated":
        p = wl.gated()
        desc = "SiLU-gated per-head RMSNorm forward, 262144 rows x D=128, x,z ~N(0,1)"
    else:
        raise SystemExit(f"unknown workload {workload}")
    t = {"x": d_bf16(p.x), "gamma": torch.from_numpy(p.gamma).to(dev)}
    if p.g is not None:
        t["g"] = d_bf16(p.g)
    if p.gres is not None:
        t["gres"] = d_bf16(p.gres)
    if p.z is not None:
        t["z"] = d_bf16(p.z)
    if p.residual is not None:
        t["residual"] = d_bf16(p.residual)
    return p, t, desc


# Host threads for the oracle: the CPU share of one GPU on the GPU hosts
# (16), whatever the machine's own count is.
CPU_SHARE_THREADS = 16


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p, workload: str, seconds: float, nthreads: int):
    """The CPU oracle (R64 mode, as it stands) on the same workload, threads
    over row blocks (forward, dx) and column blocks (dgamma): whole passes
    over the workload until `seconds` of wall time have passed (at least
    one). Returns (wall seconds, passes)."""
    import numpy as np
    import oracle

    T, D = p.x.shape
    rows = np.array_split(np.arange(T), nthreads)
    cols = np.array_split(np.arange(D), nthreads)
    rstd = np.empty(T, np.float32)

    def fwd_block(ix):
        a, b = ix[0], ix[-1] + 1
        if workload == "gated":
            _, r = oracle.gated_fwd(p.x[a:b], p.z[a:b], p.gamma, p.zero_centered, p.eps)
        elif workload == "residual":
            _, _, r = oracle.residual_fwd(p.x[a:b], p.gamma, p.zero_centered, p.eps)
        elif workload == "add":
            _, _, r = oracle.add_fwd(p.x[a:b], p.residual[a:b], p.gamma, p.zero_centered, p.eps)
        else:
            _, r = oracle.fwd(p.x[a:b], p.gamma, p.zero_centered, p.eps)
        rstd[a:b] = r

    def dx_block(ix):
        a, b = ix[0], ix[-1] + 1
        if workload == "add":
            oracle.add_bwd(p.g[a:b], p.x[a:b], p.residual[a:b], rstd[a:b], p.gamma,
                           p.zero_centered, None if p.gres is None else p.gres[a:b],
                           want_dgamma=False)
            return
        oracle.bwd_dx(p.g[a:b], p.x[a:b], rstd[a:b], p.gamma, p.zero_centered,
                      None if p.gres is None else p.gres[a:b])

    def dg_block(ix):
        a, b = ix[0], ix[-1] + 1
        if workload == "add":
            oracle.add_bwd(p.g[:, a:b], p.x[:, a:b], p.residual[:, a:b], rstd,
                           p.gamma[a:b], p.zero_centered, want_dh=False)
            return
        oracle.dgamma(p.g[:, a:b], p.x[:, a:b], rstd)

    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nthreads) as ex:
        while passes == 0 or time.perf_counter() - t0 < seconds:
            list(ex.map(fwd_block, rows))
            if p.g is not None:
                list(ex.map(dx_block, rows))
                list(ex.map(dg_block, cols))
            passes += 1
    return time.perf_counter() - t0, passes


def cpu_baseline_record(p, workload, step_bytes, seconds, what):
    """The cpu_baseline object: CPU_SHARE_THREADS threads for `seconds`,
    then one thread for half as long."""
    T, D = p.x.shape
    dt, passes = cpu_baseline(p, workload, seconds, CPU_SHARE_THREADS)
    dt1, passes1 = cpu_baseline(p, workload, seconds / 2, 1)
    return {"value": round(step_bytes * passes / dt / 1e9, 3), "unit": "GB/s",
            "cores": CPU_SHARE_THREADS, "kind": "oracle",
            "sample": f"the full workload ({T} rows x {D}), {passes} passes of {what}, "
                      f"{dt:.1f} s wall",
            "one_thread": {"value": round(step_bytes * passes1 / dt1 / 1e9, 3), "unit": "GB/s",
                           "sample": f"{passes1} passes, {dt1:.1f} s wall"},
            "cpu_model": cpu_model(), "host_threads": os.cpu_count()}


def calibration_copy(torch, dev):
    """Five plain 256 MiB device copies: the known byte count that scales
    the HBM traffic counters."""
    src = torch.empty(1 << 27, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("calibration copy: 5 x 268435456 bytes read + written", file=sys.stderr, flush=True)
    del src, dst


def copy_ceiling(torch, dev, flush_mib: int):
    """The runtime's device-to-device copy of 2 GiB into 2 GiB (one read and
    one write stream), each of 5 copies preceded by a cache flush outside its
    events: a practical ceiling for kernels that stream one input and one
    output through HBM."""
    n = 1 << 31
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    flush_buf = torch.zeros(flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    dst.copy_(src)
    ms = []
    for _ in range(5):
        flush_buf.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    del src, dst, flush_buf
    best = min(ms)
    mean = sum(ms) / len(ms)
    return {"bytes": 2 * n, "ms": round(mean, 5), "GB/s": round(2 * n / (mean * 1e-3) / 1e9, 2),
            "best_GB/s": round(2 * n / (best * 1e-3) / 1e9, 2),
            "what": "torch copy_ of 2 GiB to 2 GiB (the runtime's copy kernel), cache flushed "
                    "first, mean of 5"}


def gemm_cpu_baseline(x, w, seconds: float):
    """The CPU oracle's GEMM (double sums, as it stands) on a sample of the
    workload: blocks of 8 rows of X against all of W, threads over blocks,
    until `seconds` of wall time have passed. Returns (wall seconds, rows,
    threads)."""
    import oracle

    nthreads = CPU_SHARE_THREADS
    M = x.shape[0]
    blk = 8

    def rows_block(i):
        a = (i * blk) % M
        oracle.gemm_xwt(x[a:a + blk], w)

    done = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nthreads) as ex:
        i = 0
        while done == 0 or time.perf_counter() - t0 < seconds:
            list(ex.map(rows_block, range(i, i + nthreads)))
            i += nthreads
            done += nthreads * blk
    return time.perf_counter() - t0, done, nthreads


def bench_gemm(args, torch, irn, dev):
    """Batch-invariant BF16 GEMM leg: one bigemm_bf16_xwt per step."""
    import numpy as np
    import synth

    M, N, K = args.m, args.n, args.k
    xb = synth.normal_bf16(7007, 1, M, K)
    wb = synth.normal_bf16(7007, 2, N, K, scale=K ** -0.5)

    def d_bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x, w = d_bf16(xb), d_bf16(wb)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        irn.bigemm_bf16_xwt(x, w, y=y)

    step()
    ref = y.clone()
    step()
    torch.cuda.synchronize()
    if not torch.equal(ref, y):
        raise SystemExit("repeat GEMM is not bitwise identical")
    del ref
    if args.calibrate_copy:
        calibration_copy(torch, dev)
    for _ in range(args.warmup):
        step()
    every = max(1, args.event_every)
    sampled = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for i in range(0, args.steps, every)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev = sampled.get(i)
        if ev is not None:
            ev[0].record(stream)
        step()
        if ev is not None:
            ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = sum(a.elapsed_time(b) for a, b in sampled.values()) / len(sampled)
    flops = 2.0 * M * N * K
    ms_step = wall * 1e3 / args.steps
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (launch_ms * 1e-3) / 1e12

    # the library GEMM on the same operands, for context only
    wt = w.t()
    for _ in range(10):
        torch.matmul(x, wt)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_lib = max(10, min(args.steps, 200))
    e0.record(stream)
    for _ in range(n_lib):
        torch.matmul(x, wt)
    e1.record(stream)
    torch.cuda.synchronize()
    lib_ms = e0.elapsed_time(e1) / n_lib

    cpu = None
    if not args.no_cpu:
        dt, rows, nthreads = gemm_cpu_baseline(xb, wb, args.cpu_seconds)
        cpu = {"value": round(2.0 * rows * N * K / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": nthreads, "kind": "oracle",
               "sample": f"{rows} rows of X (blocks of 8) against all {N} rows of W, "
                         f"K={K}, {dt:.1f} s wall",
               "cpu_model": cpu_model(), "host_threads": os.cpu_count()}

    out = {
        "metric": f"Batch-invariant BF16 GEMM TFLOP/s, Y = X @ W.T, M={M} N={N} K={K}, 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate_dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"batch-invariant GEMM Y = X @ W.T, M={M}, N={N}, K={K}, "
                               "bf16 X ~N(0,1), W ~N(0,1/K)",
                   "M": M, "N": N, "K": K, "flops_per_step": flops, "parallelism": "single GPU"},
        "library_gemm": {"kernel": "torch.matmul (not batch-invariant)", "ms": round(lib_ms, 5),
                         "TFLOP/s": round(flops / (lib_ms * 1e-3) / 1e12, 2),
                         "bigemm_over_library_time": round(launch_ms / lib_ms, 4)},
        "roofline": {"bound": "mfma", "kernel": gemm_kernel_name(M, N), "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": (measured_traffic(GEMM_TRAFFIC_FILE, GEMM_SOURCES)
                                 if (M, N, K) == (4096, 4096, 4096) else None),
                     "bytes_per_launch": 2 * (M * K + N * K + M * N),
                     "flops_per_launch": flops, "launch_ms": round(launch_ms, 5),
                     "launches_timed": len(sampled)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def gemm_kernel_name(M: int, N: int) -> str:
    """The GEMM kernel and output tile a launch of M x N runs."""
    import invariant_rmsnorm_amd as irn
    tm, tn = irn.bigemm_bf16_tile(M, N)
    return f"bigemm_dl_kernel ({tm}x{tn} tile)"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="token",
                    choices=["token", "token_gres", "residual", "large", "gated", "add", "gemm"])
    ap.add_argument("--gres", action="store_true",
                    help="residual workload: pass the residual copy's gradient to the backward")
    ap.add_argument("--m", type=int, default=4096, help="gemm workload: rows of X and Y")
    ap.add_argument("--n", type=int, default=4096, help="gemm workload: rows of W, columns of Y")
    ap.add_argument("--k", type=int, default=4096, help="gemm workload: reduction length")
    ap.add_argument("--rows", type=int, default=0,
                    help="token workloads: batch rows T (default 32768, the metric's size)")
    ap.add_argument("--dim", type=int, default=0,
                    help="token and add workloads: row length D (default 4096)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time of the CPU-oracle baseline (whole passes)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="MiB read before each timed step (and, in the cold kernel pass, "
                         "between the forward and the backward) to evict the Infinity Cache; "
                         "0 = time back-to-back steps only")
    ap.add_argument("--event-every", type=int, default=10,
                    help="bracket the dominant kernel with timing events on every N-th "
                         "timed step (the roofline figure)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(rows shard along T with no communication except one dgamma exchange; "
              "see the design notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import invariant_rmsnorm_amd as irn

    irn.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "gemm":
        bench_gemm(args, torch, irn, dev)
        return
    p, t, desc = make_inputs(args.workload, torch, dev, args.rows, args.dim, args.gres)
    T, D = p.T, p.D
    zc, eps = p.zero_centered, p.eps
    x, gamma = t["x"], t["gamma"]
    y = torch.empty_like(x)
    rstd = torch.empty(T, dtype=torch.float32, device=dev)
    gated = args.workload == "gated"
    add = args.workload == "add"
    resid = args.workload == "residual"
    rout = torch.empty_like(x) if (add or resid) else None
    if not gated:
        g = t["g"]
        gres = t.get("gres")
        dx = torch.empty_like(x)
        dgamma = torch.empty(D, dtype=torch.float32, device=dev)
        ws, _ = irn.workspace_for(T, D, dev)
    stream = torch.cuda.current_stream(dev)

    def step(evs=None, dom=None, flush_between=None):
        """One pass of the path. `evs` (5 events; 2 for the gated forward)
        brackets every kernel, `dom` only the dominant one; `flush_between`
        runs between the forward and the backward, outside the events."""
        if evs is not None:
            evs[0].record(stream)
        if gated:
            if dom is not None:
                dom[0].record(stream)
            irn.rmsnorm_gated_fwd(x, t["z"], gamma, zc, eps, out=y)
            if dom is not None:
                dom[1].record(stream)
        elif add:
            irn.rmsnorm_add_fwd(x, t["residual"], gamma, zc, eps, y=y, residual_out=rout, rstd=rstd)
        elif resid:
            irn.rmsnorm_residual_fwd(x, gamma, zc, eps, y=y, residual_out=rout, rstd=rstd)
        else:
            irn.rmsnorm_fwd(x, gamma, zc, eps, y=y, rstd=rstd)
        if evs is not None:
            evs[1].record(stream)
        if not gated:
            if flush_between is not None:
                flush_between()
            if evs is not None:
                evs[2].record(stream)
            if dom is not None:
                dom[0].record(stream)
            if add:
                irn.rmsnorm_add_bwd_rows(g, x, t["residual"], rstd, gamma, zc,
                                         g_residual_out=gres, dh=dx, workspace=ws)
            else:
                irn.rmsnorm_bwd_rows(g, x, rstd, gamma, zc, g_residual=gres, dx=dx, workspace=ws)
            if dom is not None:
                dom[1].record(stream)
            if evs is not None:
                evs[3].record(stream)
            irn.rmsnorm_bwd_finish(ws, T, D, dgamma)
            if evs is not None:
                evs[4].record(stream)

    # bitwise check before timing (two identical steps)
    step()
    outs = [y] + ([] if gated else [rstd, dx, dgamma]) + ([rout] if rout is not None else [])
    ref = [o.clone() for o in outs]
    step()
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(ref, outs)):
        raise SystemExit("repeat step is not bitwise identical")
    if resid and not torch.equal(rout.view(torch.int16), x.view(torch.int16)):
        raise SystemExit("residual_out is not a byte copy of x")
    del ref

    if args.calibrate_copy:
        calibration_copy(torch, dev)

    for _ in range(args.warmup):
        step()

    # A read of a buffer four times the 256 MB Infinity Cache evicts every
    # line of the previous kernels (it leaves no dirty lines of its own).
    flush_buf = (torch.zeros(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
                 if args.flush_mib > 0 else None)

    def flush():
        if flush_buf is not None:
            flush_buf.sum()

    def event_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # Timed region (`value`): K steps, each evicted from the cache first and
    # bracketed by its own pair of events (the flush stays outside them).
    step_evs = [event_pair() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        step_evs[i][0].record(stream)
        step()
        step_evs[i][1].record(stream)
    torch.cuda.synchronize()
    loop_wall = time.perf_counter() - t0
    step_ms = sorted(a.elapsed_time(b) for a, b in step_evs)
    ms_step = sum(step_ms) / args.steps
    ms_median = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else \
        0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])

    # Warm pass: the same K steps back to back (wall clock). A timing event
    # costs the GPU a few microseconds (it waits for the stream to drain), so
    # only every `event_every`-th step brackets its dominant kernel.
    every = max(1, args.event_every)
    sampled = {i: event_pair() for i in range(0, args.steps, every)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(dom=sampled.get(i))
    torch.cuda.synchronize()
    warm_wall = time.perf_counter() - t0
    dom_ms_warm = sum(a.elapsed_time(b) for a, b in sampled.values()) / len(sampled)

    fwd_kind = "gated_fwd" if gated else "add_fwd" if add else "residual_fwd" if resid else "fwd"
    rows_kind = None if gated else (("add_" if add else "") +
                                    ("bwd_rows_gres" if gres is not None else "bwd_rows"))
    step_bytes = algo_bytes(fwd_kind, T, D)
    if not gated:
        step_bytes += algo_bytes(rows_kind, T, D) + algo_bytes("bwd_finish", T, D)
        dom, dom_bytes = ("rmsnorm_bwd_rows_kernel" + (" (fused add)" if add else ""),
                          algo_bytes(rows_kind, T, D))
    else:
        dom, dom_bytes = "rmsnorm_fwd_kernel (gated)", step_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    ms_warm = warm_wall * 1e3 / args.steps
    traffic = measured_traffic() if (args.workload == "token" and T == 32768 and D == 4096) else None

    nev = 2 if gated else 5

    def breakdown(cold: bool):
        """Per-kernel times from a separate pass whose steps bracket every
        kernel with events; `cold` flushes the cache (outside the events)
        before the forward and again before the backward."""
        n = max(10, min(args.steps, 250))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(n)]
        for i in range(n):
            if cold:
                flush()
            step(evs[i], flush_between=flush if cold else None)
        torch.cuda.synchronize()
        f = sum(e[0].elapsed_time(e[1]) for e in evs) / n
        out = {fwd_kind: {"ms": round(f, 5), "GB/s": round(algo_bytes(fwd_kind, T, D) / f / 1e6, 2)}}
        tot = f
        dom_ms = f
        if not gated:
            r = sum(e[2].elapsed_time(e[3]) for e in evs) / n
            fin = sum(e[3].elapsed_time(e[4]) for e in evs) / n
            out[rows_kind] = {"ms": round(r, 5), "GB/s": round(algo_bytes(rows_kind, T, D) / r / 1e6, 2)}
            out["bwd_finish"] = {"ms": round(fin, 5)}
            tot += r + fin
            dom_ms = r
        out["steps"] = n
        out["step_GB/s_from_kernel_events"] = round(step_bytes / tot / 1e6, 2)
        return out, dom_ms, n

    kernels, _, _ = breakdown(cold=False)
    kernels_cold, dom_ms_cold, n_cold = (breakdown(cold=True) if flush_buf is not None
                                         else (None, None, 0))
    del flush_buf
    copy = copy_ceiling(torch, dev, args.flush_mib) if args.flush_mib > 0 else None

    def roofline(ms, launches, note):
        achieved = dom_bytes / (ms * 1e-3) / 1e9
        r = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
             "bytes_per_launch": dom_bytes, "launch_ms": round(ms, 5), "launches_timed": launches,
             "timing": note}
        if copy is not None:
            r["frac_of_copy_ceiling"] = round(achieved / copy["GB/s"], 4)
        return r

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_record(p, args.workload, step_bytes, args.cpu_seconds,
                                  "gated forward" if gated else "forward + dx + dgamma")

    flushed = args.flush_mib
    out = {
        "metric": (METRIC if args.workload == "token" and T == 32768 and D == 4096
                   else f"{METRIC} [workload: {args.workload}, T={T}, D={D}]"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_median": round(ms_median, 5),
        "value_median": round(step_bytes / (ms_median * 1e-3) / 1e9, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic",
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "timing": (f"mean of HIP events around each of the {args.steps} steps; before each "
                   f"step, outside its events, a {flushed} MiB read evicts the Infinity Cache; "
                   f"the K-step loop took {loop_wall:.3f} s of wall time with those reads"
                   if flushed > 0 else "back-to-back steps (no cache flush); see warm"),
        "config": {"workload": desc, "T": T, "D": D, "zero_centered_gamma": zc,
                   "bytes_per_step": step_bytes, "parallelism": "single GPU"},
        "warm": {"value": round(step_bytes / (ms_warm * 1e-3) / 1e9, 2),
                 "pct_hbm_peak": round(100.0 * step_bytes / (ms_warm * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                 "ms_per_step": round(ms_warm, 5),
                 "timing": "wall clock over the same K steps back to back, no flush: part of x "
                           "is still in the Infinity Cache from the step before"},
        "kernels": kernels,
        "kernels_cold": kernels_cold,
        "roofline": (roofline(dom_ms_cold, n_cold, "HIP events around the kernel, the Infinity "
                              "Cache flushed just before it (x read from HBM)")
                     if dom_ms_cold is not None else
                     roofline(dom_ms_warm, len(sampled), "back to back, cache-assisted")),
        "roofline_cache_assisted": roofline(dom_ms_warm, len(sampled),
                                            "HIP events around the kernel on every "
                                            f"{every}th back-to-back step: the rows kernel finds "
                                            "part of x in the Infinity Cache"),
        "copy_ceiling": copy,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
