#!/usr/bin/env python3
"""Benchmark of the 1-bit Adam compression-phase step on one MI355X.

One step = ob_step over the whole tensor list: all W workers' momentum,
error feedback and 1-bit compression, the server's average and
re-compression, and the frozen-variance parameter update.  Inputs are
synthetic (seeded, generated on the device) and resident in HBM before the
timed region; a small pool of gradient sets is cycled so successive steps
see different gradients.

Prints one JSON line on stdout: elements/s of the whole step, the HBM
roofline of the dominant kernel (timed with HIP events on the launch stream
inside the timed region), the whole step's algorithmic GB/s, and the oracle
timed on a bounded sample on the host as a CPU baseline.
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

METRIC = "compressed optimizer-step elements/s and HBM GB/s (% of peak), 1 MI355X"
CSRC = os.path.join(ROOT, "error_compensated_bit_02_amd", "csrc")
# The device code and the host code that picks its launch shapes: stored
# counters count only while all of these are what they measured.
SOURCES = ("kernels.hip", "topk.hip", "internal.h", "api.cpp")
HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, AMD's published figure


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def grad_bytes(wl) -> int:
    return 2 if wl.grad_dtype == "bf16" else 4


def step_bytes_per_element(wl) -> float:
    """Bytes the method itself moves per parameter element per step, each
    operand touched once: gradients g*W, worker errors read and written 8W,
    momentum 8, server error 8, variance 4, parameters 8, and the sign
    messages written and read back W/8 + W/8."""
    W = wl.workers
    return 28.0 + (8.0 + grad_bytes(wl)) * W + W / 4.0


def kernel_bytes_per_element(wl) -> dict:
    """Bytes per element each kernel must move, its operands touched once."""
    W, g = wl.workers, grad_bytes(wl)
    return {
        "worker_pass1": 4.0 + (g + 4.0) * W + W / 8.0,        # read m, g, e; write signs
        "worker_pass2": 4.0 + (g + 4.0) * W + 4.0 * W,        # read m, g, e; write e
        "server_pass1": W / 8.0 + 4.0,                        # read signs, e_s
        "server_pass2_update": W / 8.0 + 12.0 + 12.0 + 1 / 8.0,  # read signs, e_s, v, p; write e_s, m, p, signs
        "server_pass2": W / 8.0 + 8.0 + 1 / 8.0,              # read signs, e_s; write e_s, signs
        "apply_update": 1 / 8.0 + 16.0,                       # read signs, v, p; write m, p
        "trust_norms": 1 / 8.0 + 8.0,                         # read signs, v, p
        # residual form: read g, x_prev and the previous server signs (the momentum); write x, signs
        "worker_residual": (g + 8.0) * W + W / 8.0 + 1 / 8.0,
        "server_residual": W / 8.0 + 8.0 + 1 / 8.0,           # read signs, z_prev; write z, server signs
        "update_residual": 1 / 8.0 + 12.0,                    # read server signs, v, p; write p
    }


def cltk_bytes_per_element(wl, density: float) -> dict:
    """Bytes per element each stage of the cyclic local top-k exchange must
    move, its own operands touched once (density d = kept fraction)."""
    W, g, d = wl.workers, grad_bytes(wl), density
    return {
        "cltk_select": g + 4.0,                    # read the leader's memory and gradient
        # read memory and gradient, write memory; write values and the index list
        "cltk_gather": (g + 8.0) * W + 4.0 * d * W + 4.0 * d,
        "cltk_average": d * (4.0 * W + 4.0),       # read values, write the average
    }


def sources_of(kernel: str) -> tuple:
    """The files whose change makes a kernel's stored counters stale: its
    device source, the shared layout constants and the launch code."""
    return ("topk.hip" if kernel.startswith("cltk_") else "kernels.hip", "internal.h", "api.cpp")


def sha256_of(name: str) -> str:
    import hashlib
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counter_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's
    reading), or None when there is none or its sources or launch code changed
    since."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    shas = data.get("sources_sha256", {})
    if any(shas.get(src) != sha256_of(src) for src in sources_of(kernel)):
        return None
    per = data.get("per_launch_bytes", {}).get(kernel)
    return None if per is None else float(per)


# rocprofv3 kernel names -> the library's kernel kinds.  Every topk_ kernel
# but the gather and the average belongs to the CLT-k select stage (eleven
# launches); its bytes are summed per exchange (per topk_reset).


def kind_of(name: str):
    import re
    m = re.search(r"ob::\(anonymous namespace\)::(\w+)(?:<([^>]*)>)?", name)
    if not m:
        return "copy" if "copyBuffer" in name else None
    base, args = m.group(1), [x.strip() for x in (m.group(2) or "").split(",")]
    if base in ("worker_kernel", "worker_chunk_kernel"):   # tiled or chunked; mode 4 is pass 2 in chunks
        return ("worker_pass1", "worker_pass2", "worker_residual_first", "worker_residual",
                "worker_pass2")[int(args[1])]
    if base == "server_kernel":
        return ("server_pass1", "server_pass2", "server_pass2_update", "server_residual_first",
                "server_residual")[int(args[0])]
    if base == "update_kernel":
        return "apply_update" if args[0] == "true" else "update_residual"
    if base.endswith("_kernel"):   # warmup, materialize, zero_errors, trust_norms, trust_ratio
        return base[: -len("_kernel")]
    if base in ("topk_gather", "topk_gather_chunk"):   # the tiled or the chunked shape
        return "cltk_gather"
    if base == "topk_average":
        return "cltk_average"
    if base.startswith("topk_"):
        return "cltk_select"
    return base


def summarize_counters(pmc_dir: str, workload: str) -> dict:
    """Turn rocprofv3 --pmc CSVs into per-launch HBM bytes.  Expects
    {pmc_dir}/step_FETCH_SIZE, step_WRITE_SIZE (bench.py runs) and
    copy_FETCH_SIZE, copy_WRITE_SIZE (bench.py --copy-calibration 1024)."""
    import csv
    import glob
    from collections import defaultdict

    def load(tag):
        """Mean counter bytes per launch of each kind, and the CLT-k select
        stage's bytes of each exchange in dispatch order."""
        files = glob.glob(os.path.join(pmc_dir, tag, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {os.path.join(pmc_dir, tag)}")
        rows = []
        for path in files:
            with open(path) as f:
                rows += [r for r in csv.DictReader(f)]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        total, launches, exchanges = defaultdict(float), defaultdict(int), []
        for r in rows:
            k = kind_of(r["Kernel_Name"])
            if k is None:
                continue
            b = float(r["Counter_Value"]) * 1024.0   # KiB -> bytes
            total[k] += b
            launches[k] += 1
            if "topk_reset" in r["Kernel_Name"]:
                exchanges.append(0.0)
            if k == "cltk_select" and exchanges:
                exchanges[-1] += b
        if exchanges:
            launches["cltk_select"] = len(exchanges)   # one select stage per exchange
        return {k: total[k] / launches[k] for k in total}, exchanges

    copy_bytes = 1024 << 20
    fetch_factor = copy_bytes / load("copy_FETCH_SIZE")[0]["copy"]
    write_factor = copy_bytes / load("copy_WRITE_SIZE")[0]["copy"]
    (fetch, fetch_x), (write, write_x) = load("step_FETCH_SIZE"), load("step_WRITE_SIZE")
    per = {k: round(fetch[k] * fetch_factor + write.get(k, 0.0) * write_factor)
           for k in fetch if k != "copy"}
    per_exchange = [round(f * fetch_factor + w * write_factor) for f, w in zip(fetch_x, write_x)]
    return {"workload": workload, "sources_sha256": {s: sha256_of(s) for s in SOURCES},
            "fetch_factor": fetch_factor, "write_factor": write_factor,
            "copy_calibration_bytes": copy_bytes, "per_launch_bytes": per,
            "cltk_select_bytes_per_exchange": per_exchange,
            "per_launch_fetch_bytes": {k: round(fetch[k] * fetch_factor) for k in per},
            "per_launch_write_bytes": {k: round(write.get(k, 0.0) * write_factor) for k in per}}


def host_copy(t):
    """The bits of a device tensor in a new host array (bf16 as uint16
    patterns, int64 words as uint64), through a preallocated pageable buffer."""
    import numpy as np
    import torch
    bits = {torch.float32: (torch.float32, np.float32, np.float32),
            torch.bfloat16: (torch.int16, np.int16, np.uint16),
            torch.int64: (torch.int64, np.int64, np.uint64)}[t.dtype]
    a = np.empty(tuple(t.shape), bits[2])
    torch.from_numpy(a.view(bits[1])).copy_(t.view(bits[0]))
    return a


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def server_pieces(n: int, chunks: int) -> int:
    """Server scales of an n-element tensor with the server split `chunks` ways
    (whole 8192-element blocks per chunk)."""
    blocks = -(-n // 8192)
    return -(-n // (8192 * -(-blocks // chunks)))


def cpu_baseline(wl, state, grads, server_chunks: int = 1, trust_wd=None, repeats: int = 5) -> dict:
    """The C++ oracle (oracle/onebit_ref.cpp) as it stands, one compression
    step over the whole tensor list on host copies of the benchmark's state
    and one gradient set: first on one core (the calling thread pinned to the
    first core it may run on), then `repeats` times from a pool of the host's
    cores (at most 16 threads, one GPU's share; one tensor per call, largest
    first), the median reported.  Each run continues the previous one's state
    in place, as consecutive steps would.  Copies to the host are outside the
    clocks."""
    import numpy as np
    import oracle.ref as ref
    from concurrent.futures import ThreadPoolExecutor
    from synth.workloads import padded_layout
    lib = ref.load()
    del lib
    off, N = padded_layout(wl.numel)
    W, T = wl.workers, wl.num_tensors
    st = {k: host_copy(state[k]) for k in ("p", "m", "v", "err_s", "err_w")}
    g = host_copy(grads)
    pieces = [server_pieces(n, server_chunks) for n in wl.numel]
    pbase = np.concatenate([[0], np.cumsum(pieces)]).astype(np.int64)
    packed_w = np.zeros((W, N // 64), np.uint64)
    scale_w = np.zeros((W, T), np.float32)
    packed_s = np.zeros(N // 64, np.uint64)
    scale_s = np.zeros(int(pbase[-1]), np.float32)

    def run(t: int) -> None:
        ref.compression_step_in_place(off[t], wl.numel[t], t, g, st["p"], st["m"], st["v"], st["err_s"],
                                      st["err_w"], packed_w, scale_w, packed_s, scale_s[pbase[t]:pbase[t + 1]],
                                      wl.beta1, wl.lr, wl.eps, server_chunks=server_chunks, trust_wd=trust_wd)

    order = sorted(range(T), key=lambda t: -wl.numel[t])
    n_total = sum(wl.numel)
    allowed = sorted(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {allowed[0]})          # this thread only: one core
    try:
        t0 = time.perf_counter()
        for t in order:
            run(t)
        dt1 = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, set(allowed))
    threads = max(1, min(16, len(allowed)))
    runs = []
    with ThreadPoolExecutor(max_workers=threads) as pool:
        for _ in range(repeats):
            t0 = time.perf_counter()
            list(pool.map(run, order))
            runs.append(time.perf_counter() - t0)
    med = sorted(runs)[len(runs) // 2]
    b_alg = step_bytes_per_element(wl)
    cpu = cpu_model()
    return {"value": n_total / dt1, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"the C++ oracle, one step over the whole list ({T} tensors, {n_total} elements, "
                      f"W={W}), single-threaded and pinned to one core of {cpu}: {dt1:.1f} s",
            "seconds": round(dt1, 3), "hbm_gbps_algorithmic": round(b_alg * n_total / dt1 / 1e9, 3),
            "host_nproc": os.cpu_count(), "host_cores_allowed": len(allowed), "cpu_model": cpu,
            "all_cores": {"value": n_total / med, "unit": "elements/s", "cores": threads, "repeats": repeats,
                          "seconds_median": round(med, 3), "seconds_min": round(min(runs), 3),
                          "seconds_max": round(max(runs), 3),
                          "hbm_gbps_algorithmic": round(b_alg * n_total / med / 1e9, 2),
                          "sample": f"the same step over the whole list, {threads} threads, one tensor per "
                                    f"call; median of {repeats} runs"}}


def time_form(form, wl, ctx, grads, steps, warmup, stream, repeats):
    """Warmup, then `repeats` timed runs of exactly `steps` steps each of one
    state form, continuing from a fresh state.  Returns ([seconds per run],
    {kernel: (total ms, launches)} over every timed run, final state)."""
    import torch
    from synth import init_state
    st = init_state(wl, "cuda")
    bufs = ctx.alloc("cuda")
    sets = len(grads)

    def step(k: int) -> None:
        if form == "residual":
            ctx.step_residual(k == 0, grads[k % sets], st["m"], st["v"], st["p"], st["err_w"],
                              st["err_s"], bufs["packed_w"], bufs["scale_w"], bufs["packed_s"],
                              bufs["scale_s"], wl.lr, stream=stream)
        else:
            ctx.step(grads[k % sets], st["m"], st["v"], st["p"], st["err_w"], st["err_s"],
                     bufs["packed_w"], bufs["scale_w"], bufs["packed_s"], bufs["scale_s"], wl.lr,
                     stream=stream)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    ctx.profile(True)
    ctx.profile_read(reset=True)
    runs, k0 = [], warmup
    for _ in range(repeats):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            step(k0 + k)
        torch.cuda.synchronize()
        runs.append(time.perf_counter() - t0)
        k0 += steps
    kernels = ctx.profile_read(reset=True)
    ctx.profile(False)
    return runs, kernels, st


def time_noalloc(wl, ctx, grads, steps, warmup, stream, repeats):
    """The residual form through ob_step_residual_noalloc (the same kernels with
    their scratch in the library's static buffer; it records no kernel events),
    timed like time_form.  None when the list needs more than that buffer."""
    import torch
    from error_compensated_bit_02_amd.binding import OB_ERR_SCRATCH, OneBitError
    from synth import init_state
    st = init_state(wl, "cuda")
    bufs = ctx.alloc("cuda")
    sets = len(grads)

    def step(k: int) -> None:
        ctx.step_residual(k == 0, grads[k % sets], st["m"], st["v"], st["p"], st["err_w"], st["err_s"],
                          bufs["packed_w"], bufs["scale_w"], bufs["packed_s"], bufs["scale_s"], wl.lr,
                          stream=stream, noalloc=True)

    try:
        step(0)
    except OneBitError as e:
        if e.status == OB_ERR_SCRATCH:
            return None
        raise
    for k in range(1, warmup):
        step(k)
    torch.cuda.synchronize()
    runs, k0 = [], warmup
    for _ in range(repeats):
        t0 = time.perf_counter()
        for k in range(steps):
            step(k0 + k)
        torch.cuda.synchronize()
        runs.append(time.perf_counter() - t0)
        k0 += steps
    del st, bufs
    med = sorted(runs)[len(runs) // 2]
    return {"ms_per_step": round(med * 1e3 / steps, 4), "ms_per_step_min": round(min(runs) * 1e3 / steps, 4),
            "ms_per_step_max": round(max(runs) * 1e3 / steps, 4), "repeats": repeats}


def time_cltk(wl, ctx, grads, density, steps, warmup, stream):
    """Warmup, then `steps` timed exchanges of the cyclic local top-k codec
    (the leader cycles with the step).  Returns (seconds, kernels)."""
    import torch
    from synth.workloads import padded_layout
    ctx.cltk_configure(density)
    _, N = padded_layout(wl.numel)
    memory = torch.zeros(wl.workers, N, dtype=torch.float32, device="cuda")
    index = torch.empty(ctx.K, dtype=torch.int32, device="cuda")
    values = torch.empty(wl.workers, ctx.K, dtype=torch.float32, device="cuda")
    average = torch.empty(ctx.K, dtype=torch.float32, device="cuda")
    sets = len(grads)
    for k in range(warmup):
        ctx.cltk_step(k, grads[k % sets], memory, index, values, average, stream=stream)
    torch.cuda.synchronize()
    ctx.profile(True)
    ctx.profile_read(reset=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ctx.cltk_step(warmup + k, grads[(warmup + k) % sets], memory, index, values, average,
                      stream=stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kernels = ctx.profile_read(reset=True)
    ctx.profile(False)
    del memory, index, values, average
    return dt, kernels


def time_warmup_phase(wl, ctx, grads, steps, warmup, stream, beta2=0.999, lr=1e-3):
    """Warmup, then `steps` timed steps of the uncompressed Adam warmup phase
    (ob_warmup_step) from a fresh state.  Returns (seconds, kernels)."""
    import torch
    from synth import init_state
    st = init_state(wl, "cuda")
    sets = len(grads)
    for k in range(warmup):
        ctx.warmup_step(grads[k % sets], st["m"], st["v"], st["p"], beta2, lr, stream=stream)
    torch.cuda.synchronize()
    ctx.profile(True)
    ctx.profile_read(reset=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ctx.warmup_step(grads[(warmup + k) % sets], st["m"], st["v"], st["p"], beta2, lr, stream=stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kernels = ctx.profile_read(reset=True)
    ctx.profile(False)
    del st
    return dt, kernels


def summarize_warmup(wl, n_elem, steps, dt, kernels, workload):
    """The warmup kernel reads g*W, m, v, p and writes m, v, p: 24 + g*W B/element."""
    b = 24.0 + grad_bytes(wl) * wl.workers
    ms, n = kernels["warmup"]
    avg = ms / n
    achieved = b * n_elem / (avg * 1e-3) / 1e9
    traffic = counter_traffic(workload, "warmup")
    return {"ms_per_step": dt * 1e3 / steps, "elements_per_s": n_elem * steps / dt,
            "roofline": {"bound": "hbm", "kernel": "warmup", "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                         "traffic": None if traffic is None else round(traffic),
                         "bytes_per_element": b, "avg_ms": round(avg, 4)}}


def summarize_cltk(wl, n_elem, steps, dt, kernels, density, workload):
    kb = cltk_bytes_per_element(wl, density)
    per = {k: (kernels[k][0] / kernels[k][1] if kernels[k][1] else 0.0) for k in kb}
    dom = max(kb, key=lambda k: per[k])
    achieved = kb[dom] * n_elem / (per[dom] * 1e-3) / 1e9
    ms = dt * 1e3 / steps
    total = sum(kb.values())
    traffic = counter_traffic(workload, dom)
    return {
        "density": density, "ms_per_exchange": ms, "elements_per_s": n_elem * steps / dt,
        "exchange_hbm_gbps_algorithmic": round(total * n_elem / (ms * 1e-3) / 1e9, 1),
        "exchange_bytes_per_element": total,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "bytes_per_element": kb[dom], "avg_ms": round(per[dom], 4)},
        "kernels": {k: {"avg_ms": round(per[k], 4), "launches": kernels[k][1]} for k in kb},
    }


def copy_ceiling(gib: int = 4, reps: int = 5) -> dict:
    """A plain device-to-device copy of `gib` GiB, timed with events on torch's
    stream: the streaming rate a read+write kernel can reach on this device."""
    import torch
    n = gib << 28                      # fp32 elements
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    del src, dst
    best = sorted(ms)[len(ms) // 2]
    return {"gbps": round(2 * 4 * n / (best * 1e-3) / 1e9, 1), "bytes_copied": 4 * n,
            "median_ms": round(best, 4), "reps": reps, "frac": round(2 * 4 * n / (best * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def add_ceiling(gib: int = 4, reps: int = 5) -> dict:
    """An in-place add e += g over two `gib` GiB arrays (two reads and one
    write per element, the worker pass's mix), timed like copy_ceiling."""
    import torch
    n = gib << 28
    g = torch.ones(n, device="cuda")
    e = torch.zeros(n, device="cuda")
    e.add_(g)
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        e.add_(g)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    del g, e
    best = sorted(ms)[len(ms) // 2]
    gbps = 3 * 4 * n / (best * 1e-3) / 1e9
    return {"gbps": round(gbps, 1), "bytes_moved": 3 * 4 * n, "median_ms": round(best, 4), "reps": reps,
            "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def step_counter_gbps(workload, per_kernel, ms_step, steps):
    """Whole-step HBM GB/s from the counter bytes of every kernel the step
    launched, or None when some kernel has no current counter figure."""
    total = 0.0
    for k, v in per_kernel.items():
        if not v["launches"]:
            continue
        b = counter_traffic(workload, k)
        if b is None:
            return None
        total += b * v["launches"] / steps
    return round(total / (ms_step * 1e-3) / 1e9, 1)


def summarize(wl, n_elem, steps, runs, kernels, workload):
    """The step's figures from `runs` (seconds per timed run of `steps`
    steps; the median is reported) and the kernels' event times over all runs."""
    dt = sorted(runs)[len(runs) // 2]
    ms_step = dt * 1e3 / steps
    b_alg = step_bytes_per_element(wl)
    step_gbps = b_alg * n_elem / (ms_step * 1e-3) / 1e9
    per_kernel = {k: {"avg_ms": (ms / n if n else 0.0), "launches": n} for k, (ms, n) in kernels.items()}
    kb = kernel_bytes_per_element(wl)
    # bytes the form's own kernels move per element per step, each operand once per kernel
    launches_per_step = {k: v["launches"] / (steps * len(runs)) for k, v in per_kernel.items()}
    b_moved = sum(kb[k] * launches_per_step[k] for k in kb if per_kernel[k]["launches"])
    moved_gbps = b_moved * n_elem / (ms_step * 1e-3) / 1e9
    dom = max((k for k in kb if per_kernel[k]["launches"]), key=lambda k: per_kernel[k]["avg_ms"])
    dom_ms = per_kernel[dom]["avg_ms"]
    achieved = kb[dom] * n_elem / (dom_ms * 1e-3) / 1e9
    traffic = counter_traffic(workload, dom)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": None if traffic is None else round(traffic),
                "algorithmic_bytes": round(kb[dom] * n_elem),
                "bytes_per_element": kb[dom], "avg_ms": round(dom_ms, 4)}
    counter_gbps = step_counter_gbps(workload, per_kernel, ms_step, steps * len(runs))
    return {
        "ms_per_step": ms_step,
        "value": n_elem / (ms_step * 1e-3),
        "repeats": len(runs),
        "ms_per_step_min": round(min(runs) * 1e3 / steps, 4),
        "ms_per_step_max": round(max(runs) * 1e3 / steps, 4),
        "step_hbm_gbps_algorithmic": round(step_gbps, 1),
        "step_hbm_gbps_counter": counter_gbps,
        "step_counter_frac_of_peak": None if counter_gbps is None else round(counter_gbps / HBM_PEAK_GBPS, 4),
        "step_frac_of_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "step_fraction": {"by_method_bytes": round(step_gbps / HBM_PEAK_GBPS, 4),
                          "method_bytes_per_element": b_alg,
                          "by_bytes_moved": round(moved_gbps / HBM_PEAK_GBPS, 4),
                          "moved_bytes_per_element": round(b_moved, 4),
                          "by_counters": None if counter_gbps is None else round(counter_gbps / HBM_PEAK_GBPS, 4)},
        "roofline": roofline,
        "kernels": {k: {"avg_ms": round(v["avg_ms"], 4), "launches": v["launches"]}
                    for k, v in per_kernel.items() if v["launches"]},
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bert_large")
    ap.add_argument("--form", choices=("both", "residual", "strict"), default="both",
                    help="state form between steps; both forms give bit-identical trajectories. "
                         "'both' times the residual form (the headline) and the strict form")
    ap.add_argument("--grad-sets", type=int, default=4, help="distinct gradient sets cycled")
    ap.add_argument("--trust-ratio", type=float, default=None, metavar="WD",
                    help="layer-wise trust-ratio update with weight decay WD")
    ap.add_argument("--server-chunks", type=int, default=1,
                    help="partitioned server: one server scale per tensor chunk (1 = per tensor)")
    ap.add_argument("--no-warmup-phase", action="store_true",
                    help="skip timing the uncompressed Adam warmup phase")
    ap.add_argument("--cltk-density", type=float, default=0.01,
                    help="also time the cyclic local top-k exchange keeping this fraction of "
                         "each tensor (0 = skip)")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed runs of --steps steps each per state form; the median is reported")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR", default=None,
                    help="write profiles/<workload>_hbm_counters.json from rocprofv3 --pmc runs "
                         "under PMC_DIR (no GPU needed), then exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 launches) for calibrating "
                         "HBM byte counters, then exit")
    args = ap.parse_args()

    if args.summarize_counters:
        data = summarize_counters(args.summarize_counters, args.workload)
        out = os.path.join(ROOT, "profiles", f"{args.workload}_hbm_counters.json")
        with open(out, "w") as f:
            json.dump(data, f, indent=1)
        log(f"bench: wrote {out}")
        for k, v in sorted(data["per_launch_bytes"].items()):
            log(f"  {k:24s} {v / 1e9:9.3f} GB per launch")
        return 0
    if args.gpus != 1:
        log(f"bench.py: --gpus {args.gpus} is not supported; this library runs on one GPU "
            f"(all W simulated workers share one GPU's HBM)")
        return 2

    import torch
    from error_compensated_bit_02_amd import OneBitAdam
    from synth import WORKLOADS, grads_for_step

    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        return 1
    if args.copy_calibration:
        n = args.copy_calibration << 18            # fp32 elements in MIB MiB
        src = torch.ones(n, device="cuda")
        dst = torch.empty(n, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copied {args.copy_calibration} MiB three times "
            f"(each launch reads and writes {args.copy_calibration} MiB)")
        return 0
    wl = WORKLOADS[args.workload]
    n_elem = sum(wl.numel)
    log(f"bench: {wl.name}: {wl.num_tensors} tensors, {n_elem} elements, W={wl.workers}, "
        f"grads {wl.grad_dtype}; steps={args.steps} warmup={args.warmup}")
    ctx = OneBitAdam(wl.numel, wl.workers, wl.grad_dtype, wl.beta1, wl.eps)
    if args.server_chunks != 1:
        ctx.set_server_chunks(args.server_chunks)
    if args.trust_ratio is not None:
        ctx.set_trust_ratio(True, args.trust_ratio)
    sets = max(1, min(args.grad_sets, args.steps + args.warmup))
    grads = [grads_for_step(wl, k, "cuda") for k in range(sets)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    forms = ["residual", "strict"] if args.form == "both" else [args.form]
    results, last_state = {}, None
    for form in forms:
        last_state = None
        torch.cuda.empty_cache()
        runs, kernels, last_state = time_form(form, wl, ctx, grads, args.steps, args.warmup, stream,
                                              max(1, args.repeats))
        results[form] = summarize(wl, n_elem, args.steps, runs, kernels, wl.name)
        r = results[form]
        log(f"bench: {form}: {r['ms_per_step']:.3f} ms/step (median of {r['repeats']} runs of "
            f"{args.steps} steps; {r['ms_per_step_min']:.3f}-{r['ms_per_step_max']:.3f}), "
            f"{100 * r['step_fraction']['by_method_bytes']:.1f}% of peak by the method's bytes, "
            f"{100 * r['step_fraction']['by_bytes_moved']:.1f}% by the bytes moved")

    noalloc = None
    if "residual" in forms:
        torch.cuda.empty_cache()
        noalloc = time_noalloc(wl, ctx, grads, args.steps, max(1, args.warmup), stream, max(1, args.repeats))
        if noalloc:
            log(f"bench: residual through ob_step_residual_noalloc: {noalloc['ms_per_step']:.3f} ms/step")

    warm = None
    if not args.no_warmup_phase:
        torch.cuda.empty_cache()
        dt, kernels = time_warmup_phase(wl, ctx, grads, args.steps, args.warmup, stream)
        warm = summarize_warmup(wl, n_elem, args.steps, dt, kernels, wl.name)
        log(f"bench: warmup-phase Adam: {warm['ms_per_step']:.3f} ms/step, "
            f"{100 * warm['roofline']['frac']:.1f}% of peak")

    cltk = None
    if args.cltk_density > 0:
        torch.cuda.empty_cache()
        dt, kernels = time_cltk(wl, ctx, grads, args.cltk_density, args.steps, args.warmup, stream)
        cltk = summarize_cltk(wl, n_elem, args.steps, dt, kernels, args.cltk_density, wl.name)
        log(f"bench: cltk density {args.cltk_density}: {cltk['ms_per_exchange']:.3f} ms/exchange, "
            f"{cltk['roofline']['kernel']} at {100 * cltk['roofline']['frac']:.1f}% of peak")

    head = results[forms[0]]
    result = {
        "metric": METRIC, "value": head["value"], "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "repeats": head["repeats"], "ms_per_step_min": head["ms_per_step_min"],
        "ms_per_step_max": head["ms_per_step_max"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "tensors": wl.num_tensors, "elements": n_elem,
                   "workers": wl.workers, "grad_dtype": wl.grad_dtype,
                   "grad_sets": sets, "state_form": forms[0], "server_chunks": args.server_chunks,
                   "trust_ratio_weight_decay": args.trust_ratio},
        "step_hbm_gbps_algorithmic": head["step_hbm_gbps_algorithmic"],
        "step_frac_of_peak": head["step_frac_of_peak"],
        "step_hbm_gbps_counter": head["step_hbm_gbps_counter"],
        "step_counter_frac_of_peak": head["step_counter_frac_of_peak"],
        "step_bytes_per_element": step_bytes_per_element(wl),
        "step_fraction": head["step_fraction"],
        "worker_elements_per_s": head["value"] * wl.workers,
        "roofline": head["roofline"],
        "kernels": head["kernels"],
    }
    if "strict" in results and forms[0] != "strict":
        result["strict_form"] = results["strict"]
    result["residual_noalloc"] = noalloc
    result["warmup_phase"] = warm
    result["cltk"] = cltk
    torch.cuda.empty_cache()
    result["copy_ceiling"] = copy_ceiling()
    result["add_ceiling"] = add_ceiling()
    log(f"bench: streaming ceilings: copy {result['copy_ceiling']['gbps']:.0f} GB/s, in-place add "
        f"{result['add_ceiling']['gbps']:.0f} GB/s; {head['roofline']['kernel']} at "
        f"{head['roofline']['achieved'] / result['add_ceiling']['gbps']:.1%} of the add")
    result["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host (cpu baseline)")
        result["cpu_baseline"] = cpu_baseline(wl, last_state, grads[0], args.server_chunks, args.trust_ratio)
    ctx.close()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
