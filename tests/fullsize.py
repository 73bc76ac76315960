"""Every element of a full-size tensor list, every step, against the C++ oracle.

The device runs the whole list in the benchmark's launch configuration; the
C++ oracle (oracle/onebit_ref.cpp, pinned on the CPU by
tests/test_oracle_cpp.py) runs the same step on host copies of the same
inputs, in place on flat host buffers in the device layout, one tensor per
call from a pool of host threads, carrying its own state from step to step.
After every step each tensor's sign words, scales, errors, momentum and
parameters are compared bit for bit (a bit-identical float is within every
tolerance of the contract).

Device outputs come to the host in host arrays allocated once per list (about
16 GB/s on MI355X against under 4 GB/s for a fresh pageable copy), and the
oracle writes its state in place, which is what lets whole trajectories of the
largest lists run in minutes.
"""
from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np
import torch

import oracle.ref as ref
from harness import Run, log
from synth import grads_for_step


def threads() -> int:
    """Host threads for the oracle: the host's cores, at most 16 (one GPU's share)."""
    return max(1, min(16, os.cpu_count() or 1))


_NP = {torch.float32: np.float32, torch.bfloat16: np.uint16, torch.int64: np.uint64, torch.int32: np.int32}
_BITS = {torch.float32: torch.float32, torch.bfloat16: torch.int16, torch.int64: torch.int64,
         torch.int32: torch.int32}


def host_array(t: torch.Tensor) -> np.ndarray:
    """An uninitialised host array for the bits of device tensor t: bf16 as
    uint16 patterns, int64 words as uint64."""
    return np.empty(tuple(t.shape), _NP[t.dtype])


def copy_to_host(dst: np.ndarray, src: torch.Tensor) -> None:
    """Copies the bits of device tensor src into host array dst (same shape)."""
    bits = _BITS[src.dtype]
    torch.from_numpy(dst.view(np.dtype(str(bits).replace("torch.", "")))).copy_(src.view(bits))


def _same(a: np.ndarray, b: np.ndarray) -> bool:
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)


class Mirror:
    """Host arrays shaped like a set of device buffers, allocated once and
    reused every step.  Copies into these preallocated pageable arrays run at
    about 16 GB/s on MI355X (a fresh pageable copy runs under 4 GB/s, and
    pinned buffers of the largest lists' size exceed what a process may pin)."""

    def __init__(self, like: Dict[str, torch.Tensor]):
        self.view = {k: host_array(v) for k, v in like.items()}

    def pull(self, dev: Dict[str, torch.Tensor]) -> None:
        for k, v in dev.items():
            copy_to_host(self.view[k], v)


class FlatOracle:
    """The C++ oracle's state for a whole padded flat list, in host memory."""

    def __init__(self, run: Run, trust_wd: Optional[float]):
        wl = run.wl
        self.wl, self.run, self.trust_wd = wl, run, trust_wd
        self.state = {}
        for k in ("p", "m", "v", "err_s", "err_w"):
            self.state[k] = host_array(run.state[k])
            copy_to_host(self.state[k], run.state[k])
        W, N, T = wl.workers, run.N, wl.num_tensors
        self.packed_w = np.zeros((W, N // 64), np.uint64)
        self.scale_w = np.zeros((W, T), np.float32)
        self.packed_s = np.zeros(N // 64, np.uint64)
        self.scale_s = np.zeros(run.piece_base[-1], np.float32)

    def _pairs(self, t: int, got: Dict[str, np.ndarray]):
        wl, run, st = self.wl, self.run, self.state
        off, pb = run.off, run.piece_base
        n = wl.numel[t]
        lo, hi = off[t], off[t] + n
        wlo, whi = lo // 64, lo // 64 + (n + 63) // 64
        return (("packed_w", self.packed_w[:, wlo:whi], got["packed_w"][:, wlo:whi]),
                ("scale_w", self.scale_w[:, t], got["scale_w"][:, t]),
                ("packed_s", self.packed_s[wlo:whi], got["packed_s"][wlo:whi]),
                ("scale_s", self.scale_s[pb[t]:pb[t + 1]], got["scale_s"][pb[t]:pb[t + 1]]),
                ("p", st["p"][lo:hi], got["p"][lo:hi]), ("m", st["m"][lo:hi], got["m"][lo:hi]),
                ("err_s", st["err_s"][lo:hi], got["err_s"][lo:hi]),
                ("err_w", st["err_w"][:, lo:hi], got["err_w"][:, lo:hi]))

    def _counts(self, t: int):
        n, W, pb = self.wl.numel[t], self.wl.workers, self.run.piece_base
        return (W + 1) * ((n + 63) // 64), (3 + W) * n + W + (pb[t + 1] - pb[t])

    def step(self, g: np.ndarray, got: Dict[str, np.ndarray], pool: ThreadPoolExecutor):
        """Runs the oracle's step on every tensor (largest first), in place, and
        compares each tensor with the device's outputs `got` as soon as it is
        done.  Returns [(tensor name, [differing buffers])] and the counts
        compared."""
        wl, run, st = self.wl, self.run, self.state
        off, pb = run.off, run.piece_base

        def one(t: int):
            ref.compression_step_in_place(off[t], wl.numel[t], t, g, st["p"], st["m"], st["v"], st["err_s"],
                                          st["err_w"], self.packed_w, self.scale_w, self.packed_s,
                                          self.scale_s[pb[t]:pb[t + 1]], wl.beta1, wl.lr, wl.eps,
                                          server_chunks=run.server_chunks, trust_wd=self.trust_wd)
            return (t, [key for key, mine, dev in self._pairs(t, got) if not _same(mine, dev)]) + self._counts(t)

        return self._collect(pool.map(one, self._order()))

    def compare(self, got: Dict[str, np.ndarray], pool: ThreadPoolExecutor):
        """Compares the device's outputs `got` with the oracle's state as it is
        (after step()), tensor by tensor."""
        def one(t: int):
            return (t, [key for key, mine, dev in self._pairs(t, got) if not _same(mine, dev)]) + self._counts(t)

        return self._collect(pool.map(one, self._order()))

    def _order(self):
        return sorted(range(self.wl.num_tensors), key=lambda t: -self.wl.numel[t])

    def _collect(self, results):
        results = list(results)
        failed = [(self.wl.tensors[t][0], bad) for t, bad, _, _ in results if bad]
        return failed, sum(r[2] for r in results), sum(r[3] for r in results)


def trajectory(wl, forms, steps: int, server_chunks: int = 1, trust_wd: Optional[float] = None) -> None:
    """`steps` steps of each state form in `forms` ("residual": ob_step_residual,
    its state materialized after every step; "strict": ob_step), run side by
    side from the same initial state on the same gradients, every element of
    each compared after every step with one C++ oracle trajectory."""
    nthreads = threads()
    log(f"{wl.name}: {steps} steps of the {' and '.join(forms)} form(s) (server chunks {server_chunks}, "
        f"trust-ratio weight decay {trust_wd}), every element against the C++ oracle ({nthreads} threads)")
    ref.load()
    t0 = time.time()
    runs = {}
    for form in forms:
        runs[form] = Run(wl, server_chunks=server_chunks, trust_wd=trust_wd)
    oracle = FlatOracle(runs[forms[0]], trust_wd)
    gbuf = grads_for_step(wl, 0, "cuda")

    def outputs(run: Run) -> Dict[str, torch.Tensor]:
        return {"p": run.state["p"], "m": run.state["m"], "err_s": run.state["err_s"],
                "err_w": run.state["err_w"], **{k: run.bufs[k] for k in ("packed_w", "scale_w", "packed_s", "scale_s")}}

    mirror = Mirror({"grads": gbuf, **outputs(runs[forms[0]])})
    log(f"  {wl.name}: set up in {time.time() - t0:.1f}s")
    words = floats = 0
    with ThreadPoolExecutor(max_workers=nthreads) as pool:
        for k in range(steps):
            t0 = time.time()
            if k:
                gbuf = grads_for_step(wl, k, "cuda", out=gbuf)
            mirror.pull({"grads": gbuf})
            g = mirror.view["grads"]   # the forms' pulls below leave the gradients in place
            for i, form in enumerate(forms):
                run = runs[form]
                view = None
                if form == "residual":
                    run.step_residual(gbuf, first=(k == 0))
                    view = run.materialized()
                    dev = {**outputs(run), "m": view["m"], "err_s": view["err_s"], "err_w": view["err_w"]}
                else:
                    run.step(gbuf)
                    dev = outputs(run)
                mirror.pull(dev)
                del view, dev
                if i == 0:
                    failed, nw, nf = oracle.step(g, mirror.view, pool)
                else:
                    failed, nw, nf = oracle.compare(mirror.view, pool)
                words += nw
                floats += nf
                assert not failed, f"{wl.name} {form} step {k}: {len(failed)} tensors differ, first {failed[:3]}"
            log(f"  {wl.name} step {k}: {words} sign words and {floats} floats compared "
                f"({' and '.join(forms)}), all bit-identical ({time.time() - t0:.1f}s)")
    for run in runs.values():
        run.ctx.close()
    del runs, oracle, mirror, gbuf
    torch.cuda.empty_cache()
