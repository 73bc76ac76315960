"""Runs the HIP path and the oracle on the same seeded inputs and compares them.

Inputs come from synth (seeded torch generators) and are copied to both
sides; the oracle never sees a value produced by the HIP path except for the
comparison itself.  Tolerances are the contract's: sign words bit-exact;
scales within 1e-5 relative; errors, momentum and parameters within 1e-6
absolute (NaN where the oracle has NaN).  Exact float equality is also
counted and reported, since the design aims at bit-identical floats.
"""
from __future__ import annotations

import sys
import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle.onebit as ob
from synth import host_slice
from synth.workloads import Workload, padded_layout

SCALE_RTOL = 1e-5
STATE_ATOL = 1e-6


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Report:
    exact_floats: int = 0
    total_floats: int = 0
    words: int = 0
    max_state_err: float = 0.0
    max_scale_rel: float = 0.0
    notes: List[str] = field(default_factory=list)


def _u64(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().view(np.uint64)


def _cmp_float(name: str, got: np.ndarray, ref: np.ndarray, rep: Report, atol=None, rtol=None):
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if np.array_equal(got.view(np.uint32), ref.view(np.uint32)):   # bit-identical: within any tolerance
        rep.exact_floats += got.size
        rep.total_floats += got.size
        return
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{name}: NaN positions differ"
    g, r = got[~nan_ref], ref[~nan_ref]
    rep.exact_floats += int(np.sum(g.view(np.uint32) == r.view(np.uint32))) + int(nan_ref.sum())
    rep.total_floats += got.size
    if g.size == 0:
        return
    diff = np.abs(g.astype(np.float64) - r.astype(np.float64))
    if atol is not None:
        worst = float(diff.max())
        rep.max_state_err = max(rep.max_state_err, worst)
        assert worst <= atol, f"{name}: max abs diff {worst:.3e} > {atol}"
    if rtol is not None:
        rel = diff / np.maximum(np.abs(r.astype(np.float64)), 1e-300)
        rel[(diff == 0)] = 0.0
        worst = float(rel.max())
        rep.max_scale_rel = max(rep.max_scale_rel, worst)
        assert worst <= rtol, f"{name}: max rel diff {worst:.3e} > {rtol}"


def _cmp_words(name: str, got: np.ndarray, ref: np.ndarray, rep: Report):
    got = np.asarray(got, np.uint64)
    ref = np.asarray(ref, np.uint64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{name}: {bad.size} sign words differ, first at {bad[0]}"
    rep.words += got.size


class Run:
    """Device buffers for one tensor list plus the library context."""

    def __init__(self, wl: Workload, device="cuda", state: Optional[Dict[str, torch.Tensor]] = None,
                 server_chunks: int = 1, trust_wd: Optional[float] = None):
        from error_compensated_bit_02_amd import OneBitAdam
        from synth import init_state
        self.wl = wl
        self.ctx = OneBitAdam(wl.numel, wl.workers, wl.grad_dtype, wl.beta1, wl.eps)
        self.server_chunks = server_chunks
        if server_chunks != 1:
            self.ctx.set_server_chunks(server_chunks)
        if trust_wd is not None:
            self.ctx.set_trust_ratio(True, trust_wd)
        counts = [len(ob.chunk_bounds(n, server_chunks)) for n in wl.numel]
        self.piece_base = [0]
        for k in counts:
            self.piece_base.append(self.piece_base[-1] + k)
        assert self.ctx.S == self.piece_base[-1]
        self.off, self.N = padded_layout(wl.numel)
        assert self.ctx.offsets == self.off
        self.state = init_state(wl, device) if state is None else state
        self.bufs = self.ctx.alloc(device)

    def step(self, grads: torch.Tensor, lr: Optional[float] = None) -> None:
        s, b = self.state, self.bufs
        self.ctx.step(grads, s["m"], s["v"], s["p"], s["err_w"], s["err_s"], b["packed_w"],
                      b["scale_w"], b["packed_s"], b["scale_s"], self.wl.lr if lr is None else lr)

    def step_split(self, grads: torch.Tensor, lr: Optional[float] = None) -> None:
        """The same step through the three separate entry points."""
        s, b = self.state, self.bufs
        self.ctx.compress_worker(grads, s["m"], s["err_w"], b["packed_w"], b["scale_w"])
        self.ctx.server_reduce(b["packed_w"], b["scale_w"], s["err_s"], b["packed_s"], b["scale_s"])
        self.ctx.apply_update(b["packed_s"], b["scale_s"], s["v"], s["m"], s["p"],
                              self.wl.lr if lr is None else lr)

    def step_residual(self, grads: torch.Tensor, first: bool, lr: Optional[float] = None) -> None:
        """The same step with err_w / err_s kept in residual form."""
        s, b = self.state, self.bufs
        self.ctx.step_residual(first, grads, s["m"], s["v"], s["p"], s["err_w"], s["err_s"],
                               b["packed_w"], b["scale_w"], b["packed_s"], b["scale_s"],
                               self.wl.lr if lr is None else lr)

    def materialized(self) -> Dict[str, torch.Tensor]:
        """Strict-form state of a residual-form run, in fresh zero-filled buffers
        (padding is never written, so it stays zero as in the strict form)."""
        s, b = self.state, self.bufs
        out = {"p": s["p"], "v": s["v"], "err_w": torch.zeros_like(s["err_w"]),
               "err_s": torch.zeros_like(s["err_s"]), "m": torch.zeros_like(s["m"])}
        self.ctx.materialize(s["err_w"], b["scale_w"], s["err_s"], b["scale_s"], out["err_w"],
                             out["err_s"], out["m"])
        return out

    def host_state(self, tensors: Sequence[int]) -> List[ob.TensorState]:
        """Per-tensor host copies (for seeding the oracle with the same initial values)."""
        out = []
        for t in tensors:
            lo, hi = self.off[t], self.off[t] + self.wl.numel[t]
            s = self.state
            out.append(ob.TensorState(host_slice(s["p"], lo, hi), host_slice(s["m"], lo, hi),
                                      host_slice(s["v"], lo, hi), host_slice(s["err_s"], lo, hi),
                                      host_slice(s["err_w"], lo, hi)))
        return out

    def compare(self, t: int, out: ob.StepOutput, rep: Report, what: str,
                state: Optional[Dict[str, torch.Tensor]] = None) -> None:
        """Compare tensor t's device state (default: this run's buffers) and
        messages with one oracle step output."""
        wl, off = self.wl, self.off
        lo, hi = off[t], off[t] + wl.numel[t]
        wlo, whi = off[t] // 64, off[t] // 64 + (wl.numel[t] + 63) // 64
        s, b = (self.state if state is None else state), self.bufs
        ref_w, ref_sw = ob.words_of(out.worker_msgs)
        _cmp_words(f"{what} packed_w", _u64(b["packed_w"][:, wlo:whi]).ravel(), ref_w.ravel(), rep)
        _cmp_words(f"{what} packed_s", _u64(b["packed_s"][wlo:whi]), out.server_msg.words, rep)
        _cmp_float(f"{what} scale_w", b["scale_w"][:, t].cpu().numpy(), ref_sw, rep, rtol=SCALE_RTOL)
        ref_ss = (out.server_msg.scales if isinstance(out.server_msg, ob.ChunkedMessage)
                  else np.array([out.server_msg.scale], np.float32))
        got_ss = b["scale_s"][self.piece_base[t]:self.piece_base[t + 1]].cpu().numpy()
        _cmp_float(f"{what} scale_s", got_ss, ref_ss, rep, rtol=SCALE_RTOL)
        st = out.state
        _cmp_float(f"{what} err_w", host_slice(s["err_w"], lo, hi), st.err_w, rep, atol=STATE_ATOL)
        _cmp_float(f"{what} err_s", host_slice(s["err_s"], lo, hi), st.err_s, rep, atol=STATE_ATOL)
        _cmp_float(f"{what} m", host_slice(s["m"], lo, hi), st.m, rep, atol=STATE_ATOL)
        _cmp_float(f"{what} p", host_slice(s["p"], lo, hi), st.p, rep, atol=STATE_ATOL)


def oracle_step(st, g, wl: Workload, server_chunks: int = 1,
                trust_wd: Optional[float] = None) -> ob.StepOutput:
    scomp = None if server_chunks == 1 else ob.ChunkedOneBitCompressor(server_chunks)
    return ob.compression_step(st, g, wl.beta1, wl.lr, wl.eps, server_comp=scomp,
                               trust_ratio_wd=trust_wd)


def parity_run(wl: Workload, steps: int, tensors: Optional[Sequence[int]] = None,
               grads_fn=None, split: bool = False, device="cuda",
               state: Optional[Dict[str, torch.Tensor]] = None, residual: bool = False,
               server_chunks: int = 1, trust_wd: Optional[float] = None) -> Report:
    """Run `steps` steps on the device and on the oracle for `tensors` (all by
    default), comparing after every step.  grads_fn(step) -> [W][N] device tensor.
    residual=True runs the residual-form step and compares its materialized state."""
    from synth import grads_for_step
    tensors = list(range(wl.num_tensors)) if tensors is None else list(tensors)
    run = Run(wl, device, state, server_chunks=server_chunks, trust_wd=trust_wd)
    ref = run.host_state(tensors)
    rep = Report()
    gbuf = None
    for k in range(steps):
        t0 = time.time()
        if grads_fn is None:
            gbuf = grads_for_step(wl, k, device, out=gbuf)
            g = gbuf
        else:
            g = grads_fn(k)
        host_g = [host_slice(g, run.off[t], run.off[t] + wl.numel[t]) for t in tensors]
        view = None
        if residual:
            run.step_residual(g, first=(k == 0))
            view = run.materialized()
        else:
            (run.step_split if split else run.step)(g)
        torch.cuda.synchronize()
        for i, t in enumerate(tensors):
            out = oracle_step(ref[i], host_g[i], wl, server_chunks, trust_wd)
            run.compare(t, out, rep, f"{wl.name} step {k} tensor {t}", state=view)
            ref[i] = out.state
        log(f"  {wl.name} step {k}: ok ({time.time() - t0:.1f}s, {len(tensors)} tensors)")
    run.ctx.close()
    return rep
