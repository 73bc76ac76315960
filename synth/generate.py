"""Seeded generators for the synthetic workloads.

Every draw comes from a torch generator seeded from (workload seed, stream
tag, step), so a run is reproducible on the device it was generated on.  The
oracle and the HIP path never generate their own inputs: a test draws them
once here and hands copies to both sides.

Recipes (standard deviations throughout, one fresh draw per step and worker):
  gradients   g_w ~ N(0, g_sigma); with g_shared = r the draw is
              sqrt(r) * c + sqrt(1 - r) * u_w, c and u_w independent
              N(0, g_sigma), so workers correlate with coefficient r;
              bf16 workloads round the fp32 draw to bf16 (round to nearest even)
  parameters  p ~ N(0, p_sigma)
  variance    "sq_normal": v = |N(0, v_a)|^2 + v_b ; "lognormal": v = exp(N(v_a, v_b))
  momentum, worker and server error buffers start at zero.
Padding elements between tensors are zero in every buffer.
"""
from __future__ import annotations

import hashlib
import math
from typing import Dict, Optional

import numpy as np
import torch

from .workloads import Workload, padded_layout


def _seed(seed: int, tag: str, step: int = 0) -> int:
    h = hashlib.sha256(f"{seed}/{tag}/{step}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int, tag: str, step: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tag, step))
    return g


def _zero_padding(buf: torch.Tensor, wl: Workload) -> None:
    off, _ = padded_layout(wl.numel)
    for t, n in enumerate(wl.numel):
        if off[t] + n < off[t + 1]:
            buf[..., off[t] + n: off[t + 1]] = 0


def init_state(wl: Workload, device="cpu", seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Flat fp32 state buffers: p, m, v, err_s of [N] and err_w of [W][N]."""
    seed = wl.seed if seed is None else seed
    _, n_pad = padded_layout(wl.numel)
    dev = torch.device(device)
    p = torch.randn(n_pad, generator=_gen(dev, seed, "params"), device=dev, dtype=torch.float32)
    p.mul_(wl.p_sigma)
    v = torch.randn(n_pad, generator=_gen(dev, seed, "variance"), device=dev, dtype=torch.float32)
    if wl.v_kind == "sq_normal":
        v.mul_(wl.v_a).abs_().square_().add_(wl.v_b)
    elif wl.v_kind == "lognormal":
        v.mul_(wl.v_b).add_(wl.v_a).exp_()
    else:
        raise ValueError(wl.v_kind)
    _zero_padding(p, wl)
    _zero_padding(v, wl)
    return {
        "p": p,
        "m": torch.zeros(n_pad, device=dev, dtype=torch.float32),
        "v": v,
        "err_s": torch.zeros(n_pad, device=dev, dtype=torch.float32),
        "err_w": torch.zeros(wl.workers, n_pad, device=dev, dtype=torch.float32),
    }


def grads_for_step(wl: Workload, step: int, device="cpu", seed: Optional[int] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-worker gradients [W][N] for one step (fp32, or bf16 for bf16 workloads)."""
    seed = wl.seed if seed is None else seed
    _, n_pad = padded_layout(wl.numel)
    dev = torch.device(device)
    dtype = torch.bfloat16 if wl.grad_dtype == "bf16" else torch.float32
    if out is None:
        out = torch.empty(wl.workers, n_pad, device=dev, dtype=dtype)
    gen = _gen(dev, seed, "grads", step)
    if dtype == torch.float32:
        torch.randn(out.shape, generator=gen, device=dev, dtype=torch.float32, out=out)
        if wl.g_shared > 0.0:
            shared = torch.randn(n_pad, generator=gen, device=dev, dtype=torch.float32)
            out.mul_(math.sqrt(1.0 - wl.g_shared)).add_(shared, alpha=math.sqrt(wl.g_shared))
            del shared
        out.mul_(wl.g_sigma)
    else:
        if wl.g_shared > 0.0:
            raise NotImplementedError("shared gradient component with bf16 gradients")
        for w in range(wl.workers):  # one worker at a time keeps the fp32 temporary small
            tmp = torch.randn(n_pad, generator=gen, device=dev, dtype=torch.float32)
            tmp.mul_(wl.g_sigma)
            out[w].copy_(tmp)   # fp32 -> bf16, round to nearest even
            del tmp
    _zero_padding(out, wl)
    return out


def host_slice(t: torch.Tensor, lo: int, hi: int) -> np.ndarray:
    """Copy t[..., lo:hi] to a host numpy array; bf16 comes back as its uint16 bit patterns."""
    s = t[..., lo:hi]
    if s.dtype == torch.bfloat16:
        return s.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    if s.dtype == torch.int64:
        return s.contiguous().cpu().numpy().view(np.uint64)
    return s.contiguous().cpu().numpy()
