"""Checkpoint and resume: k steps, the resumable state saved to host memory
and to a safetensors file, a fresh context and fresh device buffers loaded
from it, j more steps — bitwise equal to k + j uninterrupted steps, in both
state forms and for the cyclic local top-k codec."""
import os
import tempfile

import pytest
import torch

from harness import Run, log
from synth import grads_for_step
from synth.workloads import padded_layout
from test_parity_gpu import RAGGED, _wl

pytestmark = pytest.mark.gpu

K_STEPS, J_STEPS = 3, 3


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from error_compensated_bit_02_amd import load_library
    load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _resumable(run: Run, residual: bool):
    """The state a later step reads: p, m, v, the error buffers, and in the
    residual form the last step's messages and scales (the momentum and the
    scales of the stored x and z)."""
    keys = {"p": run.state["p"], "m": run.state["m"], "v": run.state["v"],
            "err_w": run.state["err_w"], "err_s": run.state["err_s"]}
    if residual:
        keys.update({k: run.bufs[k] for k in ("packed_w", "scale_w", "packed_s", "scale_s")})
    return keys


def _save_and_load(tensors):
    from safetensors.torch import load_file, save_file
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "state.safetensors")
        save_file({k: v.detach().cpu().contiguous() for k, v in tensors.items()}, path)
        return load_file(path)


def _steps(run: Run, residual: bool, ks):
    for k in ks:
        g = grads_for_step(run.wl, k, "cuda")
        if residual:
            run.step_residual(g, first=(k == 0))
        else:
            run.step(g)
    torch.cuda.synchronize()


@pytest.mark.parametrize("residual", [False, True], ids=["strict", "residual"])
def test_resume_is_bitwise_equal(residual):
    wl = _wl("resume_w4", RAGGED, 4, steps=K_STEPS + J_STEPS)
    straight = Run(wl)
    _steps(straight, residual, range(K_STEPS + J_STEPS))
    want = {k: v.clone() for k, v in _resumable(straight, residual).items()}
    straight.ctx.close()
    del straight

    first = Run(wl)
    _steps(first, residual, range(K_STEPS))
    saved = _save_and_load(_resumable(first, residual))
    first.ctx.close()
    del first
    torch.cuda.empty_cache()

    resumed = Run(wl)   # new context, new buffers
    for k, v in _resumable(resumed, residual).items():
        v.copy_(saved[k].to("cuda"))
    _steps(resumed, residual, range(K_STEPS, K_STEPS + J_STEPS))
    got = _resumable(resumed, residual)
    for k in want:
        a, b = want[k], got[k]
        same = torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b)
        assert same, f"{k} differs after resume ({'residual' if residual else 'strict'})"
    log(f"resume {'residual' if residual else 'strict'}: {len(want)} buffers bitwise equal")
    resumed.ctx.close()


def test_cltk_resume_is_bitwise_equal():
    from error_compensated_bit_02_amd import OneBitAdam
    wl = _wl("cltk_resume_w3", RAGGED, 3, steps=K_STEPS + J_STEPS)
    _, N = padded_layout(wl.numel)

    def run(steps, memory):
        ctx = OneBitAdam(wl.numel, wl.workers, wl.grad_dtype, wl.beta1, wl.eps)
        ctx.cltk_configure(0.02)
        index = torch.zeros(ctx.K, dtype=torch.int32, device="cuda")
        values = torch.zeros(wl.workers, ctx.K, device="cuda")
        average = torch.zeros(ctx.K, device="cuda")
        for k in steps:
            ctx.cltk_step(k, grads_for_step(wl, k, "cuda"), memory, index, values, average)
        torch.cuda.synchronize()
        ctx.close()
        return index, values, average

    mem_a = torch.zeros(wl.workers, N, device="cuda")
    want = run(range(K_STEPS + J_STEPS), mem_a)
    mem_b = torch.zeros(wl.workers, N, device="cuda")
    run(range(K_STEPS), mem_b)
    mem_c = _save_and_load({"memory": mem_b})["memory"].to("cuda")
    got = run(range(K_STEPS, K_STEPS + J_STEPS), mem_c)
    assert torch.equal(mem_a.view(torch.int32), mem_c.view(torch.int32))
    for a, b in zip(want, got):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
