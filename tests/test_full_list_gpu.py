"""Every element of full-size tensor lists against the C++ oracle.

The benchmark's launch configuration (the residual-form step over the whole
list, one launch per kernel) on the BERT-Large-shaped list (W = 8), the
ResNet-50-shaped list (W = 32), the BERT-base-shaped list (W = 64) and the
GPT-1.3B-shaped list with bf16 gradients (W = 8), and the BERT-Large list with
the server partitioned 8 ways and with the trust-ratio update.  After every step each
tensor's sign words, scales, materialized errors, momentum and parameters are
compared bit for bit with the C++ oracle's step, which runs on host copies of
the same inputs and carries its own state from step to step.  The warmup step
(uncompressed Adam) likewise on the BERT-Large and GPT-1.3B lists, and the
cyclic local top-k exchange on the BERT-Large and ResNet-50 lists.  The oracle
runs one tensor per call from a pool of host threads.  The C++ oracle
(oracle/onebit_ref.cpp) is pinned on the CPU by tests/test_oracle_cpp.py.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import fullsize
import oracle.ref as ref
from harness import Run, log
from synth import WORKLOADS, grads_for_step

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _host(t: torch.Tensor) -> np.ndarray:
    """A whole device buffer on the host; bf16 as its uint16 patterns, int64 words as uint64."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    a = t.contiguous().cpu().numpy()
    return a.view(np.uint64) if a.dtype == np.int64 else a


def _same(a, b) -> bool:
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), np.asarray(b, np.float32).view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)


# Every workload for its whole trajectory (the step counts of the workloads),
# in both state forms side by side against one oracle trajectory; the
# partitioned server and the trust-ratio update on the BERT-Large list for two
# steps.
CONFIGS = ["resnet50_w32", "bert_large", "bert_base_w64", "gpt_1p3b_bf16"]


@pytest.mark.parametrize("name", CONFIGS)
def test_config_trajectory_every_element(name):
    wl = WORKLOADS[name]
    fullsize.trajectory(wl, ("residual", "strict"), wl.steps)


@pytest.mark.parametrize("chunks,trust_wd", [(8, None), (1, 0.01)], ids=["server8", "trust"])
def test_bert_large_options_every_element(chunks, trust_wd):
    """The server partitioned 8 ways, and the trust-ratio update with weight decay."""
    fullsize.trajectory(WORKLOADS["bert_large"], ("residual",), 2, server_chunks=chunks, trust_wd=trust_wd)


@pytest.mark.parametrize("name,steps", [("bert_large", 2), ("gpt_1p3b_bf16", 1)])
def test_warmup_every_element_against_cpp_oracle(name, steps):
    """The warmup step (uncompressed Adam on the average gradient, from zero
    moments) over the whole list, every element of p, m and v bit for bit."""
    beta2, lr = 0.999, 1e-3
    wl = WORKLOADS[name]
    threads = max(1, min(16, os.cpu_count() or 1))
    log(f"{name}: {steps} warmup steps, every tensor against the C++ oracle ({threads} threads)")
    ref.load()
    run = Run(wl)
    run.state["m"].zero_()
    run.state["v"].zero_()
    off = run.off
    host = {k: _host(run.state[k]) for k in ("p", "m", "v")}
    states = [{k: np.ascontiguousarray(host[k][off[t]:off[t] + n]) for k in host} for t, n in enumerate(wl.numel)]
    del host
    gbuf = None
    floats = 0
    for k in range(steps):
        gbuf = grads_for_step(wl, k, "cuda", out=gbuf)
        g = _host(gbuf)
        run.ctx.warmup_step(gbuf, run.state["m"], run.state["v"], run.state["p"], beta2, lr)
        torch.cuda.synchronize()
        got = {key: _host(run.state[key]) for key in ("p", "m", "v")}

        def check(t):
            n = wl.numel[t]
            lo, hi = off[t], off[t] + n
            st = states[t]
            c = ref.warmup_step(st["p"], st["m"], st["v"], np.ascontiguousarray(g[:, lo:hi]), wl.beta1, beta2,
                                lr, wl.eps)
            bad = [key for key in ("p", "m", "v") if not _same(c[key], got[key][lo:hi])]
            states[t] = c
            return t, bad, 3 * n

        with ThreadPoolExecutor(max_workers=threads) as pool:
            results = list(pool.map(check, sorted(range(wl.num_tensors), key=lambda t: -wl.numel[t])))
        failed = [(wl.tensors[t][0], bad) for t, bad, _ in results if bad]
        floats += sum(r[2] for r in results)
        assert not failed, f"{name} warmup step {k}: {len(failed)} tensors differ, first {failed[:3]}"
        log(f"{name} warmup step {k}: {floats} floats compared, all bit-identical")
        del got, g


@pytest.mark.parametrize("name,steps", [("bert_large", 3), ("resnet50_w32", 3)])
def test_cltk_every_element_against_cpp_oracle(name, steps):
    """The cyclic local top-k exchange at density 0.01 from zero memories (the
    first exchange without a threshold prediction, then the predicted window and
    its fallback), every index, value, average and memory element bit for bit."""
    from error_compensated_bit_02_amd import OneBitAdam
    density = 0.01
    wl = WORKLOADS[name]
    threads = max(1, min(16, os.cpu_count() or 1))
    log(f"{name}: {steps} CLT-k exchanges, every tensor against the C++ oracle ({threads} threads)")
    ref.load()
    ctx = OneBitAdam(wl.numel, wl.workers, wl.grad_dtype, wl.beta1, wl.eps)
    k_off = ctx.cltk_configure(density)
    run_off = ctx.offsets
    memory = torch.zeros(wl.workers, ctx.N, device="cuda")
    index = torch.zeros(ctx.K, dtype=torch.int32, device="cuda")
    values = torch.zeros(wl.workers, ctx.K, device="cuda")
    average = torch.zeros(ctx.K, device="cuda")
    mems = [np.zeros((wl.workers, n), np.float32) for n in wl.numel]
    gbuf = None
    compared = 0
    for k in range(steps):
        gbuf = grads_for_step(wl, k, "cuda", out=gbuf)
        g = _host(gbuf)
        ctx.cltk_step(k, gbuf, memory, index, values, average)
        torch.cuda.synchronize()
        got = {"memory": _host(memory), "index": _host(index), "values": _host(values), "average": _host(average)}

        def check(t):
            n = wl.numel[t]
            lo, hi = run_off[t], run_off[t] + n
            klo, khi = k_off[t], k_off[t + 1]
            c = ref.cltk_step(mems[t], np.ascontiguousarray(g[:, lo:hi]), k, khi - klo)
            bad = [key for key, mine, dev in (
                ("index", c["index"], got["index"][klo:khi].astype(np.int64)),
                ("values", c["values"], got["values"][:, klo:khi]),
                ("average", c["average"], got["average"][klo:khi]),
                ("memory", c["memory"], got["memory"][:, lo:hi]),
            ) if not _same(mine, dev)]
            mems[t] = c["memory"]
            return t, bad, (khi - klo) * (2 + wl.workers) + wl.workers * n

        with ThreadPoolExecutor(max_workers=threads) as pool:
            results = list(pool.map(check, sorted(range(wl.num_tensors), key=lambda t: -wl.numel[t])))
        failed = [(wl.tensors[t][0], bad) for t, bad, _ in results if bad]
        compared += sum(r[2] for r in results)
        assert not failed, f"{name} exchange {k}: {len(failed)} tensors differ, first {failed[:3]}"
        log(f"{name} exchange {k}: {compared} entries compared, all bit-identical")
        del got, g
    ctx.close()
