"""Warmup phase (uncompressed Adam on the average gradient) and the switch to
the compression phase, on the GPU through the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle.onebit as ob
from harness import Report, Run, _cmp_float, log
from synth import WORKLOADS, grads_for_step, host_slice
from test_parity_gpu import RAGGED, _report, _wl

pytestmark = pytest.mark.gpu

BETA2 = 0.999
WARM_LR = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from error_compensated_bit_02_amd import load_library
    load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _adam_start(run: Run):
    """Adam starts from zero first and second moments."""
    run.state["m"].zero_()
    run.state["v"].zero_()


def _compare_mvp(run: Run, t: int, st: ob.TensorState, rep: Report, what: str):
    lo, hi = run.off[t], run.off[t] + run.wl.numel[t]
    for key, want in (("m", st.m), ("v", st.v), ("p", st.p)):
        _cmp_float(f"{what} {key}", host_slice(run.state[key], lo, hi), want, rep, atol=1e-6)


@pytest.mark.parametrize("name,sizes,W,dtype", [
    ("warmup_ragged_w3", RAGGED, 3, "f32"),
    ("warmup_ragged_bf16_w8", RAGGED, 8, "bf16"),
    ("warmup_w64", (5000, 70000), 64, "f32"),
])
def test_warmup_matches_oracle(name, sizes, W, dtype):
    wl = _wl(name, sizes, W, dtype=dtype, steps=5, g_sigma=5e-4 if dtype == "bf16" else 1e-3)
    run = Run(wl)
    _adam_start(run)
    tensors = list(range(wl.num_tensors))
    ref = run.host_state(tensors)
    rep = Report()
    for k in range(wl.steps):
        g = grads_for_step(wl, k, "cuda")
        host_g = [host_slice(g, run.off[t], run.off[t] + wl.numel[t]) for t in tensors]
        run.ctx.warmup_step(g, run.state["m"], run.state["v"], run.state["p"], BETA2, WARM_LR)
        torch.cuda.synchronize()
        for i, t in enumerate(tensors):
            ref[i] = ob.warmup_step(ref[i], host_g[i], wl.beta1, BETA2, WARM_LR, wl.eps)
            _compare_mvp(run, t, ref[i], rep, f"{name} step {k} tensor {t}")
    _report(name, rep)
    assert rep.exact_floats == rep.total_floats


@pytest.mark.parametrize("residual", [False, True], ids=["strict", "residual"])
def test_warmup_then_compression_pipeline(residual):
    """3 warmup steps, the switch (v frozen, errors zeroed), 4 compression steps:
    every step's state against the oracle run through the same phases."""
    wl = _wl("pipeline_w4", RAGGED, 4, steps=7)
    run = Run(wl)
    _adam_start(run)
    run.state["err_w"].fill_(0.25)     # garbage that the switch must clear
    run.state["err_s"].fill_(-0.5)
    tensors = list(range(wl.num_tensors))
    ref = run.host_state(tensors)
    rep = Report()
    for k in range(wl.steps):
        g = grads_for_step(wl, k, "cuda")
        host_g = [host_slice(g, run.off[t], run.off[t] + wl.numel[t]) for t in tensors]
        if k < 3:
            run.ctx.warmup_step(g, run.state["m"], run.state["v"], run.state["p"], BETA2, WARM_LR)
            torch.cuda.synchronize()
            for i, t in enumerate(tensors):
                ref[i] = ob.warmup_step(ref[i], host_g[i], wl.beta1, BETA2, WARM_LR, wl.eps)
                _compare_mvp(run, t, ref[i], rep, f"warmup step {k} tensor {t}")
            continue
        if k == 3:
            run.ctx.begin_compression(run.state["err_w"], run.state["err_s"])
            for st in ref:
                st.err_w[...] = 0.0
                st.err_s[...] = 0.0
        view = None
        if residual:
            run.step_residual(g, first=(k == 3))
            view = run.materialized()
        else:
            run.step(g)
        torch.cuda.synchronize()
        for i, t in enumerate(tensors):
            out = ob.compression_step(ref[i], host_g[i], wl.beta1, wl.lr, wl.eps)
            run.compare(t, out, rep, f"compression step {k} tensor {t}", state=view)
            ref[i] = out.state
            v_dev = host_slice(run.state["v"], run.off[t], run.off[t] + wl.numel[t])
            assert np.array_equal(v_dev, ref[i].v), "the variance must stay frozen"
    _report("pipeline " + ("residual" if residual else "strict"), rep)
    assert rep.exact_floats == rep.total_floats


def test_begin_compression_zeroes_tensors_not_padding():
    wl = _wl("switch_w2", (1000, 65, 1), 2, steps=1)
    run = Run(wl)
    run.state["err_w"].fill_(3.0)
    run.state["err_s"].fill_(3.0)
    run.ctx.begin_compression(run.state["err_w"], run.state["err_s"])
    torch.cuda.synchronize()
    for t, n in enumerate(wl.numel):
        lo, pad_hi = run.off[t], run.off[t + 1]
        assert torch.all(run.state["err_w"][:, lo:lo + n] == 0)
        assert torch.all(run.state["err_s"][lo:lo + n] == 0)
        assert torch.all(run.state["err_w"][:, lo + n:pad_hi] == 3.0)
        assert torch.all(run.state["err_s"][lo + n:pad_hi] == 3.0)


def test_warmup_full_size_bert_large_sampled():
    """The warmup kernel at full size (BERT-Large list, W = 8), sampled tensors vs the oracle."""
    wl = WORKLOADS["bert_large"]
    idx = {n: i for i, (n, _) in enumerate(wl.tensors)}
    tensors = [idx[n] for n in ("layer0.attn.q.bias", "layer7.ffn.b1", "embed.position")]
    run = Run(wl)
    _adam_start(run)
    ref = run.host_state(tensors)
    rep = Report()
    for k in range(3):
        g = grads_for_step(wl, k, "cuda")
        host_g = [host_slice(g, run.off[t], run.off[t] + wl.numel[t]) for t in tensors]
        run.ctx.warmup_step(g, run.state["m"], run.state["v"], run.state["p"], BETA2, WARM_LR)
        torch.cuda.synchronize()
        for i, t in enumerate(tensors):
            ref[i] = ob.warmup_step(ref[i], host_g[i], wl.beta1, BETA2, WARM_LR, wl.eps)
            _compare_mvp(run, t, ref[i], rep, f"bert_large warmup step {k} {wl.tensors[t][0]}")
        log(f"  bert_large warmup step {k}: ok")
        del g
    _report("bert_large warmup", rep)
    run.ctx.close()
    del run
    torch.cuda.empty_cache()
