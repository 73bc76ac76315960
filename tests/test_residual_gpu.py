"""The residual-form step (ob_step_residual + ob_materialize) against the
oracle, and against the strict-form step bit for bit."""
import pytest
import torch

from harness import Run, log, parity_run
from synth import WORKLOADS, grads_for_step
from test_parity_gpu import RAGGED, _report, _wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from error_compensated_bit_02_amd import load_library
    load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_residual_single_tensor_2p20_w4():
    wl = WORKLOADS["single_tensor_2p20"]
    rep = parity_run(wl, wl.steps, residual=True)
    _report(wl.name + " residual", rep)
    assert rep.exact_floats == rep.total_floats


def test_residual_ragged_w3():
    wl = _wl("ragged_w3_residual", RAGGED, 3, steps=5)
    rep = parity_run(wl, wl.steps, residual=True)
    _report(wl.name, rep)
    assert rep.exact_floats == rep.total_floats


@pytest.mark.parametrize("W", [8, 9])
def test_residual_ragged_f32_w8_w9(W):
    """The residual worker pass (one workgroup per 1024-element chunk and
    worker, per-chunk partials) with 8 workers and with 9, where the server
    divides by W instead of multiplying by 1/W; both must match the oracle
    exactly."""
    wl = _wl(f"ragged_w{W}_residual", RAGGED, W, steps=4)
    rep = parity_run(wl, wl.steps, residual=True)
    _report(wl.name, rep)
    assert rep.exact_floats == rep.total_floats


@pytest.mark.parametrize("W,dtype", [(1, "f32"), (2, "f32"), (16, "f32"), (3, "bf16")])
def test_residual_ragged_more_worker_counts(W, dtype):
    """One and two workers (W = 1 and 2 are powers of two, so the server
    multiplies by 1/W), sixteen, and bf16 gradients with three."""
    sigma = 5e-4 if dtype == "bf16" else 1e-3
    wl = _wl(f"ragged_w{W}_{dtype}_residual", RAGGED, W, dtype=dtype, steps=3, g_sigma=sigma)
    rep = parity_run(wl, wl.steps, residual=True)
    _report(wl.name, rep)
    assert rep.exact_floats == rep.total_floats


def test_residual_ragged_bf16_w8():
    wl = _wl("ragged_bf16_w8_residual", RAGGED, 8, dtype="bf16", steps=4, g_sigma=5e-4)
    rep = parity_run(wl, wl.steps, residual=True)
    _report(wl.name, rep)


def test_residual_w64_correlated():
    wl = _wl("w64_residual", (5000, 70000, 3 * 8192), 64, steps=3, g_shared=0.7)
    rep = parity_run(wl, wl.steps, residual=True)
    _report(wl.name, rep)


def test_residual_equals_strict_bitwise():
    """Messages and parameters after every step, and the materialized state
    after the last, are bit-identical to the strict form's."""
    wl = _wl("residual_vs_strict_w5", RAGGED, 5, steps=5)
    a, b = Run(wl), Run(wl)
    bits = lambda t: t.view(torch.int32) if t.dtype == torch.float32 else t  # noqa: E731
    for k in range(wl.steps):
        g = grads_for_step(wl, k, "cuda")
        a.step(g)
        b.step_residual(g, first=(k == 0))
        torch.cuda.synchronize()
        for key in ("packed_w", "scale_w", "packed_s", "scale_s"):
            assert torch.equal(bits(a.bufs[key]), bits(b.bufs[key])), (k, key)
        assert torch.equal(bits(a.state["p"]), bits(b.state["p"])), k
    view = b.materialized()
    torch.cuda.synchronize()
    for key in ("err_w", "err_s", "m"):
        assert torch.equal(bits(a.state[key]), bits(view[key])), key


def test_materialize_in_place_then_strict_continues():
    """Residual steps, materialize in place, then strict steps: same as strict throughout."""
    wl = _wl("residual_then_strict_w4", RAGGED, 4, steps=6)
    a, b = Run(wl), Run(wl)
    for k in range(wl.steps):
        g = grads_for_step(wl, k, "cuda")
        a.step(g)
        if k < 3:
            b.step_residual(g, first=(k == 0))
            if k == 2:
                s, bb = b.state, b.bufs
                b.ctx.materialize(s["err_w"], bb["scale_w"], s["err_s"], bb["scale_s"],
                                  s["err_w"], s["err_s"], s["m"])
        else:
            b.step(g)
    torch.cuda.synchronize()
    for key in ("p", "m", "err_s", "err_w"):
        assert torch.equal(a.state[key].view(torch.int32), b.state[key].view(torch.int32)), key


@pytest.mark.parametrize("name,sample", [
    ("bert_large", ["layer0.attn.q.bias", "layer3.attn.v.weight", "layer23.ln2.gamma", "embed.position"]),
    ("bert_base_w64", ["layer0.attn.q.bias", "layer0.attn.k.weight", "layer11.ln2.beta"]),
    ("resnet50_w32", ["stem.conv", "stage2.block1.reduce.bn.beta", "fc.bias"]),
    ("gpt_1p3b_bf16", ["h0.ln1.gamma", "h5.attn.out.bias", "ln_f.beta"]),
])
def test_residual_full_size(name, sample):
    """Full-size lists in the residual launch configuration, sampled tensors vs the oracle."""
    import oracle.onebit as ob
    from harness import Report
    from synth import host_slice
    wl = WORKLOADS[name]
    idx = {n: i for i, (n, _) in enumerate(wl.tensors)}
    tensors = [idx[n] for n in sample]
    steps = min(wl.steps, 6)
    log(f"{name} residual: {steps} steps, oracle on {sample}")
    run = Run(wl)
    ref = run.host_state(tensors)
    rep = Report()
    gbuf = None
    for k in range(steps):
        gbuf = grads_for_step(wl, k, "cuda", out=gbuf)
        host_g = [host_slice(gbuf, run.off[t], run.off[t] + wl.numel[t]) for t in tensors]
        run.step_residual(gbuf, first=(k == 0))
        view = run.materialized()
        torch.cuda.synchronize()
        for i, t in enumerate(tensors):
            out = ob.compression_step(ref[i], host_g[i], wl.beta1, wl.lr, wl.eps)
            run.compare(t, out, rep, f"{name} residual step {k} {wl.tensors[t][0]}", state=view)
            ref[i] = out.state
        del view
        log(f"  {name} residual step {k}: ok")
    _report(name + " residual", rep)
    run.ctx.close()
    del run, gbuf
    torch.cuda.empty_cache()
