"""Layer-wise trust-ratio update (ob_set_trust_ratio) against the oracle's
trust_ratio_update, in both state forms, with and without weight decay."""
import pytest
import torch

from harness import Report, Run, log, oracle_step, parity_run
from synth import WORKLOADS, grads_for_step, host_slice
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


@pytest.mark.parametrize("wd", [0.0, 0.01])
@pytest.mark.parametrize("residual", [False, True], ids=["strict", "residual"])
def test_trust_ratio_ragged(wd, residual):
    wl = _wl(f"trust_wd{wd}_w3", RAGGED, 3, steps=4)
    rep = parity_run(wl, wl.steps, residual=residual, trust_wd=wd)
    _report(f"{wl.name} {'residual' if residual else 'strict'}", rep)
    assert rep.exact_floats == rep.total_floats


def test_trust_ratio_with_partitioned_server_w1():
    """W = 1 (the server row is partial row 1, reused by the norms) and 4 server chunks."""
    wl = _wl("trust_chunks_w1", RAGGED, 1, steps=3)
    rep = parity_run(wl, wl.steps, residual=True, server_chunks=4, trust_wd=0.0)
    _report(wl.name, rep)
    assert rep.exact_floats == rep.total_floats


def test_trust_ratio_split_calls():
    wl = _wl("trust_split_w4", RAGGED, 4, steps=3)
    rep = parity_run(wl, wl.steps, split=True, trust_wd=0.001)
    _report(wl.name, rep)


def test_trust_ratio_full_size_bert_large():
    wl = WORKLOADS["bert_large"]
    idx = {n: i for i, (n, _) in enumerate(wl.tensors)}
    tensors = [idx[n] for n in ("layer0.ln1.gamma", "layer9.attn.out.weight", "embed.position")]
    run = Run(wl, trust_wd=0.01)
    ref = run.host_state(tensors)
    rep = Report()
    gbuf = None
    for k in range(3):
        gbuf = grads_for_step(wl, k, "cuda", out=gbuf)
        host_g = [host_slice(gbuf, run.off[t], run.off[t] + wl.numel[t]) for t in tensors]
        run.step_residual(gbuf, first=(k == 0))
        view = run.materialized()
        torch.cuda.synchronize()
        for i, t in enumerate(tensors):
            out = oracle_step(ref[i], host_g[i], wl, 1, 0.01)
            run.compare(t, out, rep, f"bert_large trust step {k} {wl.tensors[t][0]}", state=view)
            ref[i] = out.state
        del view
        log(f"  bert_large trust-ratio residual step {k}: ok")
    _report("bert_large trust ratio", rep)
    run.ctx.close()
    del run, gbuf
    torch.cuda.empty_cache()
