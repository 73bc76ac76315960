"""Partitioned server (one scale per tensor chunk, ob_set_server_chunks)
against the oracle's ChunkedOneBitCompressor, in both state forms."""
import pytest
import torch

import oracle.onebit as ob
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


@pytest.mark.parametrize("chunks", [2, 4, 8])
@pytest.mark.parametrize("residual", [False, True], ids=["strict", "residual"])
def test_chunked_server_ragged(chunks, residual):
    wl = _wl(f"chunks{chunks}_w3", RAGGED + (5 * 8192 + 17,), 3, steps=4)
    rep = parity_run(wl, wl.steps, residual=residual, server_chunks=chunks)
    _report(f"{wl.name} {'residual' if residual else 'strict'}", rep)
    assert rep.exact_floats == rep.total_floats


def test_chunk_count_matches_definition():
    wl = WORKLOADS["bert_large"]
    from error_compensated_bit_02_amd import OneBitAdam
    ctx = OneBitAdam(wl.numel, wl.workers)
    assert ctx.S == wl.num_tensors
    for C in (1, 3, 8, 64):
        ctx.set_server_chunks(C)
        assert ctx.S == sum(len(ob.chunk_bounds(n, C)) for n in wl.numel), C
    ctx.close()


def test_chunked_server_full_size_bert_large():
    wl = WORKLOADS["bert_large"]
    idx = {n: i for i, (n, _) in enumerate(wl.tensors)}
    tensors = [idx[n] for n in ("layer0.attn.q.bias", "layer5.attn.k.weight", "embed.position")]
    run = Run(wl, server_chunks=8)
    ref = run.host_state(tensors)
    rep = Report()
    gbuf = None
    for k in range(4):
        gbuf = grads_for_step(wl, k, "cuda", out=gbuf)
        host_g = [host_slice(gbuf, run.off[t], run.off[t] + wl.numel[t]) for t in tensors]
        run.step_residual(gbuf, first=(k == 0))
        view = run.materialized()
        torch.cuda.synchronize()
        for i, t in enumerate(tensors):
            out = oracle_step(ref[i], host_g[i], wl, 8)
            run.compare(t, out, rep, f"bert_large chunks8 step {k} {wl.tensors[t][0]}", state=view)
            ref[i] = out.state
        del view
        log(f"  bert_large chunks8 residual step {k}: ok")
    _report("bert_large server chunks 8", rep)
    run.ctx.close()
    del run, gbuf
    torch.cuda.empty_cache()
