"""Every element of a full-size tensor list against the C++ oracle.

The benchmark's launch configuration (the residual-form step over the whole
list, one launch per kernel) on the BERT-Large-shaped list with 8 workers and
the ResNet-50-shaped list with 32 workers; after every step, each tensor's
sign words, scales, materialized errors, momentum and parameters are compared
with the C++ oracle's step on the same inputs (copied to the host before the
step).  The C++ oracle (oracle/onebit_ref.cpp) is pinned on the CPU by
tests/test_oracle_cpp.py.
"""
import numpy as np
import pytest
import torch

import oracle.onebit as ob
import oracle.ref as ref
from harness import Report, Run, log
from synth import WORKLOADS, grads_for_step, host_slice

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _as_step_output(c: dict, v: np.ndarray, n: int) -> ob.StepOutput:
    W = c["packed_w"].shape[0]
    msgs = [ob.OneBitMessage(c["packed_w"][w], np.float32(c["scale_w"][w]), n) for w in range(W)]
    state = ob.TensorState(c["p"], c["m"], v, c["err_s"], c["err_w"])
    return ob.StepOutput(state, msgs, ob.OneBitMessage(c["packed_s"], np.float32(c["scale_s"]), n))


@pytest.mark.parametrize("name,steps", [("resnet50_w32", 3), ("bert_large", 2)])
def test_every_element_against_cpp_oracle(name, steps):
    wl = WORKLOADS[name]
    log(f"{name}: {steps} residual-form steps, every tensor against the C++ oracle")
    ref.load()
    run = Run(wl)
    host = run.host_state(range(wl.num_tensors))
    rep = Report()
    gbuf = None
    for k in range(steps):
        gbuf = grads_for_step(wl, k, "cuda", out=gbuf)
        run.step_residual(gbuf, first=(k == 0))
        view = run.materialized()
        torch.cuda.synchronize()
        for t in range(wl.num_tensors):
            lo, hi = run.off[t], run.off[t] + wl.numel[t]
            st = host[t]
            c = ref.compression_step(st.p, st.m, st.v, st.err_s, st.err_w, host_slice(gbuf, lo, hi),
                                     wl.beta1, wl.lr, wl.eps)
            out = _as_step_output(c, st.v, wl.numel[t])
            run.compare(t, out, rep, f"{name} step {k} {wl.tensors[t][0]}", state=view)
            host[t] = out.state
        del view
        log(f"{name} step {k}: {rep.words} sign words and {rep.total_floats} floats compared, "
            f"{rep.exact_floats} floats bit-identical")
    assert rep.exact_floats == rep.total_floats
