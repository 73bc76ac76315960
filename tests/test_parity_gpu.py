"""Parity of the HIP path (through the C ABI) with the oracle, element by element.

Small and ragged tensor lists are compared in full after every step; the
full-size workloads run in the launch configuration the benchmark times
(ob_step over the whole tensor list) and are compared on sampled tensors,
plus properties checked on every element of every tensor.
"""
import numpy as np
import pytest
import torch

import oracle.onebit as ob
from harness import Report, Run, log, parity_run
from synth import WORKLOADS, grads_for_step, host_slice, init_state
from synth.workloads import Workload, padded_layout

pytestmark = pytest.mark.gpu

RAGGED = (1, 63, 64, 65, 1000, 8191, 8192, 8193, 20000, 100003)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from error_compensated_bit_02_amd import load_library
    load_library()          # with a GPU present, a missing library is an error, not a skip
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _wl(name, sizes, W, dtype="f32", steps=4, **kw):
    return Workload(name=name, tensors=tuple((f"t{i}", (n,)) for i, n in enumerate(sizes)),
                    workers=W, grad_dtype=dtype, steps=steps, g_sigma=kw.pop("g_sigma", 1e-3),
                    v_kind="sq_normal", v_a=1e-3, v_b=1e-12, **kw)


def _report(name, rep: Report):
    log(f"{name}: {rep.words} sign words bit-exact; {rep.exact_floats}/{rep.total_floats} floats "
        f"bit-identical; max |state diff| {rep.max_state_err:.3g}; max scale rel {rep.max_scale_rel:.3g}")


def test_single_tensor_2p20_w4_10_steps():
    wl = WORKLOADS["single_tensor_2p20"]
    rep = parity_run(wl, wl.steps)
    _report(wl.name, rep)
    assert rep.exact_floats == rep.total_floats


def test_ragged_list_w3():
    wl = _wl("ragged_w3", RAGGED, 3, steps=6)
    rep = parity_run(wl, wl.steps)
    _report(wl.name, rep)
    assert rep.exact_floats == rep.total_floats


def test_ragged_list_bf16_w8():
    wl = _wl("ragged_bf16_w8", RAGGED, 8, dtype="bf16", steps=4, g_sigma=5e-4)
    rep = parity_run(wl, wl.steps)
    _report(wl.name, rep)


def test_single_worker():
    wl = _wl("w1", (1000, 8192, 9000), 1, steps=4)
    rep = parity_run(wl, wl.steps)
    _report(wl.name, rep)


def test_many_workers_w64_correlated():
    wl = _wl("w64", (5000, 70000, 3 * 8192), 64, steps=3, g_shared=0.7)
    rep = parity_run(wl, wl.steps)
    _report(wl.name, rep)


@pytest.mark.parametrize("residual", [False, True], ids=["strict", "residual"])
def test_many_workers_w200(residual):
    """W = 200 (not a power of two): worker groups of up to 16, the server's
    word loads in groups of 8 with a ragged last group, 201 partial-sum rows."""
    wl = _wl("w200", (1, 65, 8193, 20000), 200, steps=2)
    rep = parity_run(wl, wl.steps, residual=residual)
    _report(wl.name, rep)


def test_split_calls_equal_oracle():
    wl = _wl("ragged_split_w5", RAGGED, 5, steps=3)
    rep = parity_run(wl, wl.steps, split=True)
    _report(wl.name, rep)


def test_split_calls_equal_fused_step_bitwise():
    wl = _wl("split_vs_fused_w4", RAGGED, 4, steps=3)
    a, b = Run(wl), Run(wl)
    for k in range(wl.steps):
        g = grads_for_step(wl, k, "cuda")
        a.step(g)
        b.step_split(g)
    torch.cuda.synchronize()
    for key in ("p", "m", "err_s", "err_w"):
        assert torch.equal(a.state[key].view(torch.int32), b.state[key].view(torch.int32)), key
    for key in ("packed_w", "scale_w", "packed_s", "scale_s"):
        assert torch.equal(a.bufs[key], b.bufs[key]), key


def test_worker_subranges():
    """Compressing workers [0,2) and [2,5) separately equals all five at once."""
    wl = _wl("subrange_w5", RAGGED, 5, steps=1)
    a, b = Run(wl), Run(wl)
    g = grads_for_step(wl, 0, "cuda")
    a.ctx.compress_worker(g, a.state["m"], a.state["err_w"], a.bufs["packed_w"], a.bufs["scale_w"])
    b.ctx.compress_worker(g, b.state["m"], b.state["err_w"], b.bufs["packed_w"], b.bufs["scale_w"], 0, 2)
    b.ctx.compress_worker(g, b.state["m"], b.state["err_w"], b.bufs["packed_w"], b.bufs["scale_w"], 2, 5)
    torch.cuda.synchronize()
    assert torch.equal(a.state["err_w"], b.state["err_w"])
    assert torch.equal(a.bufs["packed_w"], b.bufs["packed_w"])
    assert torch.equal(a.bufs["scale_w"], b.bufs["scale_w"])


def test_worker_subranges_large_tensor_against_oracle():
    """A tensor of 4097 tiles (its scales take the finalize with a workgroup per
    (worker, tensor)) beside a small one: workers [1, 3) then [0, 1) through
    ob_compress_worker equal all three at once, and the scales and signs of a
    sampled worker equal the oracle's."""
    n_big = 4097 * 8192 - 5
    wl = _wl("subrange_big_w3", (n_big, 777), 3, steps=1)
    a, b = Run(wl), Run(wl)
    g = grads_for_step(wl, 0, "cuda")
    a.ctx.compress_worker(g, a.state["m"], a.state["err_w"], a.bufs["packed_w"], a.bufs["scale_w"])
    b.ctx.compress_worker(g, b.state["m"], b.state["err_w"], b.bufs["packed_w"], b.bufs["scale_w"], 1, 3)
    b.ctx.compress_worker(g, b.state["m"], b.state["err_w"], b.bufs["packed_w"], b.bufs["scale_w"], 0, 1)
    torch.cuda.synchronize()
    assert torch.equal(a.state["err_w"], b.state["err_w"])
    assert torch.equal(a.bufs["packed_w"], b.bufs["packed_w"])
    assert torch.equal(a.bufs["scale_w"], b.bufs["scale_w"])
    off = a.off
    for t, n in enumerate(wl.numel):
        # worker 2 from the initial state: m = 0 (read only here) and e = 0
        m = host_slice(a.state["m"], off[t], off[t] + n)
        x = ob.worker_momentum(m, host_slice(g, off[t], off[t] + n)[2], wl.beta1) + np.zeros(n, np.float32)
        msg = ob.OneBitCompressor.compress(x)
        got_w = a.bufs["packed_w"][2, off[t] // 64: off[t] // 64 + (n + 63) // 64].cpu().numpy().view(np.uint64)
        assert np.array_equal(got_w, msg.words), t
        assert a.bufs["scale_w"][2, t].item() == float(msg.scale), t


@pytest.mark.parametrize("residual", [False, True], ids=["strict", "residual"])
def test_special_values_zero_nan_subnormal(residual):
    """A zero tensor (scale 0, all bits 1), a tensor with -0/+0 and a NaN
    (scale NaN), and a tensor of subnormal gradients, against the oracle, in
    both state forms."""
    sizes = (130, 70, 200)
    wl = _wl("special_w2", sizes, 2, steps=3)
    run_state = init_state(wl, "cuda")
    off, _ = padded_layout(wl.numel)

    def grads_fn(k):
        g = grads_for_step(wl, k, "cuda")
        g[:, off[0]:off[0] + 130] = 0.0
        g[:, off[1]:off[1] + 70] = -0.0
        g[0, off[1] + 5] = float("nan")
        g[:, off[2]:off[2] + 200] *= 1e-38 / 1e-3     # subnormal and tiny normals
        return g
    rep = parity_run(wl, wl.steps, grads_fn=grads_fn, state=run_state, residual=residual)
    _report(wl.name, rep)


def test_padding_never_written():
    wl = _wl("padding_w3", (1000, 65, 1), 3, steps=2)
    run = Run(wl)
    canary = 12345.0
    pads = [(run.off[t] + n, run.off[t + 1]) for t, n in enumerate(wl.numel)]
    for key in ("p", "m", "err_s", "err_w", "v"):
        for lo, hi in pads:
            run.state[key][..., lo:hi] = canary
    for k in range(wl.steps):
        run.step(grads_for_step(wl, k, "cuda"))
        run.step_split(grads_for_step(wl, k + 10, "cuda"))
    torch.cuda.synchronize()
    for key in ("p", "m", "err_s", "err_w", "v"):
        for lo, hi in pads:
            assert torch.all(run.state[key][..., lo:hi] == canary), key
    # padding bits of each tensor's last word are zero
    for t, n in enumerate(wl.numel):
        if n % 64:
            last = run.off[t] // 64 + (n + 63) // 64 - 1
            mask = ~np.uint64((1 << (n % 64)) - 1)
            for w in range(wl.workers):
                assert int(run.bufs["packed_w"][w, last].cpu().numpy().view(np.uint64) & mask) == 0
            assert int(run.bufs["packed_s"][last].cpu().numpy().view(np.uint64) & mask) == 0


def test_two_runs_bitwise_identical():
    wl = _wl("determinism_w6", RAGGED, 6, steps=3)
    runs = [Run(wl), Run(wl)]
    for k in range(wl.steps):
        g = grads_for_step(wl, k, "cuda")
        for r in runs:
            r.step(g)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int32) if t.dtype == torch.float32 else t  # noqa: E731
    for key in ("p", "m", "err_s", "err_w"):
        assert torch.equal(bits(runs[0].state[key]), bits(runs[1].state[key])), key
    for key in ("packed_w", "scale_w", "packed_s", "scale_s"):
        assert torch.equal(bits(runs[0].bufs[key]), bits(runs[1].bufs[key])), key


def test_bad_arguments_are_rejected_before_launch():
    from error_compensated_bit_02_amd import OneBitError
    wl = _wl("badargs", (100,), 2, steps=1)
    run = Run(wl)
    s, b = run.state, run.bufs
    g = grads_for_step(wl, 0, "cuda")
    lib = run.ctx.lib
    ptrs = [g.data_ptr(), s["m"].data_ptr(), s["err_w"].data_ptr(), b["packed_w"].data_ptr(),
            b["scale_w"].data_ptr()]
    assert lib.ob_compress_worker(run.ctx._ctx, 0, 3, *ptrs, None) == 1          # w_end > W
    assert lib.ob_compress_worker(run.ctx._ctx, 1, 1, *ptrs, None) == 1          # empty range
    bad = list(ptrs)
    bad[1] += 4                                                                   # misaligned m
    assert lib.ob_compress_worker(run.ctx._ctx, 0, 2, *bad, None) == 2
    assert lib.ob_apply_update(run.ctx._ctx, b["packed_s"].data_ptr(), b["scale_s"].data_ptr(),
                               s["v"].data_ptr(), s["m"].data_ptr(), s["p"].data_ptr(),
                               float("inf"), None) == 1
    with pytest.raises(OneBitError):
        run.ctx.step(g[:, :50], s["m"], s["v"], s["p"], s["err_w"], s["err_s"], b["packed_w"],
                     b["scale_w"], b["packed_s"], b["scale_s"], 1e-4)
    torch.cuda.synchronize()
    assert torch.all(s["err_w"] == 0)     # nothing was launched


# ---------------------------------------------------------------------------
# full-size workloads, in the benchmark's launch configuration
# ---------------------------------------------------------------------------

def _names_to_index(wl, names):
    idx = {n: i for i, (n, _) in enumerate(wl.tensors)}
    return [idx[n] for n in names]


def _whole_list_properties(run: Run):
    """On every element of every tensor: m equals the decoded server message,
    every scale is finite and positive."""
    b, s, wl = run.bufs, run.state, run.wl
    assert torch.isfinite(b["scale_w"]).all() and (b["scale_w"] > 0).all()
    assert torch.isfinite(b["scale_s"]).all() and (b["scale_s"] > 0).all()
    shifts = torch.arange(64, device=b["packed_s"].device, dtype=torch.int64)
    for t, n in enumerate(wl.numel):
        lo = run.off[t]
        words = b["packed_s"][lo // 64: lo // 64 + (n + 63) // 64]
        bits = ((words.view(-1, 1) >> shifts) & 1).view(-1)[:n].bool()
        ss = b["scale_s"][t]
        expect = torch.where(bits, ss, -ss)
        assert torch.equal(s["m"][lo:lo + n], expect), wl.tensors[t][0]


def _full_size(name, sample_names):
    wl = WORKLOADS[name]
    tensors = _names_to_index(wl, sample_names)
    log(f"{name}: {wl.num_tensors} tensors, N={sum(wl.numel)}, W={wl.workers}, {wl.steps} steps; "
        f"oracle on {[wl.tensors[t][0] for t in tensors]}")
    run = Run(wl)
    ref = run.host_state(tensors)
    rep = Report()
    gbuf = None
    for k in range(wl.steps):
        gbuf = grads_for_step(wl, k, "cuda", out=gbuf)
        host_g = [host_slice(gbuf, run.off[t], run.off[t] + wl.numel[t]) for t in tensors]
        run.step(gbuf)
        torch.cuda.synchronize()
        for i, t in enumerate(tensors):
            out = ob.compression_step(ref[i], host_g[i], wl.beta1, wl.lr, wl.eps)
            run.compare(t, out, rep, f"{name} step {k} {wl.tensors[t][0]}")
            ref[i] = out.state
        log(f"  {name} step {k}: ok")
    _whole_list_properties(run)
    _report(name, rep)
    run.ctx.close()
    del run, gbuf
    torch.cuda.empty_cache()


def test_full_size_bert_large_w8():
    _full_size("bert_large", ["layer0.attn.q.weight", "layer0.attn.q.bias", "layer0.ln1.gamma",
                              "layer11.ffn.b1", "layer23.ln2.beta", "embed.position"])


def test_full_size_bert_base_w64():
    _full_size("bert_base_w64", ["layer0.attn.q.bias", "layer0.attn.k.weight", "layer6.ffn.b1",
                                 "layer11.ln2.beta"])


def test_full_size_gpt_1p3b_bf16_w8():
    _full_size("gpt_1p3b_bf16", ["h0.ln1.gamma", "h0.attn.qkv.bias", "h0.attn.out.weight",
                                 "h23.mlp.b2", "ln_f.beta"])


def test_full_size_resnet50_w32():
    _full_size("resnet50_w32", ["stem.conv", "stem.bn.gamma", "stage0.block0.reduce.conv",
                                "stage1.block0.spatial.conv", "stage3.block2.expand.bn.beta",
                                "fc.bias"])
