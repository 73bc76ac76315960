"""Cyclic local top-k codec (ob_cltk_step) against the oracle's cltk_step."""
import numpy as np
import pytest
import torch

import oracle.onebit as ob
from harness import log
from synth import WORKLOADS, grads_for_step, host_slice, init_state
from synth.workloads import Workload, padded_layout
from test_parity_gpu import RAGGED, _wl

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


def _run(wl: Workload, density: float, steps: int, tensors=None, grads_fn=None, memory=None):
    from error_compensated_bit_02_amd import OneBitAdam
    ctx = OneBitAdam(wl.numel, wl.workers, wl.grad_dtype, wl.beta1, wl.eps)
    k_off = ctx.cltk_configure(density)
    off, N = padded_layout(wl.numel)
    tensors = list(range(wl.num_tensors)) if tensors is None else tensors
    for t in range(wl.num_tensors):
        assert k_off[t + 1] - k_off[t] == min(ob.cltk_k(wl.numel[t], density), wl.numel[t])
    mem = init_state(wl, "cuda")["err_w"] if memory is None else memory
    if memory is None:
        mem.normal_(0.0, 1e-3)
        for t, n in enumerate(wl.numel):
            mem[:, off[t] + n: off[t + 1]] = 0.0
    K = ctx.K
    index = torch.zeros(K, dtype=torch.int32, device="cuda")
    values = torch.zeros(wl.workers, K, dtype=torch.float32, device="cuda")
    average = torch.zeros(K, dtype=torch.float32, device="cuda")
    ref_mem = [host_slice(mem, off[t], off[t] + wl.numel[t]) for t in tensors]
    exact = total = 0
    for k in range(steps):
        g = grads_for_step(wl, k, "cuda") if grads_fn is None else grads_fn(k)
        host_g = [host_slice(g, off[t], off[t] + wl.numel[t]) for t in tensors]
        ctx.cltk_step(k, g, mem, index, values, average)
        torch.cuda.synchronize()
        for i, t in enumerate(tensors):
            kt = ob.cltk_k(wl.numel[t], density)
            out = ob.cltk_step(ref_mem[i], host_g[i], k, kt)
            lo, hi = k_off[t], k_off[t + 1]
            got_idx = index[lo:hi].cpu().numpy()
            assert np.array_equal(got_idx, out.index), f"step {k} tensor {t}: index differs"
            got_vals = values[:, lo:hi].cpu().numpy()
            assert np.array_equal(got_vals.view(np.uint32), out.values.view(np.uint32)), (k, t)
            got_avg = average[lo:hi].cpu().numpy()
            assert np.array_equal(got_avg.view(np.uint32), out.average.view(np.uint32)), (k, t)
            got_mem = host_slice(mem, off[t], off[t] + wl.numel[t])
            assert np.array_equal(got_mem.view(np.uint32), out.memory.view(np.uint32)), (k, t)
            ref_mem[i] = out.memory
            exact += got_idx.size + got_vals.size + got_avg.size + got_mem.size
            total += got_idx.size + got_vals.size + got_avg.size + got_mem.size
        log(f"  {wl.name} cltk step {k}: ok")
    ctx.close()
    return exact, total


@pytest.mark.parametrize("W,density", [(3, 0.01), (4, 0.1), (1, 0.5), (8, 1.0)])
def test_cltk_ragged(W, density):
    wl = _wl(f"cltk_w{W}", RAGGED, W, steps=4)
    exact, total = _run(wl, density, wl.steps)
    log(f"cltk W={W} density={density}: {exact}/{total} values bit-identical")


def test_cltk_tiled_gather_many_small_tensors():
    """Lists of more than 2^16 tiles take the tiled gather, whose workgroups
    stream groups of workers (shorter lists take the chunked one, which every
    other test here covers).  66,000 tensors of 1 to 300 elements and three
    multi-tile ones with W = 17: groups of 9 and 8 workers on ragged tiles,
    every element of every tensor against the oracle, from the first exchange
    (no threshold prediction) on."""
    from error_compensated_bit_02_amd import OneBitAdam
    rng = np.random.default_rng(17)
    sizes = [int(n) for n in rng.integers(1, 301, size=66000)] + [8193, 20000, 65573]
    W, density, steps = 17, 0.01, 3
    wl = _wl("cltk_many_small_w17", sizes, W, steps=steps)
    tiles = sum((n + 8191) // 8192 for n in sizes)
    assert tiles > 1 << 16
    ctx = OneBitAdam(wl.numel, W, wl.grad_dtype, wl.beta1, wl.eps)
    k_off = ctx.cltk_configure(density)
    off, N = padded_layout(wl.numel)
    mem = torch.zeros(W, N, device="cuda")
    mem.normal_(0.0, 1e-3)
    for t, n in enumerate(wl.numel):
        mem[:, off[t] + n: off[t + 1]] = 0.0
    ref_mem = mem.cpu().numpy()
    index = torch.zeros(ctx.K, dtype=torch.int32, device="cuda")
    values = torch.zeros(W, ctx.K, dtype=torch.float32, device="cuda")
    average = torch.zeros(ctx.K, dtype=torch.float32, device="cuda")
    for k in range(steps):
        g = grads_for_step(wl, k, "cuda")
        host_g = g.cpu().numpy()
        ctx.cltk_step(k, g, mem, index, values, average)
        torch.cuda.synchronize()
        got_mem, got_idx = mem.cpu().numpy(), index.cpu().numpy()
        got_vals, got_avg = values.cpu().numpy(), average.cpu().numpy()
        for t, n in enumerate(wl.numel):
            lo, hi, klo, khi = off[t], off[t] + n, k_off[t], k_off[t + 1]
            out = ob.cltk_step(ref_mem[:, lo:hi], host_g[:, lo:hi], k, ob.cltk_k(n, density))
            assert np.array_equal(got_idx[klo:khi], out.index), f"step {k} tensor {t}: index differs"
            assert np.array_equal(got_vals[:, klo:khi].view(np.uint32), out.values.view(np.uint32)), (k, t)
            assert np.array_equal(got_avg[klo:khi].view(np.uint32), out.average.view(np.uint32)), (k, t)
            assert np.array_equal(got_mem[:, lo:hi].view(np.uint32), out.memory.view(np.uint32)), (k, t)
            ref_mem[:, lo:hi] = out.memory
        log(f"  {wl.name} cltk step {k}: {len(sizes)} tensors, every element bit-identical")
    ctx.close()


def test_cltk_ties_and_zeros():
    """Many equal magnitudes (ties broken by position) and zero memories."""
    wl = _wl("cltk_ties_w2", (5000, 64, 130), 2, steps=3)
    off, _ = padded_layout(wl.numel)

    def grads_fn(k):
        g = grads_for_step(wl, k, "cuda")
        g.copy_(torch.round(g * 1024.0) / 1024.0)   # few distinct magnitudes -> many ties
        for t, n in enumerate(wl.numel):
            g[:, off[t] + n: off[t + 1]] = 0.0
        return g
    memory = torch.zeros(wl.workers, padded_layout(wl.numel)[1], device="cuda")
    exact, total = _run(wl, 0.05, wl.steps, grads_fn=grads_fn, memory=memory)
    log(f"cltk ties: {exact}/{total}")


def test_cltk_all_keys_equal():
    """Every |x| equal (constant gradients, zero memories): every key is a
    candidate and every selected entry is a tie, taken from the lowest index."""
    wl = _wl("cltk_equal_w3", (70000, 8193, 64, 1), 3, steps=2)
    off, N = padded_layout(wl.numel)

    def grads_fn(k):
        g = torch.zeros(wl.workers, N, device="cuda")
        for w in range(wl.workers):
            for t, n in enumerate(wl.numel):
                g[w, off[t]: off[t] + n] = 0.25 * (w + 1) * (1 if k % 2 == 0 else -1)
        return g
    memory = torch.zeros(wl.workers, N, device="cuda")
    _run(wl, 0.3, wl.steps, grads_fn=grads_fn, memory=memory)


def test_cltk_threshold_jumps():
    """The select prepares its candidates for a window around the previous
    exchange's threshold: gradient scales that swing by 1000x between
    exchanges move the threshold far outside it (the fallback path), steady
    ones keep it inside (the predicted path); both must give the same results."""
    wl = _wl("cltk_jumps_w3", RAGGED, 3, steps=8)
    scales = (1.0, 1.0, 1e3, 1e3, 1.0, 1e-3, 1e-3, 1.0)

    def grads_fn(k):
        return grads_for_step(wl, k, "cuda") * scales[k]
    _run(wl, 0.05, wl.steps, grads_fn=grads_fn)


def test_cltk_threshold_drops_below_the_window():
    """A threshold far below the predicted window (memories cleared and the
    gradients 10^4 times smaller) takes the fallback path for a downward
    miss; the exchange after it is predicted again.  Every element of every
    tensor against the oracle."""
    from error_compensated_bit_02_amd import OneBitAdam
    W, density = 3, 0.05
    wl = _wl("cltk_drop_w3", RAGGED, W, steps=4)
    scales = (1.0, 1.0, 1e-4, 1e-4)
    ctx = OneBitAdam(wl.numel, W, wl.grad_dtype, wl.beta1, wl.eps)
    k_off = ctx.cltk_configure(density)
    off, N = padded_layout(wl.numel)
    mem = torch.zeros(W, N, device="cuda")
    ref_mem = mem.cpu().numpy()
    index = torch.zeros(ctx.K, dtype=torch.int32, device="cuda")
    values = torch.zeros(W, ctx.K, dtype=torch.float32, device="cuda")
    average = torch.zeros(ctx.K, dtype=torch.float32, device="cuda")
    for k, scale in enumerate(scales):
        if k == 2:   # clear the memories: only the small gradients remain
            mem.zero_()
            ref_mem[:] = 0.0
        g = grads_for_step(wl, k, "cuda") * scale
        host_g = g.cpu().numpy()
        ctx.cltk_step(k, g, mem, index, values, average)
        torch.cuda.synchronize()
        got_mem, got_idx = mem.cpu().numpy(), index.cpu().numpy()
        got_vals, got_avg = values.cpu().numpy(), average.cpu().numpy()
        for t, n in enumerate(wl.numel):
            lo, hi, klo, khi = off[t], off[t] + n, k_off[t], k_off[t + 1]
            out = ob.cltk_step(ref_mem[:, lo:hi], host_g[:, lo:hi], k, ob.cltk_k(n, density))
            assert np.array_equal(got_idx[klo:khi], out.index), f"exchange {k} tensor {t}: index differs"
            assert np.array_equal(got_vals[:, klo:khi].view(np.uint32), out.values.view(np.uint32)), (k, t)
            assert np.array_equal(got_avg[klo:khi].view(np.uint32), out.average.view(np.uint32)), (k, t)
            assert np.array_equal(got_mem[:, lo:hi].view(np.uint32), out.memory.view(np.uint32)), (k, t)
            ref_mem[:, lo:hi] = out.memory
        log(f"  {wl.name} exchange {k} (gradient scale {scale}): every element bit-identical")
    ctx.close()


def test_cltk_configure_rejects_bad_density():
    from error_compensated_bit_02_amd import OneBitAdam, OneBitError
    ctx = OneBitAdam((100, 7), 2, "f32", 0.9, 1e-8)
    for bad in (0.0, -0.1, 1.5, float("nan")):
        with pytest.raises(OneBitError):
            ctx.cltk_configure(bad)
    assert ctx.cltk_configure(1.0) == [0, 100, 107]
    assert ctx.cltk_configure(0.001) == [0, 1, 2]
    ctx.close()


def test_cltk_bf16():
    wl = _wl("cltk_bf16_w8", RAGGED, 8, dtype="bf16", steps=3, g_sigma=5e-4)
    _run(wl, 0.02, wl.steps)


def test_cltk_full_size_bert_large_sampled():
    wl = WORKLOADS["bert_large"]
    idx = {n: i for i, (n, _) in enumerate(wl.tensors)}
    tensors = [idx[n] for n in ("layer0.attn.q.bias", "layer3.attn.v.weight", "embed.position")]
    _run(wl, 0.01, 3, tensors=tensors)


def test_cltk_full_size_bert_base_w64_sampled():
    """64 workers in groups of 16: every group rebuilds the selection; the
    first writes the index list."""
    wl = WORKLOADS["bert_base_w64"]
    idx = {n: i for i, (n, _) in enumerate(wl.tensors)}
    tensors = [idx[n] for n in ("layer0.attn.q.bias", "layer5.attn.k.weight", "layer11.ln2.beta")]
    _run(wl, 0.01, 2, tensors=tensors)


def test_cltk_full_size_gpt_1p3b_bf16_sampled():
    wl = WORKLOADS["gpt_1p3b_bf16"]
    idx = {n: i for i, (n, _) in enumerate(wl.tensors)}
    tensors = [idx[n] for n in ("h0.ln1.gamma", "h0.attn.qkv.bias", "ln_f.beta")]
    _run(wl, 0.01, 2, tensors=tensors)


def test_cltk_golden_worked_example():
    """The hand-derived example of tests/golden/cltk_worked.txt through the C ABI:
    the GPU must reproduce the hand values exactly (density 0.3: k = 2 of 6)."""
    from error_compensated_bit_02_amd import OneBitAdam
    from golden_io import floats, ints, load
    g = load("cltk_worked.txt")
    ctx = OneBitAdam([6], 3, "f32", 0.9, 1e-8)
    assert ctx.cltk_configure(0.3) == [0, 2]
    memory = torch.zeros(3, 64, device="cuda")
    index = torch.zeros(2, dtype=torch.int32, device="cuda")
    values = torch.zeros(3, 2, device="cuda")
    average = torch.zeros(2, device="cuda")
    for step in (0, 1):
        grads = torch.zeros(3, 64, device="cuda")
        for w in range(3):
            grads[w, :6] = torch.tensor(floats(g[f"step{step}.g{w}"]))
        ctx.cltk_step(step, grads, memory, index, values, average)
        torch.cuda.synchronize()
        assert index.cpu().tolist() == ints(g[f"step{step}.index"]), step
        for w in range(3):
            assert values[w].cpu().tolist() == floats(g[f"step{step}.values{w}"]), (step, w)
            assert memory[w, :6].cpu().tolist() == floats(g[f"step{step}.mem{w}"]), (step, w)
        assert average.cpu().tolist() == floats(g[f"step{step}.average"]), step
    ctx.close()
