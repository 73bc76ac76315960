"""ob_step_residual_noalloc (the step with its scratch in the library's static
per-GPU buffer) against ob_step_residual (the context's own scratch).

Both entry points run the same step on separate copies of the same state and
gradients; after every call every output -- parameters, the residual-form
errors, the sign messages and the scales -- must be bit-identical.  Calls come
in a row on one GPU with shrinking inputs (a list needing nearly the whole
static buffer, then the BERT-Large-shaped list, then a small ragged list with
the trust-ratio update), so a call that read what an earlier, larger call left
in the shared buffer would show.  A list needing more than the buffer is
rejected before anything is enqueued.
"""
import pytest
import torch

from error_compensated_bit_02_amd import OneBitAdam
from error_compensated_bit_02_amd.binding import OB_ERR_SCRATCH, OneBitError
from synth import WORKLOADS, grads_for_step, init_state
from synth.workloads import Workload

pytestmark = pytest.mark.gpu

STATIC_BYTES = 64 << 20   # the static buffer's size, as include/ob.h states it
TILE = 8192


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _need(numel, W):
    """Bytes of static scratch a list needs, by the formula of include/ob.h."""
    tiles = sum(-(-n // TILE) for n in numel)
    up = lambda b: -(-b // 256) * 256   # noqa: E731
    return up((W + 1) * tiles * 16) + up(W * tiles * 128) + up(len(numel) * 4)


def _wl(name, sizes, W, steps=2):
    return Workload(name=name, tensors=tuple((f"t{i}", (n,)) for i, n in enumerate(sizes)), workers=W,
                    grad_dtype="f32", steps=steps, g_sigma=1e-3, v_kind="sq_normal", v_a=1e-3, v_b=1e-12)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _compare_entry_points(wl, steps, trust_wd=None):
    print(f"{wl.name}: {wl.num_tensors} tensors, {sum(wl.numel)} elements, W={wl.workers}, "
          f"{_need(wl.numel, wl.workers) / 2**20:.1f} MiB of static scratch, {steps} steps", flush=True)
    ctx = OneBitAdam(wl.numel, wl.workers, wl.grad_dtype, wl.beta1, wl.eps)
    if trust_wd is not None:
        ctx.set_trust_ratio(True, trust_wd)
    runs = []
    for _ in range(2):
        runs.append((init_state(wl, "cuda"), ctx.alloc("cuda")))
    gbuf = None
    for k in range(steps):
        gbuf = grads_for_step(wl, k, "cuda", out=gbuf)
        for noalloc, (st, b) in zip((False, True), runs):
            ctx.step_residual(k == 0, gbuf, st["m"], st["v"], st["p"], st["err_w"], st["err_s"], b["packed_w"],
                              b["scale_w"], b["packed_s"], b["scale_s"], wl.lr, noalloc=noalloc)
        torch.cuda.synchronize()
        (sa, ba), (sb, bb) = runs
        for key in ("p", "err_w", "err_s"):
            assert torch.equal(_bits(sa[key]), _bits(sb[key])), f"{wl.name} step {k}: {key} differs"
        for key in ("packed_w", "scale_w", "packed_s", "scale_s"):
            assert torch.equal(_bits(ba[key]), _bits(bb[key])), f"{wl.name} step {k}: {key} differs"
        print(f"  {wl.name} step {k}: every output bit-identical", flush=True)
    ctx.close()
    del runs, gbuf
    torch.cuda.empty_cache()


def test_noalloc_equals_step_residual_on_shrinking_inputs():
    # 1: nearly the whole buffer (64 workers, one tensor of 7000 tiles plus a ragged one)
    near = _wl("near_max_w64", (7000 * TILE - 5, 1000), 64)
    assert STATIC_BYTES - 4 * 2**20 < _need(near.numel, 64) <= STATIC_BYTES
    _compare_entry_points(near, 2)
    # 2: the BERT-Large-shaped list (8 workers), the benchmark's workload
    _compare_entry_points(WORKLOADS["bert_large"], 2)
    # 3: a small ragged list with the trust-ratio update (its ratios sit in the buffer too)
    _compare_entry_points(_wl("ragged_w3", (1, 63, 64, 65, 1000, 8191, 8192, 8193, 20000), 3, steps=3), 3,
                          trust_wd=0.01)


def test_noalloc_rejects_a_list_beyond_the_buffer():
    over = _wl("over_max_w64", (7400 * TILE,), 64)
    assert _need(over.numel, 64) > STATIC_BYTES
    ctx = OneBitAdam(over.numel, over.workers, "f32", over.beta1, over.eps)
    st, b = init_state(over, "cuda"), ctx.alloc("cuda")
    g = grads_for_step(over, 0, "cuda")
    before = st["p"].clone()
    with pytest.raises(OneBitError) as err:
        ctx.step_residual(True, g, st["m"], st["v"], st["p"], st["err_w"], st["err_s"], b["packed_w"], b["scale_w"],
                          b["packed_s"], b["scale_s"], over.lr, noalloc=True)
    assert err.value.status == OB_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.equal(st["p"], before) and not b["packed_w"].any()   # nothing was enqueued
    ctx.close()
    del st, b, g, before
    torch.cuda.empty_cache()
