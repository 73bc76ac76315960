"""Pins of the C++ oracle (oracle/onebit_ref.cpp), CPU only.

The C++ oracle is a second, independent implementation of the compression
step.  It is pinned to things other than itself: math.fsum (the correctly
rounded sum; an fp32 square is exact in fp64, so fsum of the squares is the
exact sum rounded once), hand-made rounding ties, a pure-Python packer, the
hand-derived worked example in tests/golden/, and, element by element and bit
for bit, the numpy oracle (itself pinned by tests/pins.py) over ragged sizes,
several worker counts, bf16 gradients, special values and chained steps.
"""
import math

import numpy as np
import pytest

import oracle.onebit as ob
import oracle.ref as ref
from golden_io import floats, ints, load


def _rng(seed):
    return np.random.default_rng(seed)


def _fsum_sq(x):
    return math.fsum(float(v) * float(v) for v in np.asarray(x, dtype=np.float32).ravel())


def _random_finite(rng, n):
    """fp32 values with every exponent, subnormals included (random bit patterns)."""
    u = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    return np.where(np.isfinite(x), x, np.float32(1.5)).astype(np.float32)


@pytest.mark.parametrize("kind", ["normal", "wide", "subnormal", "mixed"])
def test_sum_of_squares_is_fsum(kind):
    rng = _rng(11)
    for n in (1, 2, 63, 1000, 20000):
        if kind == "normal":
            x = rng.normal(0.0, 1e-3, n).astype(np.float32)
        elif kind == "wide":
            x = _random_finite(rng, n)
        elif kind == "subnormal":
            x = (rng.integers(-(1 << 23), 1 << 23, n).astype(np.int64) * 2.0 ** -149).astype(np.float32)
        else:
            x = np.concatenate([rng.normal(0, 1e30, n // 2), rng.normal(0, 1e-30, n - n // 2)]).astype(np.float32)
        assert ref.sum_of_squares(x) == _fsum_sq(x), (kind, n)
        assert ref.sum_of_squares(x) == ob.sum_of_squares(x), (kind, n)


def test_sum_of_squares_rounding_ties():
    t = np.float32(2.0 ** -27)   # t^2 = 2^-54, a quarter of an ulp of 1
    one = np.float32(1.0)
    cases = {
        (one, t): 1.0,                              # below half an ulp: down
        (one, t, t): 1.0,                           # exactly half, even: stays
        (one, t, t, t): 1.0 + 2.0 ** -52,           # above half: up
        (np.float32(1.0 + 2.0 ** -23), t, t): None,  # a longer significand: checked against fsum only
    }
    for xs, want in cases.items():
        x = np.array(xs, dtype=np.float32)
        got = ref.sum_of_squares(x)
        assert got == _fsum_sq(x), xs
        if want is not None:
            assert got == want, xs
    # sticky bit: half an ulp plus a tiny remainder rounds up
    x = np.array([1.0, 2.0 ** -27, 2.0 ** -27, 2.0 ** -60], dtype=np.float32)
    assert ref.sum_of_squares(x) == 1.0 + 2.0 ** -52 == _fsum_sq(x)


def test_scale_closed_forms_and_nonfinite():
    for a in (0.75, 3.0, 2.0 ** -70, 2.0 ** 60, 1e-45):
        for n in (1, 5, 64, 1001):
            x = np.full(n, np.float32(a))
            x[::3] = -x[::3]
            assert ref.scale(x) == np.float32(a), (a, n)
    assert ref.scale(np.zeros(10, np.float32)) == 0.0
    for bad in (np.nan, np.inf, -np.inf):
        x = np.ones(70, np.float32)
        x[33] = bad
        assert math.isnan(ref.sum_of_squares(x)) and np.isnan(ref.scale(x))
    x = np.array([3.0, 4.0], np.float32)
    assert ref.scale(x) == np.float32(math.sqrt(12.5))


def test_pack_signs_brute_force():
    rng = _rng(3)
    x = np.array([0.0, -0.0, 1e-45, -1e-45, np.inf, -np.inf, np.nan, 1.0, -1.0], dtype=np.float32)
    assert int(ref.pack_signs(x)[0]) == sum(1 << k for k, b in enumerate([1, 1, 1, 0, 1, 0, 0, 1, 0]) if b)
    for n in (1, 63, 64, 65, 127, 129, 1000, 4097):
        x = rng.normal(size=n).astype(np.float32)
        want = [0] * ((n + 63) // 64)
        for i in range(n):
            if x[i] >= 0:
                want[i // 64] |= 1 << (i % 64)
        assert [int(w) for w in ref.pack_signs(x)] == want, n


def test_golden_two_step():
    g = load("worked_two_workers.txt")
    beta1, lr, eps = (floats(g[k])[0] for k in ("beta1", "lr", "eps"))
    f = lambda k: np.array(floats(g[k]), dtype=np.float32)  # noqa: E731
    p, m, v = f("p0"), np.zeros(2, np.float32), f("v")
    err_s, err_w = np.zeros(2, np.float32), np.zeros((2, 2), np.float32)
    for step in ("step1", "step2"):
        grads = np.stack([f(step + ".g0"), f(step + ".g1")])
        out = ref.compression_step(p, m, v, err_s, err_w, grads, beta1, lr, eps)
        for w in range(2):
            assert [int(x) for x in out["packed_w"][w]] == ints(g[f"{step}.word{w}"]), (step, w)
            assert float(out["scale_w"][w]) == floats(g[f"{step}.scale{w}"])[0], (step, w)
            assert out["err_w"][w].tolist() == floats(g[f"{step}.err{w}"]), (step, w)
        assert [int(x) for x in out["packed_s"]] == ints(g[step + ".server_word"]), step
        assert float(out["scale_s"]) == floats(g[step + ".server_scale"])[0], step
        assert out["err_s"].tolist() == floats(g[step + ".err_s"]), step
        assert out["m"].tolist() == floats(g[step + ".m"]), step
        assert out["p"].tolist() == floats(g[step + ".p"]), step
        p, m, err_s, err_w = out["p"], out["m"], out["err_s"], out["err_w"]


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _same(a, b):
    return np.array_equal(_bits(a), _bits(b))


@pytest.mark.parametrize("n,W,dtype", [(1, 1, "f32"), (63, 2, "f32"), (64, 3, "f32"), (65, 8, "f32"),
                                       (1000, 9, "f32"), (8193, 4, "f32"), (777, 8, "bf16"),
                                       (130, 64, "f32")])
def test_step_equals_numpy_oracle(n, W, dtype):
    """Three chained steps from the same state: every output bit-identical."""
    rng = _rng(1000 + n + W)
    beta1, lr, eps = 0.9, 1e-4, 1e-8
    st = ob.TensorState(p=rng.normal(0, 0.02, n).astype(np.float32), m=np.zeros(n, np.float32),
                        v=(np.abs(rng.normal(0, 1e-3, n)) ** 2 + 1e-12).astype(np.float32),
                        err_s=np.zeros(n, np.float32), err_w=np.zeros((W, n), np.float32))
    cst = {"p": st.p.copy(), "m": st.m.copy(), "err_s": st.err_s.copy(), "err_w": st.err_w.copy()}
    for k in range(3):
        g = rng.normal(0, 1e-3, (W, n)).astype(np.float32)
        if k == 1:   # special values: zeros, negative zeros, subnormals
            g[:, ::7] = 0.0
            g[:, 3::11] = -0.0
            g[:, 5::13] = np.float32(1e-42)
        if dtype == "bf16":
            g = (g.view(np.uint32) >> np.uint32(16)).astype(np.uint16)   # truncated bf16 patterns
        out = ob.compression_step(st, g, beta1, lr, eps)
        c = ref.compression_step(cst["p"], cst["m"], st.v, cst["err_s"], cst["err_w"], g, beta1, lr, eps)
        words, scales = ob.words_of(out.worker_msgs)
        assert _same(c["packed_w"], words) and _same(c["scale_w"], scales), k
        assert _same(c["packed_s"], out.server_msg.words) and c["scale_s"] == out.server_msg.scale, k
        for key, want in (("p", out.state.p), ("m", out.state.m), ("err_s", out.state.err_s),
                          ("err_w", out.state.err_w)):
            assert _same(c[key], want), (k, key)
        st = out.state
        cst = {key: c[key] for key in ("p", "m", "err_s", "err_w")}


def test_step_nan_gradient_matches_numpy_oracle():
    rng = _rng(5)
    n, W = 200, 3
    st = ob.TensorState(p=rng.normal(0, 0.02, n).astype(np.float32), m=np.zeros(n, np.float32),
                        v=np.full(n, 1e-6, np.float32), err_s=np.zeros(n, np.float32),
                        err_w=np.zeros((W, n), np.float32))
    g = rng.normal(0, 1e-3, (W, n)).astype(np.float32)
    g[1, 17] = np.nan
    out = ob.compression_step(st, g, 0.9, 1e-4, 1e-8)
    c = ref.compression_step(st.p, st.m, st.v, st.err_s, st.err_w, g, 0.9, 1e-4, 1e-8)
    assert np.isnan(c["scale_w"][1]) and not np.isnan(c["scale_w"][0])
    words, scales = ob.words_of(out.worker_msgs)
    assert _same(c["packed_w"], words)
    np.testing.assert_array_equal(c["scale_w"], scales)
    for key, want in (("p", out.state.p), ("m", out.state.m), ("err_s", out.state.err_s),
                      ("err_w", out.state.err_w)):
        np.testing.assert_array_equal(c[key], want, err_msg=key)


def test_rejects_bad_arguments():
    lib = ref.load()
    one = np.zeros(1, np.float32)
    w = np.zeros(1, np.uint64)
    assert lib.ref_compression_step(0, 1, one, 0.9, 1e-4, 1e-8, one, one, one, one, one, w, one, w, one) == 1
    assert lib.ref_compression_step(1, 0, one, 0.9, 1e-4, 1e-8, one, one, one, one, one, w, one, w, one) == 1


def test_single_tensor_workload_trajectory_equals_numpy_oracle():
    """The single-tensor workload (n = 2^20, W = 4, 10 steps, its seeded inputs
    generated on the CPU): the two oracles agree bit for bit after every step."""
    from synth import WORKLOADS, grads_for_step, host_slice, init_state
    wl = WORKLOADS["single_tensor_2p20"]
    n = wl.numel[0]
    st0 = init_state(wl, "cpu")
    st = ob.TensorState(*(host_slice(st0[k], 0, n) for k in ("p", "m", "v", "err_s", "err_w")))
    cst = {k: getattr(st, k).copy() for k in ("p", "m", "err_s", "err_w")}
    for k in range(wl.steps):
        g = host_slice(grads_for_step(wl, k, "cpu"), 0, n)
        out = ob.compression_step(st, g, wl.beta1, wl.lr, wl.eps)
        c = ref.compression_step(cst["p"], cst["m"], st.v, cst["err_s"], cst["err_w"], g, wl.beta1, wl.lr,
                                 wl.eps)
        words, scales = ob.words_of(out.worker_msgs)
        assert _same(c["packed_w"], words) and _same(c["scale_w"], scales), k
        assert _same(c["packed_s"], out.server_msg.words) and c["scale_s"] == out.server_msg.scale, k
        for key in ("p", "m", "err_s", "err_w"):
            assert _same(c[key], getattr(out.state, key)), (k, key)
        st = out.state
        cst = {key: c[key] for key in ("p", "m", "err_s", "err_w")}


@pytest.mark.parametrize("n,W,dtype", [(1, 1, "f32"), (65, 3, "f32"), (1000, 8, "f32"), (777, 8, "bf16"),
                                       (300, 64, "f32")])
def test_warmup_equals_numpy_oracle(n, W, dtype):
    """Three chained warmup steps from zero moments: p, m, v bit-identical."""
    rng = _rng(2000 + n + W)
    st = ob.TensorState(p=rng.normal(0, 0.02, n).astype(np.float32), m=np.zeros(n, np.float32),
                        v=np.zeros(n, np.float32), err_s=np.zeros(n, np.float32),
                        err_w=np.zeros((W, n), np.float32))
    c = {"p": st.p.copy(), "m": st.m.copy(), "v": st.v.copy()}
    for k in range(3):
        g = rng.normal(0, 1e-3, (W, n)).astype(np.float32)
        if dtype == "bf16":
            g = (g.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        st = ob.warmup_step(st, g, 0.9, 0.999, 1e-3, 1e-8)
        c = ref.warmup_step(c["p"], c["m"], c["v"], g, 0.9, 0.999, 1e-3, 1e-8)
        for key in ("p", "m", "v"):
            assert _same(c[key], getattr(st, key)), (k, key)


def test_warmup_moments_match_torch_adam():
    """The C++ warmup's m and v equal torch.optim.Adam's exp_avg and exp_avg_sq
    on the averaged gradient (torch's lerp form rounds differently: 1e-5 rel)."""
    import torch
    rng = _rng(16)
    n, W = 300, 4
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    c = {"p": p0.copy(), "m": np.zeros(n, np.float32), "v": np.zeros(n, np.float32)}
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.Adam([tp], lr=1e-3, betas=(0.9, 0.999), eps=1e-8)
    for _ in range(4):
        g = (rng.standard_normal((W, n)) * 1e-3).astype(np.float32)
        c = ref.warmup_step(c["p"], c["m"], c["v"], g, 0.9, 0.999, 1e-3, 1e-8)
        tp.grad = torch.from_numpy(g.astype(np.float64).mean(axis=0).astype(np.float32))
        opt.step()
        s = opt.state[tp]
        assert np.allclose(c["m"], s["exp_avg"].numpy(), rtol=1e-5, atol=1e-10)
        assert np.allclose(c["v"], s["exp_avg_sq"].numpy(), rtol=1e-5, atol=1e-14)


def test_cltk_golden_worked_example():
    """The hand-derived two-exchange CLT-k example in tests/golden/ (ties at the
    selection boundary in both steps, the leader moving from worker 0 to 1)."""
    g = load("cltk_worked.txt")
    k = ints(g["k"])[0]
    f = lambda key: np.array(floats(g[key]), dtype=np.float32)  # noqa: E731
    mem = np.zeros((3, 6), np.float32)
    for step in (0, 1):
        grads = np.stack([f(f"step{step}.g{w}") for w in range(3)])
        c = ref.cltk_step(mem, grads, step, k)
        assert c["index"].tolist() == ints(g[f"step{step}.index"]), step
        for w in range(3):
            assert c["values"][w].tolist() == floats(g[f"step{step}.values{w}"]), (step, w)
            assert c["memory"][w].tolist() == floats(g[f"step{step}.mem{w}"]), (step, w)
        assert c["average"].tolist() == floats(g[f"step{step}.average"]), step
        mem = c["memory"]


def test_cltk_equals_numpy_oracle_with_ties():
    """Random small tensors drawn from a few values (many ties, -0 and +0), random
    k and leader, chained exchanges: every output bit-identical to the numpy
    oracle's, which is itself pinned to a pure-Python sort."""
    rng = _rng(22)
    for _ in range(40):
        W, n = int(rng.integers(1, 6)), int(rng.integers(1, 200))
        mem = rng.choice(np.array([-2, -1, -0.0, 0, 1, 2, 3], np.float32), (W, n))
        for step in range(3):
            g = rng.choice(np.array([-1, 0, 1, 0.5, -0.0], np.float32), (W, n))
            k = int(rng.integers(1, n + 1))
            o = ob.cltk_step(mem, g, step, k)
            c = ref.cltk_step(mem, g, step, k)
            assert np.array_equal(c["index"], o.index)
            for key, want in (("values", o.values), ("average", o.average), ("memory", o.memory)):
                assert _same(c[key], want), key
            mem = o.memory


@pytest.mark.parametrize("n,W,density,dtype", [(8193, 4, 0.01, "f32"), (20000, 8, 0.1, "bf16"), (777, 3, 1.0, "f32")])
def test_cltk_equals_numpy_oracle_random(n, W, density, dtype):
    rng = _rng(3000 + n)
    mem = rng.normal(0, 1e-3, (W, n)).astype(np.float32)
    k = ob.cltk_k(n, density)
    for step in range(4):
        g = rng.normal(0, 1e-3, (W, n)).astype(np.float32)
        if dtype == "bf16":
            g = (g.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        o = ob.cltk_step(mem, g, step, k)
        c = ref.cltk_step(mem, g, step, k)
        assert np.array_equal(c["index"], o.index)
        for key, want in (("values", o.values), ("average", o.average), ("memory", o.memory)):
            assert _same(c[key], want), (step, key)
        mem = o.memory


@pytest.mark.parametrize("n,W,chunks,trust_wd", [(70001, 3, 2, None), (70001, 3, 8, None), (8193, 4, 3, None),
                                                 (100, 2, 4, None), (20000, 3, 1, 0.0), (20000, 3, 1, 0.01),
                                                 (70001, 2, 4, 0.01)])
def test_partitioned_server_and_trust_ratio_equal_numpy_oracle(n, W, chunks, trust_wd):
    """The server partitioned into chunks of whole 8192-element blocks, and the
    trust-ratio update: three chained steps, every output bit-identical to the
    numpy oracle's."""
    rng = _rng(4000 + n + chunks)
    st = ob.TensorState(p=rng.normal(0, 0.02, n).astype(np.float32), m=np.zeros(n, np.float32),
                        v=(np.abs(rng.normal(0, 1e-3, n)) ** 2 + 1e-12).astype(np.float32),
                        err_s=np.zeros(n, np.float32), err_w=np.zeros((W, n), np.float32))
    cst = {"p": st.p.copy(), "m": st.m.copy(), "err_s": st.err_s.copy(), "err_w": st.err_w.copy()}
    scomp = None if chunks == 1 else ob.ChunkedOneBitCompressor(chunks)
    for k in range(3):
        g = rng.normal(0, 1e-3, (W, n)).astype(np.float32)
        out = ob.compression_step(st, g, 0.9, 1e-4, 1e-8, server_comp=scomp, trust_ratio_wd=trust_wd)
        c = ref.compression_step(cst["p"], cst["m"], st.v, cst["err_s"], cst["err_w"], g, 0.9, 1e-4, 1e-8,
                                 server_chunks=chunks, trust_wd=trust_wd)
        words, scales = ob.words_of(out.worker_msgs)
        assert _same(c["packed_w"], words) and _same(c["scale_w"], scales), k
        want_ss = out.server_msg.scales if chunks > 1 else np.array([out.server_msg.scale], np.float32)
        assert _same(c["packed_s"], out.server_msg.words) and _same(c["scales_s"], want_ss), k
        for key in ("p", "m", "err_s", "err_w"):
            assert _same(c[key], getattr(out.state, key)), (k, key)
        st = out.state
        cst = {key: c[key] for key in ("p", "m", "err_s", "err_w")}


@pytest.mark.parametrize("dtype,chunks,trust_wd", [("f32", 1, None), ("bf16", 1, None), ("f32", 2, None),
                                                   ("f32", 1, 0.01)])
def test_in_place_flat_step_equals_per_tensor_step(dtype, chunks, trust_wd):
    """The in-place step over a padded flat list (row strides N, the layout the
    device buffers use) equals the contiguous per-tensor step bit for bit, over
    three chained steps; padding is neither read nor written."""
    rng = _rng(29)
    sizes, W = (1, 65, 8192, 8193, 20000, 70001), 3
    off = [0]
    for n in sizes:
        off.append(off[-1] + (n + 63) // 64 * 64)
    N, T = off[-1], len(sizes)
    pieces = [-(-n // (8192 * -(-(-(-n // 8192)) // chunks))) for n in sizes]
    pbase = np.concatenate([[0], np.cumsum(pieces)])
    canary = np.float32(123.5)
    flat = {k: np.full(N, canary, np.float32) for k in ("p", "m", "v", "err_s")}
    flat["err_w"] = np.full((W, N), canary, np.float32)
    per = []
    for t, n in enumerate(sizes):
        lo = off[t]
        vals = {"p": rng.normal(0, 0.02, n), "m": rng.normal(0, 1e-3, n), "v": rng.normal(0, 1e-3, n) ** 2 + 1e-12,
                "err_s": rng.normal(0, 1e-4, n)}
        for k, x in vals.items():
            flat[k][lo:lo + n] = x
        flat["err_w"][:, lo:lo + n] = rng.normal(0, 1e-4, (W, n))
        per.append({k: flat[k][..., lo:lo + n].copy() for k in flat})
    packed_w = np.zeros((W, N // 64), np.uint64)
    scale_w = np.zeros((W, T), np.float32)
    packed_s = np.zeros(N // 64, np.uint64)
    scale_s = np.zeros(pbase[-1], np.float32)
    for step in range(3):
        g32 = rng.normal(0, 1e-3, (W, N)).astype(np.float32)
        g = (g32.view(np.uint32) >> 16).astype(np.uint16) if dtype == "bf16" else g32
        for t, n in enumerate(sizes):
            lo, nw = off[t], (n + 63) // 64
            ref.compression_step_in_place(lo, n, t, g, flat["p"], flat["m"], flat["v"], flat["err_s"], flat["err_w"],
                                          packed_w, scale_w, packed_s, scale_s[pbase[t]:pbase[t + 1]], 0.9, 1e-4,
                                          1e-8, server_chunks=chunks, trust_wd=trust_wd)
            c = ref.compression_step(per[t]["p"], per[t]["m"], per[t]["v"], per[t]["err_s"], per[t]["err_w"],
                                     np.ascontiguousarray(g[:, lo:lo + n]), 0.9, 1e-4, 1e-8, server_chunks=chunks,
                                     trust_wd=trust_wd)
            w0 = lo // 64
            assert np.array_equal(packed_w[:, w0:w0 + nw], c["packed_w"]), (step, t)
            assert np.array_equal(packed_s[w0:w0 + nw], c["packed_s"]), (step, t)
            assert _same(scale_w[:, t], c["scale_w"]) and _same(scale_s[pbase[t]:pbase[t + 1]], c["scales_s"])
            for k in ("p", "m", "err_s", "err_w"):
                assert _same(flat[k][..., lo:lo + n], c[k]), (step, t, k)
            per[t].update({k: c[k] for k in ("p", "m", "err_s", "err_w")})
    for t, n in enumerate(sizes):   # padding untouched
        pad = slice(off[t] + n, off[t + 1])
        for k in flat:
            assert np.all(flat[k][..., pad] == canary), (t, k)


def test_in_place_flat_step_rejects_bad_ranges():
    W, N = 2, 128
    f = lambda *s: np.zeros(s, np.float32)   # noqa: E731
    args = dict(grads=f(W, N), p=f(N), m=f(N), v=f(N), err_s=f(N), err_w=f(W, N),
                packed_w=np.zeros((W, 2), np.uint64), scale_w=f(W, 1), packed_s=np.zeros(2, np.uint64),
                scale_s=f(1), beta1=0.9, lr=1e-4, eps=1e-8)
    with pytest.raises(ValueError):
        ref.compression_step_in_place(64, 65, 0, **args)            # past the end
    with pytest.raises(ValueError):
        ref.compression_step_in_place(1, 10, 0, **args)             # not word-aligned
    with pytest.raises(TypeError):
        bad = dict(args, err_w=f(N, W).T)                            # not contiguous
        ref.compression_step_in_place(0, 10, 0, **bad)
    ref.compression_step_in_place(64, 64, 0, **args)                # the last whole tensor fits
