"""Pins of the oracle against things other than itself.

Each pin_* function raises AssertionError when the oracle disagrees with
exact rational arithmetic (tests/exact.py), brute force on tiny inputs, a
closed form, a hand-derived worked example (tests/golden/), an invariant of
the method, or an independent library routine (math.fsum, torch.optim.Adam).
The functions call the oracle through its module attributes so that the
mutation test can swap a planted mistake into the oracle and check that some
pin catches it.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

import oracle.onebit as ob
from exact import f32_add, f32_div, f32_mul, f32_sqrt, f32_sub, frac, round_f32
from golden_io import floats, ints, load

F32 = np.float32


def _rng(seed):
    return np.random.default_rng(seed)


def _wide_f32(rng, n):
    """fp32 values of random sign spanning many binades, with some zeros and subnormals."""
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.integers(-30, 30, n)
    x = (mant * np.exp2(expo.astype(np.float64))).astype(np.float32)
    x *= np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
    if n >= 8:
        x[rng.integers(0, n, max(1, n // 50))] = 0.0
        x[rng.integers(0, n, max(1, n // 50))] = np.float32(-0.0)
        x[rng.integers(0, n, max(1, n // 100))] = np.float32(3e-42)   # subnormal
    return x


# ---------------------------------------------------------------------------
# hand-derived worked examples
# ---------------------------------------------------------------------------

def pin_golden_compress():
    g = load("compress_layout.txt")
    for case in ("a", "c", "d"):
        x = np.array(floats(g[f"{case}.x"]), dtype=np.float32)
        if case == "a":
            x[3] = np.float32(-0.0)      # the text "-0" parses as +0.0 in some readers
        msg, e = ob.error_compensated_compress(x)
        assert [int(w) for w in msg.words] == ints(g[f"{case}.word"]), case
        assert float(msg.scale) == floats(g[f"{case}.scale"])[0], case
        assert e.tolist() == floats(g[f"{case}.err"]), case
    n = int(g["b.n"][0])
    x = -np.ones(n, dtype=np.float32)
    x[ints(g["b.positive"])] = 1.0
    msg, e = ob.error_compensated_compress(x)
    assert [int(w) for w in msg.words] == ints(g["b.word"])
    assert float(msg.scale) == floats(g["b.scale"])[0]
    assert np.all(e == 0)


def pin_golden_two_step():
    g = load("worked_two_workers.txt")
    beta1, lr, eps = (floats(g[k])[0] for k in ("beta1", "lr", "eps"))
    f = lambda k: np.array(floats(g[k]), dtype=np.float32)  # noqa: E731
    st = ob.TensorState(p=f("p0"), m=np.zeros(2, np.float32), v=f("v"),
                        err_s=np.zeros(2, np.float32), err_w=np.zeros((2, 2), np.float32))
    for step in ("step1", "step2"):
        grads = np.stack([f(step + ".g0"), f(step + ".g1")])
        out = ob.compression_step(st, grads, beta1, lr, eps)
        for w in range(2):
            assert [int(x) for x in out.worker_msgs[w].words] == ints(g[f"{step}.word{w}"]), (step, w)
            assert float(out.worker_msgs[w].scale) == floats(g[f"{step}.scale{w}"])[0], (step, w)
            assert out.state.err_w[w].tolist() == floats(g[f"{step}.err{w}"]), (step, w)
        assert [int(x) for x in out.server_msg.words] == ints(g[step + ".server_word"]), step
        assert float(out.server_msg.scale) == floats(g[step + ".server_scale"])[0], step
        assert out.state.err_s.tolist() == floats(g[step + ".err_s"]), step
        assert out.state.m.tolist() == floats(g[step + ".m"]), step
        assert out.state.p.tolist() == floats(g[step + ".p"]), step
        st = out.state


# ---------------------------------------------------------------------------
# signs and packing: brute force
# ---------------------------------------------------------------------------

def pin_sign_special_values():
    x = np.array([0.0, -0.0, 1e-45, -1e-45, np.inf, -np.inf, np.nan, 1.0, -1.0], dtype=np.float32)
    assert ob.sign_bits(x).tolist() == [True, True, True, False, True, False, False, True, False]


def pin_pack_brute_force():
    rng = _rng(1)
    # every pattern of up to 10 bits
    for n in range(1, 11):
        for pat in range(1 << n):
            bits = np.array([(pat >> k) & 1 for k in range(n)], dtype=bool)
            words = ob.pack_signs(bits)
            assert len(words) == 1 and int(words[0]) == pat
    # random patterns across word boundaries: word j bit k <-> element 64 j + k
    for n in (63, 64, 65, 127, 128, 129, 1000, 4097):
        bits = rng.random(n) < 0.5
        ref = [0] * ((n + 63) // 64)
        for i in range(n):
            if bits[i]:
                ref[i // 64] |= 1 << (i % 64)
        assert [int(w) for w in ob.pack_signs(bits)] == ref, n
        assert ob.unpack_signs(ob.pack_signs(bits), n).tolist() == bits.tolist(), n


# ---------------------------------------------------------------------------
# sum of squares and the scale: exact arithmetic and a library routine
# ---------------------------------------------------------------------------

def pin_sum_of_squares_fsum():
    rng = _rng(2)
    for n in (1, 2, 3, 64, 1000, 12345, 100003):
        x = _wide_f32(rng, n)
        ref = math.fsum((x.astype(np.float64) ** 2).tolist())   # squares of fp32 are exact in fp64
        assert ob.sum_of_squares(x) == ref, n
    x = rng.standard_normal(1 << 18).astype(np.float32) * np.float32(1e-3)
    assert ob.sum_of_squares(x) == math.fsum((x.astype(np.float64) ** 2).tolist())


def pin_sum_of_squares_fraction():
    rng = _rng(3)
    for n in (1, 5, 17, 300):
        x = _wide_f32(rng, n)
        exact = sum((frac(v) ** 2 for v in x), Fraction(0))
        assert ob.sum_of_squares(x) == float(exact), n   # float(Fraction) rounds correctly


def pin_scale_is_nearest_rms():
    """The scale is the fp32 value nearest the true RMS sqrt(sum x^2 / n)."""
    rng = _rng(4)
    for trial in range(300):
        n = int(rng.integers(1, 200))
        x = _wide_f32(rng, n) if trial % 2 else rng.standard_normal(n).astype(np.float32)
        s = ob.onebit_scale(x)
        q = sum((frac(v) ** 2 for v in x), Fraction(0)) / n
        lo = np.nextafter(s, np.float32(0))
        hi = np.nextafter(s, np.float32(np.inf))
        mid_lo = (frac(lo) + frac(s)) / 2
        mid_hi = (frac(s) + frac(hi)) / 2
        assert (s == 0 and q == 0) or (mid_lo ** 2 <= q <= mid_hi ** 2), (trial, s)


def pin_scale_closed_forms():
    rng = _rng(5)
    for _ in range(50):
        n = int(rng.integers(1, 5000))
        a = np.float32(abs(rng.standard_normal()) * 10.0 ** rng.integers(-20, 20))
        x = np.where(rng.random(n) < 0.5, a, -a).astype(np.float32)
        msg, e = ob.error_compensated_compress(x)
        assert msg.scale == a          # every |x_i| = a  ->  RMS = a
        assert np.all(e == 0)
    assert ob.onebit_scale(np.zeros(77, np.float32)) == 0
    for v in (np.float32(-3.25), np.float32(1e-40), np.float32(7e30)):
        assert ob.onebit_scale(np.array([v])) == abs(v)
    assert np.isnan(ob.onebit_scale(np.array([1.0, np.nan], np.float32)))
    assert np.isnan(ob.onebit_scale(np.array([1.0, np.inf], np.float32)))


# ---------------------------------------------------------------------------
# error feedback: the error is exactly x minus the reconstruction
# ---------------------------------------------------------------------------

def pin_error_feedback_exact():
    rng = _rng(6)
    for n in (1, 65, 999):
        x = _wide_f32(rng, n)
        msg, e = ob.error_compensated_compress(x)
        s = msg.scale
        rec = ob.OneBitCompressor.decompress(msg)
        for i in range(n):
            d = s if x[i] >= 0 else -s
            assert rec[i] == d and np.signbit(rec[i]) == np.signbit(d)
            assert e[i] == f32_sub(x[i], d), (n, i)


def pin_telescoping():
    """sum_t C(x_t) + e_T = sum_t m_t for one worker, within the accumulated rounding."""
    rng = _rng(7)
    n, T = 513, 12
    e = np.zeros(n, np.float32)
    sent = np.zeros(n, np.float64)
    pushed = np.zeros(n, np.float64)
    bound = np.zeros(n, np.float64)
    for _ in range(T):
        m_t = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        x = m_t + e
        msg, e = ob.error_compensated_compress(x)
        sent += ob.OneBitCompressor.decompress(msg).astype(np.float64)
        pushed += m_t.astype(np.float64)
        bound += np.spacing(np.abs(x)).astype(np.float64) + np.spacing(np.abs(e)).astype(np.float64)
    assert np.all(np.abs(sent + e.astype(np.float64) - pushed) <= bound)
    # and the error does not grow without bound (it is the residual of a contraction)
    assert np.max(np.abs(e)) < 10 * np.max(np.abs(pushed)) / T + 1e-2


def pin_step_telescoping():
    """Through whole steps, what each worker sent plus its final error equals
    the sum of its momenta (c1*m_{t-1} + c2*g_w,t, m_{t-1} the shared momentum
    entering step t), and what the server sent (the new momenta) plus its final
    error equals the sum of the averaged worker messages; both within the
    accumulated fp32 rounding."""
    rng = _rng(16)
    n, W, T, beta1 = 300, 3, 8, 0.9
    st = ob.TensorState(np.zeros(n, np.float32), np.zeros(n, np.float32), np.ones(n, np.float32),
                        np.zeros(n, np.float32), np.zeros((W, n), np.float32))
    sent_w = np.zeros((W, n)); pushed_w = np.zeros((W, n)); bound_w = np.zeros((W, n))
    sent_s = np.zeros(n); pushed_s = np.zeros(n); bound_s = np.zeros(n)
    for _ in range(T):
        g = (rng.standard_normal((W, n)) * 1e-3).astype(np.float32)
        out = ob.compression_step(st, g, beta1, 1e-4, 1e-8)
        dec = np.stack([ob.OneBitCompressor.decompress(mm).astype(np.float64) for mm in out.worker_msgs])
        for w in range(W):
            mw = beta1 * st.m.astype(np.float64) + (1 - beta1) * g[w].astype(np.float64)
            sent_w[w] += dec[w]
            pushed_w[w] += mw
            bound_w[w] += 4 * np.spacing(np.abs(mw).astype(np.float32)) + 2 * np.spacing(
                np.abs(out.state.err_w[w])) + np.spacing(np.abs(st.err_w[w]))
        y = dec.mean(axis=0)
        sent_s += out.state.m.astype(np.float64)
        pushed_s += y
        bound_s += 2 * W * np.spacing(np.abs(y).astype(np.float32)) + 2 * np.spacing(
            np.abs(out.state.err_s)) + np.spacing(np.abs(st.err_s))
        st = out.state
    assert np.all(np.abs(sent_w + st.err_w - pushed_w) <= bound_w)
    assert np.all(np.abs(sent_s + st.err_s - pushed_s) <= bound_s)


# ---------------------------------------------------------------------------
# worker momentum, server average and update: each fp32 operation rounds once
# ---------------------------------------------------------------------------

def pin_worker_momentum_rounding():
    rng = _rng(8)
    n = 400
    m = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    for beta1 in (0.9, 0.5, 0.99, 0.0):
        out = ob.worker_momentum(m, g, beta1)
        c1 = np.float32(beta1)
        c2 = round_f32(Fraction(1) - Fraction(beta1))   # exact 1 - beta1, rounded once to fp32
        for i in range(n):
            ref = f32_add(f32_mul(c1, m[i]), f32_mul(c2, g[i]))
            assert out[i] == ref, (beta1, i)


def pin_bf16_widening():
    rng = _rng(9)
    u = rng.integers(0, 1 << 16, 5000, dtype=np.uint32).astype(np.uint16)
    out = ob.widen_grad(u)
    for k in range(0, 5000, 7):
        bits = int(u[k])
        sign = -1.0 if bits >> 15 else 1.0
        expo = (bits >> 7) & 0xFF
        mant = bits & 0x7F
        if expo == 0xFF:
            assert (np.isnan(out[k]) if mant else out[k] == sign * np.inf)
            continue
        val = sign * (mant / 128.0) * 2.0 ** -126 if expo == 0 else sign * (1 + mant / 128.0) * 2.0 ** (expo - 127)
        assert out[k] == np.float32(val), bits


def pin_server_average_exact():
    rng = _rng(10)
    n = 300
    for W in (1, 2, 3, 4, 7, 8):
        xs = [(rng.standard_normal(n) * 10.0 ** rng.integers(-4, 2)).astype(np.float32) for _ in range(W)]
        msgs = [ob.OneBitCompressor.compress(x) for x in xs]
        y = ob.server_average(msgs)
        for i in range(0, n, 3):
            acc = np.float32(0.0)
            for w in range(W):
                d = msgs[w].scale if xs[w][i] >= 0 else -msgs[w].scale
                acc = f32_add(acc, d)
            assert y[i] == f32_div(acc, np.float32(W)), (W, i)


def pin_update_rounding():
    rng = _rng(11)
    n = 300
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = np.exp(rng.standard_normal(n) * 2 - 14).astype(np.float32)
    for lr, eps in ((1e-4, 1e-8), (0.5, 1e-3)):
        out = ob.preconditioned_update(p, m, v, lr, eps)
        for i in range(n):
            d = f32_add(f32_sqrt(v[i]), np.float32(eps))
            ref = f32_sub(p[i], f32_mul(np.float32(lr), f32_div(m[i], d)))
            assert out[i] == ref, (lr, i)


# ---------------------------------------------------------------------------
# reductions of the whole step to textbook methods and special cases
# ---------------------------------------------------------------------------

def pin_identity_compressor_is_momentum_sgd():
    """Without compression the step is momentum SGD on the worker-averaged
    gradient, preconditioned by 1/(sqrt(v)+eps); compared with a float64 loop."""
    rng = _rng(12)
    n, W, T = 257, 5, 6
    beta1, lr, eps = 0.9, 0.3, 1e-3
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    v = (rng.standard_normal(n) * 1e-3).astype(np.float32) ** 2 + np.float32(1e-12)
    st = ob.TensorState(p.copy(), np.zeros(n, np.float32), v, np.zeros(n, np.float32),
                        np.zeros((W, n), np.float32))
    m64 = np.zeros(n)
    p64 = p.astype(np.float64)
    for _ in range(T):
        g = (rng.standard_normal((W, n)) * 1e-3).astype(np.float32)
        out = ob.compression_step(st, g, beta1, lr, eps, comp=ob.IdentityCompressor)
        m64 = beta1 * m64 + (1 - beta1) * g.astype(np.float64).mean(axis=0)
        step64 = lr * m64 / (np.sqrt(v.astype(np.float64)) + eps)
        p64 = p64 - step64
        assert np.allclose(out.state.m, m64, rtol=1e-5, atol=1e-9)
        assert np.allclose(st.p - out.state.p, step64, rtol=1e-4, atol=1e-9)
        assert np.all(out.state.err_w == 0) and np.all(out.state.err_s == 0)
        st = out.state
    assert np.allclose(st.p, p64, rtol=1e-5, atol=1e-7)


def pin_single_worker_first_step():
    """W = 1 from zero errors: the server re-compresses +-s_0, which is its own
    1-bit code, so the server error stays exactly 0 and m = s_0 * sign(x_0)."""
    rng = _rng(13)
    for n in (1, 64, 1000, 4099):
        g = (rng.standard_normal((1, n)) * 1e-3).astype(np.float32)
        m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        st = ob.TensorState(np.zeros(n, np.float32), m0, np.ones(n, np.float32),
                            np.zeros(n, np.float32), np.zeros((1, n), np.float32))
        out = ob.compression_step(st, g, 0.9, 1e-4, 1e-8)
        x0 = ob.worker_momentum(m0, g[0], 0.9)
        s0 = out.worker_msgs[0].scale
        assert out.server_msg.scale == s0
        assert np.all(out.state.err_s == 0)
        assert np.array_equal(out.state.m, np.where(x0 >= 0, s0, -s0).astype(np.float32))
        assert np.array_equal(out.server_msg.words, out.worker_msgs[0].words)


def pin_zero_gradients():
    n, W = 130, 3
    p = np.linspace(-1, 1, n).astype(np.float32)
    st = ob.TensorState(p.copy(), np.zeros(n, np.float32), np.full(n, 0.01, np.float32),
                        np.zeros(n, np.float32), np.zeros((W, n), np.float32))
    out = ob.compression_step(st, np.zeros((W, n), np.float32), 0.9, 1e-4, 1e-8)
    assert np.array_equal(out.state.p, p)
    full = [0xFFFFFFFFFFFFFFFF, 0xFFFFFFFFFFFFFFFF, 0x3]       # 130 bits set, padding 0
    for msg in out.worker_msgs + [out.server_msg]:
        assert msg.scale == 0 and [int(w) for w in msg.words] == full


def pin_identical_workers():
    """Equal messages from all workers average back to that message: exactly
    when the scale is a power of two and W a power of two, within one ulp otherwise."""
    rng = _rng(14)
    n = 200
    for W in (2, 4, 8):
        x = np.where(rng.random(n) < 0.5, 0.25, -0.25).astype(np.float32)
        msg = ob.OneBitCompressor.compress(x)
        y = ob.server_average([msg] * W)
        assert np.array_equal(y, ob.OneBitCompressor.decompress(msg))
    for W in (3, 5, 8):
        x = rng.standard_normal(n).astype(np.float32)
        msg = ob.OneBitCompressor.compress(x)
        y = ob.server_average([msg] * W)
        ref = ob.OneBitCompressor.decompress(msg)
        assert np.all(np.abs(y - ref) <= np.spacing(np.abs(ref)))


def pin_warmup_matches_torch_adam():
    """Warmup m and v equal torch.optim.Adam's exp_avg / exp_avg_sq on the
    averaged gradient; the parameter equals Adam's once Adam's bias correction
    is undone through its lr and eps (lr' = lr*bc1/sqrt(bc2), eps' = eps/sqrt(bc2))."""
    import torch
    rng = _rng(15)
    n, W, T = 300, 4, 5
    beta1, beta2, lr, eps = 0.9, 0.999, 1e-3, 1e-6
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    st = ob.TensorState(p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32),
                        np.zeros(n, np.float32), np.zeros((W, n), np.float32))
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.Adam([tp], lr=lr, betas=(beta1, beta2), eps=eps)
    for t in range(1, T + 1):
        g = (rng.standard_normal((W, n)) * 1e-3).astype(np.float32)
        p_before = st.p.copy()
        st = ob.warmup_step(st, g, beta1, beta2, lr, eps)
        gbar = g.astype(np.float64).mean(axis=0).astype(np.float32)
        bc1, bc2 = 1 - beta1 ** t, 1 - beta2 ** t
        opt.param_groups[0]["lr"] = lr * bc1 / math.sqrt(bc2)
        opt.param_groups[0]["eps"] = eps / math.sqrt(bc2)
        tp.grad = torch.from_numpy(gbar)
        tbefore = tp.detach().clone().numpy()
        opt.step()
        s = opt.state[tp]
        assert np.allclose(st.m, s["exp_avg"].numpy(), rtol=1e-5, atol=1e-10)
        assert np.allclose(st.v, s["exp_avg_sq"].numpy(), rtol=1e-5, atol=1e-14)
        assert np.allclose(p_before - st.p, tbefore - tp.detach().numpy(), rtol=2e-3, atol=1e-9)


def pin_message_format_accounting():
    """1 bit per element plus 32 bits per tensor: about 32x smaller than fp32."""
    assert ob.message_bytes(1) == 12 and ob.message_bytes(64) == 12 and ob.message_bytes(65) == 20
    n = 1 << 20
    assert abs(4 * n / ob.message_bytes(n) - 32.0) < 0.01


def pin_chunk_partition():
    """Chunks tile each tensor exactly once, in whole 8192-element blocks (the
    last may be shorter), at most C of them, and C = 1 is the whole tensor."""
    for n in (1, 64, 8191, 8192, 8193, 20000, 100003, 1 << 20):
        assert ob.chunk_bounds(n, 1) == [(0, n)]
        for C in (2, 3, 4, 8, 64):
            b = ob.chunk_bounds(n, C)
            assert b[0][0] == 0 and b[-1][1] == n and len(b) <= C
            assert all(b[i][1] == b[i + 1][0] for i in range(len(b) - 1))
            assert all((hi - lo) % 8192 == 0 for lo, hi in b[:-1])
            assert len({hi - lo for lo, hi in b[:-1]}) <= 1
    # C chunks of a tensor of exactly C blocks are the blocks themselves
    assert ob.chunk_bounds(4 * 8192, 4) == [(i * 8192, (i + 1) * 8192) for i in range(4)]


def pin_chunked_scales_closed_form():
    """With |x| = a_j on chunk j, chunk j's scale is a_j and the error is 0;
    with one chunk the message equals the per-tensor message."""
    rng = _rng(17)
    n, C = 3 * 8192 + 100, 4
    bounds = ob.chunk_bounds(n, C)
    mags = [np.float32(0.5), np.float32(3.0), np.float32(1e-3), np.float32(7.25)]
    x = np.empty(n, np.float32)
    for (lo, hi), a in zip(bounds, mags):
        x[lo:hi] = np.where(rng.random(hi - lo) < 0.5, a, -a)
    comp = ob.ChunkedOneBitCompressor(C)
    msg, e = ob.error_compensated_compress(x, comp)
    assert msg.scales.tolist() == [float(a) for a in mags[:len(bounds)]]
    assert np.all(e == 0)
    y = rng.standard_normal(n).astype(np.float32)
    one = ob.ChunkedOneBitCompressor(1).compress(y)
    ref = ob.OneBitCompressor.compress(y)
    assert np.array_equal(one.words, ref.words) and one.scales[0] == ref.scale
    assert np.array_equal(ob.ChunkedOneBitCompressor.decompress(one), ob.OneBitCompressor.decompress(ref))
    # each chunk's scale is that chunk's own RMS
    msg = comp.compress(y)
    for (lo, hi), s in zip(msg.bounds, msg.scales):
        assert s == ob.onebit_scale(y[lo:hi])


def pin_chunked_server_step():
    """A C-way partitioned server keeps the step's invariants: W = 1 at the
    first step still leaves e_s = 0 when every chunk of the worker message
    has one magnitude, and the server error telescopes."""
    rng = _rng(18)
    n = 2 * 8192 + 300
    g = np.empty((1, n), np.float32)
    g[0] = np.where(rng.random(n) < 0.5, 1.0, -1.0).astype(np.float32)
    st = ob.TensorState(np.zeros(n, np.float32), np.zeros(n, np.float32), np.ones(n, np.float32),
                        np.zeros(n, np.float32), np.zeros((1, n), np.float32))
    out = ob.compression_step(st, g, 0.9, 1e-4, 1e-8, server_comp=ob.ChunkedOneBitCompressor(3))
    assert np.all(out.state.err_s == 0)
    assert len(out.server_msg.scales) == 3
    assert np.all(np.abs(out.state.m) == out.worker_msgs[0].scale)


def pin_trust_ratio():
    """The trust ratio is the fp32 value nearest ||p|| / ||u|| (exact rational
    midpoints), scales exactly with p, and is 1 for a zero tensor."""
    rng = _rng(19)
    for trial in range(40):
        n = int(rng.integers(1, 300))
        p = (rng.standard_normal(n) * 0.02).astype(np.float32)
        u = (rng.standard_normal(n) * 10.0 ** rng.integers(-4, 2)).astype(np.float32)
        r = ob.trust_ratio(p, u)
        q2 = sum((frac(x) ** 2 for x in p), Fraction(0)) / sum((frac(x) ** 2 for x in u), Fraction(0))
        lo, hi = np.nextafter(r, np.float32(0)), np.nextafter(r, np.float32(np.inf))
        mid_lo, mid_hi = (frac(lo) + frac(r)) / 2, (frac(r) + frac(hi)) / 2
        assert mid_lo ** 2 <= q2 <= mid_hi ** 2, trial
        assert ob.trust_ratio(p * np.float32(8.0), u) == r * np.float32(8.0)
        assert ob.trust_ratio(p, u * np.float32(0.25)) == r * np.float32(4.0)
    assert ob.trust_ratio(np.zeros(5, np.float32), np.ones(5, np.float32)) == 1.0
    assert ob.trust_ratio(np.ones(5, np.float32), np.zeros(5, np.float32)) == 1.0


def pin_trust_ratio_update():
    """p - lr*(r*u) with every fp32 operation rounded once, and when
    ||p|| = ||u|| the ratio is 1 and the step is the plain preconditioned step."""
    rng = _rng(20)
    n = 200
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = np.exp(rng.standard_normal(n) * 2 - 14).astype(np.float32)
    for wd in (0.0, 0.01):
        out = ob.trust_ratio_update(p, m, v, 1e-3, 1e-8, wd)
        u = np.array([f32_div(m[i], f32_add(f32_sqrt(v[i]), np.float32(1e-8))) for i in range(n)], np.float32)
        if wd > 0:
            u = np.array([f32_add(u[i], f32_mul(np.float32(wd), p[i])) for i in range(n)], np.float32)
        r = ob.trust_ratio(p, u)
        for i in range(n):
            assert out[i] == f32_sub(p[i], f32_mul(np.float32(1e-3), f32_mul(r, u[i]))), (wd, i)
    # |p_i| = |u_i| = 1 everywhere -> r = 1 -> identical to the plain step
    ones = np.where(rng.random(n) < 0.5, 1.0, -1.0).astype(np.float32)
    v1 = np.full(n, 0.25, np.float32)
    m1 = ones * np.float32(0.5)          # u = m / (sqrt(v) + 0) = +-1 with eps = 0
    assert np.array_equal(ob.trust_ratio_update(ones, m1, v1, 0.1, 0.0),
                          ob.preconditioned_update(ones, m1, v1, 0.1, 0.0))


def pin_golden_cltk():
    """Hand-derived two-exchange example (tests/golden/cltk_worked.txt): ties at
    the boundary in both steps, the leader cycling from worker 0 to worker 1."""
    g = load("cltk_worked.txt")
    k = ints(g["k"])[0]
    f = lambda key: np.array(floats(g[key]), dtype=np.float32)  # noqa: E731
    mem = np.zeros((3, 6), np.float32)
    for step in (0, 1):
        grads = np.stack([f(f"step{step}.g{w}") for w in range(3)])
        out = ob.cltk_step(mem, grads, step, k)
        assert out.index.tolist() == ints(g[f"step{step}.index"]), step
        for w in range(3):
            assert out.values[w].tolist() == floats(g[f"step{step}.values{w}"]), (step, w)
            assert out.memory[w].tolist() == floats(g[f"step{step}.mem{w}"]), (step, w)
        assert out.average.tolist() == floats(g[f"step{step}.average"]), step
        mem = out.memory


def pin_cltk_brute_force():
    """Top-k positions by a pure-Python sort of (|x|, -index), ties included."""
    rng = _rng(21)
    for trial in range(30):
        W, n = int(rng.integers(1, 5)), int(rng.integers(1, 80))
        mem = rng.choice(np.array([-2, -1, -0.0, 0, 1, 2, 3], np.float32), (W, n))
        g = rng.choice(np.array([-1, 0, 1, 0.5], np.float32), (W, n))
        k = int(rng.integers(1, n + 1))
        step = int(rng.integers(0, 10))
        out = ob.cltk_step(mem, g, step, k)
        x = [[float(np.float32(mem[w][i] + g[w][i])) for i in range(n)] for w in range(W)]
        lead = x[step % W]
        ranked = sorted(range(n), key=lambda i: (-abs(lead[i]), i))
        assert out.index.tolist() == sorted(ranked[:k]), trial
        for w in range(W):
            assert out.values[w].tolist() == [x[w][i] for i in sorted(ranked[:k])]
            kept = set(ranked[:k])
            assert out.memory[w].tolist() == [0.0 if i in kept else x[w][i] for i in range(n)]


def pin_cltk_commutative():
    """The page's claim: with one index set for all workers, the average of
    the compressed messages is the compression of the average (same positions),
    so the exchange is an all-reduce; and memory + message = x exactly."""
    rng = _rng(22)
    W, n, k = 4, 3000, 40
    mem = (rng.standard_normal((W, n)) * 1e-3).astype(np.float32)
    g = (rng.standard_normal((W, n)) * 1e-3).astype(np.float32)
    for step in range(W + 1):
        out = ob.cltk_step(mem, g, step, k)
        x = mem + g
        dense_avg = np.zeros(n, np.float32)
        for w in range(W):
            dense_avg = dense_avg + x[w]
        dense_avg = dense_avg / np.float32(W)
        assert np.array_equal(out.average, dense_avg[out.index])
        for w in range(W):
            back = out.memory[w].copy()
            back[out.index] = out.values[w]
            assert np.array_equal(back, x[w])
        # the leader's kept entries dominate its dropped ones
        lead = np.abs(x[step % W])
        dropped = np.delete(lead, out.index)
        assert lead[out.index].min() >= (dropped.max() if dropped.size else 0)
    assert ob.cltk_k(100, 0.01) == 1 and ob.cltk_k(1000, 0.01) == 10 and ob.cltk_k(5, 0.01) == 1


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
