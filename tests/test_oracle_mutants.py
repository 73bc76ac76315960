"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin
catches each one: a dropped term, a wrong sign or index, a transposed operand,
a wrong constant, a wrong bit order."""
import numpy as np
import pytest

import oracle.onebit as ob
import pins

F32 = np.float32


def _step_factory(no_worker_err=False, no_server_err=False, keep_old_m=False, reverse_workers=False):
    def compression_step(st, grads, beta1, lr, eps, comp=ob.OneBitCompressor):
        W = grads.shape[0]
        msgs, err_w = [], np.empty_like(st.err_w)
        for w in range(W):
            gw = grads[W - 1 - w] if reverse_workers else grads[w]
            x = ob.worker_momentum(st.m, gw, beta1)
            if not no_worker_err:
                x = x + st.err_w[w]
            msg, err_w[w] = ob.error_compensated_compress(x, comp)
            msgs.append(msg)
        z = ob.server_average(msgs, comp)
        if not no_server_err:
            z = z + st.err_s
        smsg, err_s = ob.error_compensated_compress(z, comp)
        m = st.m.copy() if keep_old_m else comp.decompress(smsg).astype(np.float32)
        p = ob.preconditioned_update(st.p, m, st.v, lr, eps)
        return ob.StepOutput(ob.TensorState(p, m, st.v, err_s, err_w), msgs, smsg)
    return compression_step


def _server(skip_first=False, divisor=lambda W: W):
    def server_average(msgs, comp=ob.OneBitCompressor):
        acc = np.zeros_like(comp.decompress(msgs[0]), dtype=np.float32)
        for msg in (msgs[1:] if skip_first and len(msgs) > 1 else msgs):
            acc = acc + comp.decompress(msg)
        return acc / F32(divisor(len(msgs)))
    return server_average


def _ecc(kind):
    def error_compensated_compress(x, comp=ob.OneBitCompressor):
        msg = comp.compress(x)
        if kind == "plus":
            return msg, x + comp.decompress(msg)
        return msg, np.zeros_like(x)
    return error_compensated_compress


_orig_sos = ob.sum_of_squares

MUTANTS = {
    "momentum_fp32_complement": ("worker_momentum",
        lambda m, g, b: F32(b) * m + (F32(1.0) - F32(b)) * ob.widen_grad(g)),
    "momentum_transposed": ("worker_momentum",
        lambda m, g, b: F32(b) * ob.widen_grad(g) + F32(1.0 - b) * m),
    "momentum_drops_m": ("worker_momentum", lambda m, g, b: F32(1.0 - b) * ob.widen_grad(g)),
    "sign_of_zero_negative": ("sign_bits", lambda x: x > F32(0.0)),
    "pack_msb_first": ("pack_signs", lambda bits: np.array(
        [int("".join("1" if b else "0" for b in
                     np.concatenate([bits.ravel(), np.zeros((-bits.size) % 64, bool)])[64 * j: 64 * j + 64]), 2)
         for j in range((bits.size + 63) // 64)], dtype=np.uint64)),
    "unpack_off_by_one": ("unpack_signs", lambda words, n: (
        (np.asarray(words, np.uint64)[:, None] >> (np.arange(64, dtype=np.uint64) + np.uint64(1)) % np.uint64(64))
        & np.uint64(1)).ravel()[:n].astype(bool)),
    "scale_mean_abs": ("onebit_scale", lambda x: F32(np.mean(np.abs(x.astype(np.float64))))),
    "scale_divides_after_sqrt": ("onebit_scale", lambda x: F32(np.sqrt(_orig_sos(x)) / x.size)),
    "scale_fp32_sum": ("onebit_scale", lambda x: F32(np.sqrt(np.sum(x * x, dtype=np.float32) / F32(x.size)))),
    "sum_of_squares_drops_last": ("sum_of_squares", lambda x: _orig_sos(np.asarray(x).ravel()[:-1])),
    "sum_of_squares_fp64_plain": ("sum_of_squares",
        lambda x: float(np.add.reduce(np.asarray(x, np.float64).ravel()[::-1] ** 2))),
    "error_sign_flipped": ("error_compensated_compress", _ecc("plus")),
    "no_error_feedback": ("error_compensated_compress", _ecc("zero")),
    "server_no_divide": ("server_average", _server(divisor=lambda W: 1)),
    "server_divides_by_w_minus_1": ("server_average", _server(divisor=lambda W: max(W - 1, 1))),
    "server_skips_worker0": ("server_average", _server(skip_first=True)),
    "step_drops_worker_error": ("compression_step", _step_factory(no_worker_err=True)),
    "step_drops_server_error": ("compression_step", _step_factory(no_server_err=True)),
    "step_keeps_old_momentum": ("compression_step", _step_factory(keep_old_m=True)),
    "step_pairs_wrong_worker": ("compression_step", _step_factory(reverse_workers=True)),
    "update_eps_inside_sqrt": ("preconditioned_update",
        lambda p, m, v, lr, eps: p - F32(lr) * (m / np.sqrt(v + F32(eps)))),
    "update_wrong_sign": ("preconditioned_update",
        lambda p, m, v, lr, eps: p + F32(lr) * (m / (np.sqrt(v) + F32(eps)))),
    "update_multiplies": ("preconditioned_update",
        lambda p, m, v, lr, eps: p - F32(lr) * (m * (np.sqrt(v) + F32(eps)))),
    "bf16_widen_wrong_shift": ("widen_grad", lambda g: g if g.dtype == np.float32 else
        (g.astype(np.uint32) << np.uint32(15)).view(np.float32)),
}


def _warmup_v_linear(st, grads, beta1, beta2, lr, eps):
    W = grads.shape[0]
    acc = np.zeros(grads.shape[1], np.float32)
    for w in range(W):
        acc = acc + ob.widen_grad(grads[w])
    gbar = acc / F32(W)
    m = F32(beta1) * st.m + F32(1.0 - beta1) * gbar
    v = F32(beta2) * st.v + F32(1.0 - beta2) * np.abs(gbar)
    p = ob.preconditioned_update(st.p, m, v, lr, eps)
    return ob.TensorState(p, m, v, st.err_s.copy(), st.err_w.copy())


MUTANTS["warmup_v_not_squared"] = ("warmup_step", _warmup_v_linear)


def _chunks_off_by_one_block(n, chunks):
    blocks = -(-n // ob.CHUNK_BLOCK)
    size = ob.CHUNK_BLOCK * max(1, -(-blocks // chunks) - (1 if blocks > chunks else 0))
    return [(lo, min(lo + size, n)) for lo in range(0, n, size)]


MUTANTS["chunk_size_one_block_short"] = ("chunk_bounds", _chunks_off_by_one_block)
MUTANTS["chunk_bounds_not_block_aligned"] = ("chunk_bounds",
    lambda n, c: [(lo, min(lo + -(-n // c), n)) for lo in range(0, n, -(-n // c))])


MUTANTS["trust_ratio_inverted"] = ("trust_ratio", lambda p, u: F32(1.0) if (
    ob.sum_of_squares(p) == 0 or ob.sum_of_squares(u) == 0) else F32(
    np.sqrt(ob.sum_of_squares(u)) / np.sqrt(ob.sum_of_squares(p))))
MUTANTS["trust_ratio_squared_norms"] = ("trust_ratio", lambda p, u: F32(1.0) if (
    ob.sum_of_squares(p) == 0 or ob.sum_of_squares(u) == 0) else F32(
    ob.sum_of_squares(p) / ob.sum_of_squares(u)))


def _cltk_mutant(kind):
    orig = ob.cltk_step

    def cltk_step(memory, grads, step, k):
        if kind == "leader":
            return orig(memory, grads, step + 1, k)
        out = orig(memory, grads, step, k)
        if kind == "memory_keeps_sent":
            out.memory = np.stack([memory[w] + ob.widen_grad(grads[w]) for w in range(memory.shape[0])])
        if kind == "ties_high_index":
            W, n = memory.shape
            x = np.stack([memory[w] + ob.widen_grad(grads[w]) for w in range(W)])
            lead = np.abs(x[step % W]).astype(np.float64)
            order = np.lexsort((-np.arange(n), -lead))
            out.index = np.sort(order[:k])
        return out
    return cltk_step


MUTANTS["cltk_wrong_leader"] = ("cltk_step", _cltk_mutant("leader"))
MUTANTS["cltk_memory_keeps_sent"] = ("cltk_step", _cltk_mutant("memory_keeps_sent"))
MUTANTS["cltk_ties_to_high_index"] = ("cltk_step", _cltk_mutant("ties_high_index"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ob, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except Exception as exc:  # an assertion or a crash both expose the mutant
            caught.append((pin.__name__, type(exc).__name__))
            break
    assert caught, f"planted mistake {name!r} passed every pin"
