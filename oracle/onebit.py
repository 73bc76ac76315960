"""Oracle for the compression phase of 1-bit Adam: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the build
entry module and the CPU-baseline leg of the benchmark may import this module.
The product path (the HIP library and its Python binding) never imports,
links or runs it, and this module imports nothing from the product path.

What is computed, and where it comes from
-----------------------------------------
Source pages: the nubint.ai review of "1-bit Adam: Communication Efficient
Large-Scale Training with Adam's Convergence Speed" (Tang, Gan et al.), cited
below as [1BA] with the section named.

* Two phases: a full-precision Adam warmup, then momentum SGD whose momentum is
  compressed to 1 bit ([1BA] One-line summary; Proposed method, bullet 1).
* Adam's variance settles during warmup and is then held fixed as the
  preconditioner of the compression phase ([1BA] Abstract; Proposed method,
  bullet 2).
* Error-compensated compression is applied to the momentum rather than to the
  gradient ([1BA] Abstract; Proposed method, bullet 3).
* Workers exchange compressed messages through a collective ([1BA] Proposed
  method, bullet 4); on one device the exchange is a local average of the W
  decompressed messages, followed by a server-side error-compensated
  re-compression of that average.

The pages give no formulas.  The readings taken where they are silent:
  R1  scale of a 1-bit message: s = ||x||_2 / sqrt(n) for the n elements of one
      tensor (it keeps the L2 norm: ||s * sign(x)||_2 = ||x||_2).  Computed as
      fp32( sqrt64( fl64(exact sum of x_i^2) / n ) ): the sum of squares is
      exact and rounded once to fp64, then fp64 division and square root, then
      one rounding to fp32.
  R2  sign(x) = +1 for x >= 0, including -0.0; NaN gives bit 0.
  R3  message layout: uint64 words, word j bit k holds element 64*j + k (least
      significant bit first); bits past the tensor's end are 0.
  R4  one scale per (worker, tensor) and one per tensor for the server message.
  R5  worker momentum m_w = c1*m + c2*g_w with c1 = fp32(beta1) and
      c2 = fp32(1 - beta1), the complement taken in double precision from the
      hyper-parameter and rounded once; each product and the sum rounded once
      in fp32, no fused multiply-add.
  R6  server average: fp32 sum over workers in ascending order starting from
      +0.0, then one fp32 division by W.
  R7  after the step every worker's momentum is the server's reconstruction
      (one shared momentum, as momentum SGD has one momentum).
  R8  update p <- p - lr * (m / (sqrt(v) + eps)), fp32, correctly rounded sqrt
      and division, no bias correction, no weight decay.
  R9  any non-finite element in a tensor makes that tensor's scale NaN.
  R10 warmup (uncompressed Adam): gbar = fp32 average of the W gradients as in
      R6; m <- c1*m + c2*gbar; v <- fp32(b2)*v + fp32(1 - b2)*(gbar*gbar);
      p <- p - lr*(m/(sqrt(v)+eps)); no bias correction.
  R11 partitioned server (optional, C chunks): when the server role is split
      C ways, rank j holds chunk j of every tensor and gives it its own scale.
      Chunk j of an n-element tensor covers [j*S, min((j+1)*S, n)) with
      S = 8192 * ceil(ceil(n / 8192) / C): whole 8192-element blocks, so no
      chunk boundary splits a sign word; a tensor has ceil(n / S) <= C chunks.
      C = 1 is the per-tensor scale of R4.
  R14 layer-wise trust ratio (optional; the fugumt page on "1-bit LAMB" says it
      keeps LAMB's layer-wise adaptive learning rates under compressed
      communication, with no formula): the compressed momentum m, the frozen
      variance and the update direction u = m/(sqrt(v)+eps) (+ wd*p when a
      weight decay wd > 0 is given) as in R8; per tensor the trust ratio
      r = fp32(sqrt64(fl64(sum p^2)) / sqrt64(fl64(sum u^2))), r = 1 when either
      sum is 0; p <- p - lr*(r*u).
  R15 cyclic local top-k (the review of "ScaleCom", Proposed method: a
      commutative compressor, cyclic local top-k, that aligns the workers'
      sparsity; an alternative codec for the exchange): at step t the leader
      is worker t mod W; per tensor, x_w = mem_w + g_w (fp32); the index set
      is the k positions of largest |x_leader| (ties to the lower index),
      listed in ascending order; every worker sends its x_w at those
      positions; its memory becomes x_w with those positions set to 0 (plain
      error feedback: the page names a low-pass filter on the memory without
      its form, so none is applied); the server averages the W messages as in
      R6.  k = max(1, ceil(density * n)).

All floating point below is numpy float32 (IEEE binary32, round to nearest
even; numpy never contracts a*b+c) except the scale, which is fp64 as R1 says.
Every function here is pinned by tests against exact arithmetic, brute force,
closed forms or a library routine; none is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

F32 = np.float32
_WORD_SHIFTS = np.arange(64, dtype=np.uint64)


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------

def widen_grad(g: np.ndarray) -> np.ndarray:
    """Gradient as fp32: fp32 passes through; bf16, given as uint16 bit
    patterns, widens exactly (its bits are the top half of an fp32)."""
    if g.dtype == np.float32:
        return g
    if g.dtype == np.uint16:
        return (g.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise TypeError(f"unsupported gradient dtype {g.dtype}")


def worker_momentum(m: np.ndarray, g: np.ndarray, beta1: float) -> np.ndarray:
    """Worker momentum from its gradient (R5): m_w = c1*m + c2*g_w."""
    c1 = F32(beta1)
    c2 = F32(1.0 - float(beta1))
    return c1 * m + c2 * widen_grad(g)


def sign_bits(x: np.ndarray) -> np.ndarray:
    """1-bit code of each element (R2): True where x >= 0 (also for -0.0)."""
    return x >= F32(0.0)


def pack_signs(bits: np.ndarray) -> np.ndarray:
    """Pack booleans into uint64 words, element 64*j + k at bit k of word j (R3)."""
    n = bits.size
    nw = (n + 63) // 64
    padded = np.zeros(nw * 64, dtype=np.uint64)
    padded[:n] = bits.ravel()
    return np.bitwise_or.reduce(padded.reshape(nw, 64) << _WORD_SHIFTS, axis=1)


def unpack_signs(words: np.ndarray, n: int) -> np.ndarray:
    """Inverse of pack_signs for the first n elements."""
    words = np.asarray(words, dtype=np.uint64)
    bits = (words[:, None] >> _WORD_SHIFTS) & np.uint64(1)
    return bits.ravel()[:n].astype(bool)


def sum_of_squares(x: np.ndarray) -> float:
    """fl64 of the exact sum of x_i^2 over fp32 values (R1).

    Each fp32 value is +-M * 2^(k-149) with M an integer below 2^24, so its
    square is M^2 * 2^(2k-298) with M^2 below 2^48.  Squares are grouped by k
    and summed as integers (each M^2 split into two 24-bit halves so that
    numpy's float64 bincount only ever holds integers below 2^53, which it
    adds exactly), the groups are combined as one Python integer, and that
    integer divided by 2^298 is rounded once (CPython's int / int is
    correctly rounded).  Non-finite input gives NaN (R9).
    """
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    if x.size == 0:
        return 0.0
    if x.size >= (1 << 29):
        raise ValueError("tensor too large for the exact-integer sum")
    if not np.all(np.isfinite(x)):
        return float("nan")
    u = x.view(np.uint32)
    biased = ((u >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64)
    frac = (u & np.uint32(0x7FFFFF)).astype(np.uint64)
    mant = np.where(biased > 0, frac | np.uint64(1 << 23), frac)
    k = np.maximum(biased - 1, 0)
    sq = mant * mant
    hi = (sq >> np.uint64(24)).astype(np.float64)
    lo = (sq & np.uint64(0xFFFFFF)).astype(np.float64)
    hsum = np.bincount(k, weights=hi, minlength=254)
    lsum = np.bincount(k, weights=lo, minlength=254)
    total = 0
    for kk in np.nonzero((hsum > 0) | (lsum > 0))[0]:
        total += ((int(hsum[kk]) << 24) + int(lsum[kk])) << (2 * int(kk))
    return total / (1 << 298)


def onebit_scale(x: np.ndarray) -> np.float32:
    """Scale of the 1-bit message of one tensor (R1): fp32(sqrt(fl64(sum x^2)/n))."""
    n = x.size
    s64 = np.sqrt(np.float64(sum_of_squares(x)) / np.float64(n))
    return F32(s64)


# ---------------------------------------------------------------------------
# compressors: compress(x) -> message, decompress(message) -> fp32 values
# ---------------------------------------------------------------------------

@dataclass
class OneBitMessage:
    """Packed sign words plus one fp32 scale for one tensor."""
    words: np.ndarray   # uint64 [ceil(n/64)]
    scale: np.float32
    n: int


class OneBitCompressor:
    """sign bits + one scale per tensor ([1BA] One-line summary and Abstract: 1-bit compression)."""

    @staticmethod
    def compress(x: np.ndarray) -> OneBitMessage:
        return OneBitMessage(pack_signs(sign_bits(x)), onebit_scale(x), x.size)

    @staticmethod
    def decompress(msg: OneBitMessage) -> np.ndarray:
        s = msg.scale
        return np.where(unpack_signs(msg.words, msg.n), s, -s).astype(np.float32)


CHUNK_BLOCK = 8192


def chunk_bounds(n: int, chunks: int) -> List[Tuple[int, int]]:
    """Element ranges of the server chunks of an n-element tensor (R11)."""
    blocks = -(-n // CHUNK_BLOCK)
    size = CHUNK_BLOCK * -(-blocks // chunks)
    return [(lo, min(lo + size, n)) for lo in range(0, n, size)]


@dataclass
class ChunkedMessage:
    """Packed sign words of the whole tensor plus one fp32 scale per chunk."""
    words: np.ndarray
    scales: np.ndarray   # fp32 [chunks]
    bounds: List[Tuple[int, int]]
    n: int


class ChunkedOneBitCompressor:
    """The 1-bit compressor applied chunk by chunk (R11): signs of every
    element, one scale per chunk."""

    def __init__(self, chunks: int):
        self.chunks = chunks

    def compress(self, x: np.ndarray) -> ChunkedMessage:
        bounds = chunk_bounds(x.size, self.chunks)
        scales = np.array([onebit_scale(x[lo:hi]) for lo, hi in bounds], dtype=np.float32)
        return ChunkedMessage(pack_signs(sign_bits(x)), scales, bounds, x.size)

    @staticmethod
    def decompress(msg: ChunkedMessage) -> np.ndarray:
        bits = unpack_signs(msg.words, msg.n)
        out = np.empty(msg.n, dtype=np.float32)
        for (lo, hi), s in zip(msg.bounds, msg.scales):
            out[lo:hi] = np.where(bits[lo:hi], s, -s)
        return out


class IdentityCompressor:
    """No compression: the message is the value itself.  With it the step must
    reduce to preconditioned momentum SGD."""

    @staticmethod
    def compress(x: np.ndarray) -> np.ndarray:
        return x.copy()

    @staticmethod
    def decompress(msg: np.ndarray) -> np.ndarray:
        return msg


def error_compensated_compress(x: np.ndarray, comp=OneBitCompressor):
    """Compress x and keep what was lost ([1BA] Abstract; Proposed method,
    bullet 3): message = C(x), new error = x - decompress(C(x))."""
    msg = comp.compress(x)
    return msg, x - comp.decompress(msg)


def server_average(msgs: Sequence, comp=OneBitCompressor) -> np.ndarray:
    """Average of the W decompressed messages (R6): ascending fp32 sum from +0.0, then / W."""
    acc = np.zeros_like(comp.decompress(msgs[0]), dtype=np.float32)
    for msg in msgs:
        acc = acc + comp.decompress(msg)
    return acc / F32(len(msgs))


def preconditioned_update(p: np.ndarray, m: np.ndarray, v: np.ndarray,
                          lr: float, eps: float) -> np.ndarray:
    """Momentum step preconditioned by the frozen variance (R8; [1BA] Abstract,
    Proposed method, bullet 2): p - lr * (m / (sqrt(v) + eps))."""
    return p - F32(lr) * (m / (np.sqrt(v) + F32(eps)))


def trust_ratio(p: np.ndarray, u: np.ndarray) -> np.float32:
    """LAMB's layer-wise trust ratio ||p|| / ||u|| of one tensor (R14)."""
    sp, su = sum_of_squares(p), sum_of_squares(u)
    if sp == 0.0 or su == 0.0:
        return F32(1.0)
    return F32(np.sqrt(np.float64(sp)) / np.sqrt(np.float64(su)))


def trust_ratio_update(p: np.ndarray, m: np.ndarray, v: np.ndarray, lr: float, eps: float,
                       weight_decay: float = 0.0) -> np.ndarray:
    """The preconditioned update scaled per tensor by the trust ratio (R14)."""
    u = m / (np.sqrt(v) + F32(eps))
    if weight_decay > 0.0:
        u = u + F32(weight_decay) * p
    r = trust_ratio(p, u)
    return p - F32(lr) * (r * u)


# ---------------------------------------------------------------------------
# one compression-phase step of one tensor, and of a tensor list
# ---------------------------------------------------------------------------

@dataclass
class TensorState:
    p: np.ndarray        # fp32 [n] parameters
    m: np.ndarray        # fp32 [n] momentum (one, shared by all workers: R7)
    v: np.ndarray        # fp32 [n] variance, frozen in this phase
    err_s: np.ndarray    # fp32 [n] server error
    err_w: np.ndarray    # fp32 [W][n] worker errors

    def copy(self) -> "TensorState":
        return TensorState(self.p.copy(), self.m.copy(), self.v.copy(),
                           self.err_s.copy(), self.err_w.copy())


@dataclass
class StepOutput:
    state: TensorState
    worker_msgs: List      # W messages
    server_msg: object     # one message


def compression_step(st: TensorState, grads: np.ndarray, beta1: float, lr: float,
                     eps: float, comp=OneBitCompressor, server_comp=None,
                     trust_ratio_wd=None) -> StepOutput:
    """One compression-phase step of one tensor.

    grads is [W][n] (fp32, or bf16 as uint16 bit patterns).  Order:
    per worker w (each independent): m_w, x_w = m_w + e_w, message and new e_w;
    server: y = average of the messages, z = y + e_s, message and new e_s;
    m <- decompress(server message); p <- preconditioned update with m.
    server_comp (default: comp) compresses the server's value, for example
    ChunkedOneBitCompressor(C) for a C-way partitioned server (R11).
    trust_ratio_wd, when not None, selects the trust-ratio update of R14 with
    that weight decay.
    """
    scomp = comp if server_comp is None else server_comp
    W = grads.shape[0]
    msgs = []
    err_w = np.empty_like(st.err_w)
    for w in range(W):
        x = worker_momentum(st.m, grads[w], beta1) + st.err_w[w]
        msg, err_w[w] = error_compensated_compress(x, comp)
        msgs.append(msg)
    z = server_average(msgs, comp) + st.err_s
    smsg, err_s = error_compensated_compress(z, scomp)
    m = scomp.decompress(smsg).astype(np.float32)
    if trust_ratio_wd is None:
        p = preconditioned_update(st.p, m, st.v, lr, eps)
    else:
        p = trust_ratio_update(st.p, m, st.v, lr, eps, trust_ratio_wd)
    return StepOutput(TensorState(p, m, st.v, err_s, err_w), msgs, smsg)


def compression_step_all(states: List[TensorState], grads: List[np.ndarray], beta1: float,
                         lr: float, eps: float) -> List[StepOutput]:
    """The step over a tensor list: tensors are independent (one scale each)."""
    return [compression_step(st, g, beta1, lr, eps) for st, g in zip(states, grads)]


# ---------------------------------------------------------------------------
# warmup phase: uncompressed Adam (R10)
# ---------------------------------------------------------------------------

def warmup_step(st: TensorState, grads: np.ndarray, beta1: float, beta2: float,
                lr: float, eps: float) -> TensorState:
    """One full-precision Adam step on the averaged gradient ([1BA] Proposed
    method, bullet 1).  Error buffers are untouched (they stay zero)."""
    W = grads.shape[0]
    acc = np.zeros(grads.shape[1], dtype=np.float32)
    for w in range(W):
        acc = acc + widen_grad(grads[w])
    gbar = acc / F32(W)
    m = F32(beta1) * st.m + F32(1.0 - float(beta1)) * gbar
    v = F32(beta2) * st.v + F32(1.0 - float(beta2)) * (gbar * gbar)
    p = preconditioned_update(st.p, m, v, lr, eps)
    return TensorState(p, m, v, st.err_s.copy(), st.err_w.copy())


@dataclass
class TopKResult:
    index: np.ndarray    # int64 [k] ascending positions within the tensor
    values: np.ndarray   # fp32 [W][k] each worker's message
    average: np.ndarray  # fp32 [k] the server's average
    memory: np.ndarray   # fp32 [W][n] the workers' new memories


def cltk_k(n: int, density: float) -> int:
    """Entries kept per tensor (R15)."""
    return max(1, int(np.ceil(density * n)))


def cltk_step(memory: np.ndarray, grads: np.ndarray, step: int, k: int) -> TopKResult:
    """One cyclic-local-top-k exchange of one tensor (R15)."""
    W, n = memory.shape
    x = np.stack([memory[w] + widen_grad(grads[w]) for w in range(W)])
    lead = np.abs(x[step % W]).astype(np.float64)
    order = np.lexsort((np.arange(n), -lead))          # |x| descending, index ascending
    index = np.sort(order[:k])
    values = x[:, index]
    mem = x.copy()
    mem[:, index] = F32(0.0)
    acc = np.zeros(k, dtype=np.float32)
    for w in range(W):
        acc = acc + values[w]
    return TopKResult(index, values, acc / F32(W), mem)


def message_bytes(n: int) -> int:
    """Bytes of one tensor's 1-bit message: the packed words plus the fp32 scale."""
    return 8 * ((n + 63) // 64) + 4


def split_state(flat: dict, numel: Sequence[int], offsets: Sequence[int],
                tensors: Sequence[int]) -> List[TensorState]:
    """Cut per-tensor states out of host copies of flat buffers (p, m, v, err_s
    of [N], err_w of [W][N]) given each tensor's start offset."""
    out = []
    for t in tensors:
        lo, hi = offsets[t], offsets[t] + numel[t]
        out.append(TensorState(flat["p"][lo:hi].copy(), flat["m"][lo:hi].copy(),
                               flat["v"][lo:hi].copy(), flat["err_s"][lo:hi].copy(),
                               flat["err_w"][:, lo:hi].copy()))
    return out


def words_of(msgs: Sequence[OneBitMessage]) -> Tuple[np.ndarray, np.ndarray]:
    """Stack W messages into ([W][nw] words, [W] scales)."""
    return (np.stack([m.words for m in msgs]), np.array([m.scale for m in msgs], dtype=np.float32))
