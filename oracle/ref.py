"""ctypes front of the C++ oracle (oracle/onebit_ref.cpp): one compression-phase
step, one warmup step and one cyclic-local-top-k exchange of one tensor, plain
and single-threaded.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the build
entry module and the CPU-baseline leg of the benchmark may import this module.
It shares nothing with the product path: the library is built from
oracle/onebit_ref.cpp alone with the host compiler (g++), without floating-point
contraction, and loads no part of the HIP library.

The C++ oracle implements the same readings as oracle/onebit.py (R1-R9 in its
header) in independent code: the exact sum of squares in a fixed-point integer
accumulator instead of Python integers, the step as explicit loops.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "onebit_ref.cpp")
LIB = os.path.join(HERE, "libonebit_ref.so")
# -ffp-contract=off: every fp32 product and sum rounds once; no -ffast-math
FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]

_lib: Optional[ctypes.CDLL] = None
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_u64p = np.ctypeslib.ndpointer(dtype=np.uint64, flags="C_CONTIGUOUS")


def build(verbose: bool = False) -> str:
    """Compile libonebit_ref.so next to its source; returns its path."""
    cxx = os.environ.get("CXX") or shutil.which("g++") or "g++"
    tmp = LIB + ".tmp"
    cmd = [cxx, *FLAGS, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"building the C++ oracle failed ({proc.returncode}):\n{proc.stderr}")
    os.replace(tmp, LIB)
    return LIB


def load() -> ctypes.CDLL:
    """The C++ oracle library, built first if it is missing or older than its source."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    lib.ref_sum_of_squares.restype = ctypes.c_double
    lib.ref_sum_of_squares.argtypes = [_f32p, ctypes.c_int64]
    lib.ref_scale.restype = ctypes.c_float
    lib.ref_scale.argtypes = [_f32p, ctypes.c_int64]
    lib.ref_pack_signs.restype = None
    lib.ref_pack_signs.argtypes = [_f32p, ctypes.c_int64, _u64p]
    lib.ref_compression_step.restype = ctypes.c_int
    lib.ref_compression_step.argtypes = [ctypes.c_int64, ctypes.c_int32, _f32p, ctypes.c_double,
                                         ctypes.c_double, ctypes.c_double, _f32p, _f32p, _f32p, _f32p,
                                         _f32p, _u64p, _f32p, _u64p, _f32p]
    lib.ref_compression_step_opts.restype = ctypes.c_int
    lib.ref_compression_step_opts.argtypes = [ctypes.c_int64, ctypes.c_int32, _f32p, ctypes.c_double,
                                              ctypes.c_double, ctypes.c_double, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_double, _f32p, _f32p, _f32p, _f32p, _f32p, _u64p, _f32p,
                                              _u64p, _f32p]
    vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.ref_compression_step_strided.restype = ctypes.c_int
    lib.ref_compression_step_strided.argtypes = [i64, i32, vp, i32, i64, dbl, dbl, dbl, i32, i32, dbl,
                                                 vp, vp, vp, vp, vp, i64, vp, i64, vp, i64, vp, vp]
    lib.ref_warmup_step.restype = ctypes.c_int
    lib.ref_warmup_step.argtypes = [ctypes.c_int64, ctypes.c_int32, _f32p, ctypes.c_double, ctypes.c_double,
                                    ctypes.c_double, ctypes.c_double, _f32p, _f32p, _f32p]
    lib.ref_cltk_step.restype = ctypes.c_int
    lib.ref_cltk_step.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, _f32p, _f32p,
                                  np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS"), _f32p, _f32p]
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def sum_of_squares(x) -> float:
    x = _f32(x).ravel()
    return float(load().ref_sum_of_squares(x, x.size))


def scale(x) -> np.float32:
    x = _f32(x).ravel()
    return np.float32(load().ref_scale(x, x.size))


def pack_signs(x) -> np.ndarray:
    x = _f32(x).ravel()
    words = np.zeros((x.size + 63) // 64, dtype=np.uint64)
    load().ref_pack_signs(x, x.size, words)
    return words


def widen(g: np.ndarray) -> np.ndarray:
    """fp32 gradients as they are; bf16 (uint16 bit patterns) widened exactly."""
    if g.dtype == np.uint16:
        return (g.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return _f32(g)


def compression_step(p, m, v, err_s, err_w, grads, beta1: float, lr: float, eps: float,
                     server_chunks: int = 1, trust_wd=None) -> dict:
    """One step of one tensor on copies of the state.  grads [W][n] (fp32 or
    bf16 bit patterns).  Returns the new p, m, err_s, err_w and the messages:
    packed_w [W][ceil(n/64)], scale_w [W], packed_s [ceil(n/64)], scales_s (fp32,
    one per server chunk) and scale_s (the first).  server_chunks = C > 1
    partitions the server (R11); trust_wd, when not None, scales the update by
    the trust ratio with that weight decay (R14)."""
    g = np.ascontiguousarray(widen(np.asarray(grads)))
    W, n = g.shape
    nw = (n + 63) // 64
    blocks = -(-n // 8192)
    pieces = -(-n // (8192 * -(-blocks // int(server_chunks))))
    out = {"p": _f32(p).copy(), "m": _f32(m).copy(), "err_s": _f32(err_s).copy(),
           "err_w": _f32(err_w).reshape(W, n).copy(),
           "packed_w": np.zeros((W, nw), dtype=np.uint64), "scale_w": np.zeros(W, dtype=np.float32),
           "packed_s": np.zeros(nw, dtype=np.uint64), "scales_s": np.zeros(pieces, dtype=np.float32)}
    st = load().ref_compression_step_opts(n, W, g, float(beta1), float(lr), float(eps), int(server_chunks),
                                          0 if trust_wd is None else 1,
                                          0.0 if trust_wd is None else float(trust_wd), out["p"], out["m"],
                                          _f32(v), out["err_s"], out["err_w"], out["packed_w"],
                                          out["scale_w"], out["packed_s"], out["scales_s"])
    if st != 0:
        raise ValueError("ref_compression_step_opts rejected its arguments")
    out["scale_s"] = out["scales_s"][0]
    return out


def _addr(a: np.ndarray, dtype, index: int, count: int) -> int:
    """Address of element `index` of the flat C-contiguous array `a`, after
    checking that elements [index, index + count) lie inside it."""
    if a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"expected a C-contiguous {np.dtype(dtype)} array, got {a.dtype}")
    if index < 0 or count < 0 or index + count > a.size:
        raise IndexError(f"elements [{index}, {index + count}) outside an array of {a.size}")
    return a.ctypes.data + index * a.itemsize


def compression_step_in_place(lo: int, n: int, col: int, grads, p, m, v, err_s, err_w, packed_w, scale_w,
                              packed_s, scale_s, beta1: float, lr: float, eps: float,
                              server_chunks: int = 1, trust_wd=None) -> None:
    """One step of the tensor at elements [lo, lo + n) of padded flat host
    buffers, in place (lo a multiple of 64):
      grads [W][N] fp32, or uint16 bf16 bit patterns;  p, m, v, err_s [N] fp32;
      err_w [W][N] fp32;  packed_w [W][N/64] uint64;  scale_w [W][T] fp32 (column
      col written);  packed_s [N/64] uint64;  scale_s this tensor's server
      scales (a contiguous fp32 array of one entry per server chunk, written).
    The same arithmetic as compression_step, without copying the tensor out."""
    g = np.asarray(grads)
    for a in (g, p, m, v, err_s, err_w, packed_w, scale_w, packed_s, scale_s):
        if not a.flags["C_CONTIGUOUS"]:   # a flattening copy would take the writes
            raise TypeError("every buffer must be C-contiguous")
    W, N = g.shape
    T = scale_w.shape[1]
    if lo % 64 or n < 1 or lo + n > N or not 0 <= col < T:
        raise ValueError("tensor range outside the flat layout")
    if err_w.shape != (W, N) or packed_w.shape != (W, N // 64) or scale_w.shape[0] != W:
        raise ValueError("per-worker buffers do not match the gradients' [W][N]")
    blocks = -(-n // 8192)
    pieces = -(-n // (8192 * -(-blocks // int(server_chunks))))
    if scale_s.size != pieces:
        raise ValueError(f"scale_s holds {scale_s.size} entries, the server has {pieces} chunks")
    bf16 = g.dtype == np.uint16
    gdt = np.uint16 if bf16 else np.float32
    nw = (n + 63) // 64
    last = (W - 1) * N + lo   # first element of the last row's range
    st = load().ref_compression_step_strided(
        n, W, _addr(g.reshape(-1), gdt, lo, last - lo + n), 1 if bf16 else 0, N,
        float(beta1), float(lr), float(eps), int(server_chunks), 0 if trust_wd is None else 1,
        0.0 if trust_wd is None else float(trust_wd),
        _addr(p, np.float32, lo, n), _addr(m, np.float32, lo, n), _addr(v, np.float32, lo, n),
        _addr(err_s, np.float32, lo, n), _addr(err_w.reshape(-1), np.float32, lo, last - lo + n), N,
        _addr(packed_w.reshape(-1), np.uint64, lo // 64, (W - 1) * (N // 64) + nw), N // 64,
        _addr(scale_w.reshape(-1), np.float32, col, (W - 1) * T + 1), T,
        _addr(packed_s, np.uint64, lo // 64, nw), _addr(scale_s, np.float32, 0, pieces))
    if st != 0:
        raise ValueError("ref_compression_step_strided rejected its arguments")


def warmup_step(p, m, v, grads, beta1: float, beta2: float, lr: float, eps: float) -> dict:
    """One warmup (uncompressed Adam) step of one tensor on copies of p, m, v;
    grads [W][n] fp32 or bf16 bit patterns.  Returns the new p, m, v."""
    g = np.ascontiguousarray(widen(np.asarray(grads)))
    W, n = g.shape
    out = {"p": _f32(p).copy(), "m": _f32(m).copy(), "v": _f32(v).copy()}
    st = load().ref_warmup_step(n, W, g, float(beta1), float(beta2), float(lr), float(eps),
                                out["p"], out["m"], out["v"])
    if st != 0:
        raise ValueError("ref_warmup_step rejected its arguments")
    return out


def cltk_step(memory, grads, step: int, k: int) -> dict:
    """One cyclic-local-top-k exchange of one tensor on a copy of the memories
    [W][n]; grads [W][n] fp32 or bf16 bit patterns.  Returns index (int64 [k],
    ascending), values [W][k], average [k] and the new memory [W][n]."""
    g = np.ascontiguousarray(widen(np.asarray(grads)))
    W, n = g.shape
    out = {"memory": _f32(memory).reshape(W, n).copy(), "index": np.zeros(k, dtype=np.int64),
           "values": np.zeros((W, k), dtype=np.float32), "average": np.zeros(k, dtype=np.float32)}
    st = load().ref_cltk_step(n, W, int(step), int(k), g, out["memory"], out["index"], out["values"],
                              out["average"])
    if st != 0:
        raise ValueError("ref_cltk_step rejected its arguments")
    return out
