"""Thin ctypes binding of libob.so (the C ABI in include/ob.h).

Argument marshalling only: every step of the method runs in the HIP kernels.
PyTorch supplies device memory and the current stream.  Loading fails loudly
when the built library is missing; there is no other implementation to fall
back to.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libob.so")

OB_OK, OB_ERR_INVALID, OB_ERR_ALIGN, OB_ERR_NOMEM, OB_ERR_DEVICE, OB_ERR_SCRATCH = 0, 1, 2, 3, 4, 5
OB_GRAD_F32, OB_GRAD_BF16 = 0, 1

_c_void_p = ctypes.c_void_p
_i32, _i64, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double

# name -> (restype, argtypes); mirrors include/ob.h
SIGNATURES = {
    "ob_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ob_layout": (ctypes.c_int, [_i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "ob_init": (ctypes.c_int, [ctypes.POINTER(_c_void_p), _i32, ctypes.POINTER(_i64), _i32, _i32,
                               _f64, _f64]),
    "ob_destroy": (None, [_c_void_p]),
    "ob_compress_worker": (ctypes.c_int, [_c_void_p, _i32, _i32] + [_c_void_p] * 6),
    "ob_server_reduce": (ctypes.c_int, [_c_void_p] * 7),
    "ob_apply_update": (ctypes.c_int, [_c_void_p] * 6 + [_f64, _c_void_p]),
    "ob_step": (ctypes.c_int, [_c_void_p] * 11 + [_f64, _c_void_p]),
    "ob_step_residual": (ctypes.c_int, [_c_void_p, _i32] + [_c_void_p] * 10 + [_f64, _c_void_p]),
    "ob_step_residual_noalloc": (ctypes.c_int, [_c_void_p, _i32] + [_c_void_p] * 10 + [_f64, _c_void_p]),
    "ob_materialize": (ctypes.c_int, [_c_void_p] * 9),
    "ob_warmup_step": (ctypes.c_int, [_c_void_p] * 5 + [_f64, _f64, _c_void_p]),
    "ob_begin_compression": (ctypes.c_int, [_c_void_p] * 4),
    "ob_set_server_chunks": (ctypes.c_int, [_c_void_p, _i32]),
    "ob_server_scale_count": (_i32, [_c_void_p]),
    "ob_set_trust_ratio": (ctypes.c_int, [_c_void_p, _i32, _f64]),
    "ob_cltk_configure": (ctypes.c_int, [_c_void_p, _f64, ctypes.POINTER(_i64)]),
    "ob_cltk_layout": (ctypes.c_int, [_c_void_p, ctypes.POINTER(_i64)]),
    "ob_cltk_step": (ctypes.c_int, [_c_void_p, _i64] + [_c_void_p] * 5 + [_c_void_p]),
    "ob_profile_enable": (ctypes.c_int, [_c_void_p, _i32]),
    "ob_profile_kinds": (_i32, []),
    "ob_profile_kind_name": (ctypes.c_char_p, [_i32]),
    "ob_profile_read": (ctypes.c_int, [_c_void_p, ctypes.POINTER(_f64), ctypes.POINTER(_i64), _i32]),
}

_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libob.so once (torch is imported first, so its HIP runtime is the one shared)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m error_compensated_bit_02_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class OneBitError(RuntimeError):
    """A call of the C ABI returned a status other than OB_OK (in .status)."""

    def __init__(self, message: str, status=None):
        super().__init__(message)
        self.status = status


def _check(status: int, what: str) -> None:
    if status != OB_OK:
        msg = load_library().ob_status_string(status).decode()
        raise OneBitError(f"{what}: {msg} (status {status})", status)


def layout(numel: Sequence[int]) -> List[int]:
    """Padded element offsets off[0..T] (host only)."""
    lib = load_library()
    T = len(numel)
    arr = (_i64 * T)(*numel)
    out = (_i64 * (T + 1))()
    _check(lib.ob_layout(T, arr, out), "ob_layout")
    return list(out)


def _ptr(t: torch.Tensor, dtype, numel: int, name: str) -> int:
    if not t.is_cuda:
        raise OneBitError(f"{name} must be a device tensor")
    if t.dtype not in dtype:
        raise OneBitError(f"{name} has dtype {t.dtype}, expected one of {dtype}")
    if not t.is_contiguous():
        raise OneBitError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise OneBitError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class OneBitAdam:
    """Context for one tensor list: owns an ob_ctx (device scratch) and checks
    buffer shapes before calling into the library.

    Buffers (all contiguous device tensors in the padded layout):
      grads [W][N] float32 or bfloat16; m, v, params, err_s [N] float32;
      err_w [W][N] float32; packed_w [W][Nw] int64 (sign words);
      scale_w [W][T] float32; packed_s [Nw] int64; scale_s [S] float32
      (S = T, or one per tensor chunk after set_server_chunks).
      CLT-k codec (after cltk_configure): memory [W][N] float32; index [K]
      int32; values [W][K] float32; average [K] float32.
    """

    def __init__(self, numel: Sequence[int], workers: int, grad_dtype: str = "f32",
                 beta1: float = 0.9, eps: float = 1e-8):
        self.lib = load_library()
        self.numel = [int(n) for n in numel]
        self.T = len(self.numel)
        self.W = int(workers)
        self.grad_dtype = grad_dtype
        self.beta1, self.eps = float(beta1), float(eps)
        self.offsets = layout(self.numel)
        self.N = self.offsets[-1]
        self.Nw = self.N // 64
        code = {"f32": OB_GRAD_F32, "bf16": OB_GRAD_BF16}[grad_dtype]
        ctx = _c_void_p()
        arr = (_i64 * self.T)(*self.numel)
        _check(self.lib.ob_init(ctypes.byref(ctx), self.T, arr, self.W, code, self.beta1, self.eps),
               "ob_init")
        self._ctx = ctx
        self.S = self.lib.ob_server_scale_count(self._ctx)

    def set_trust_ratio(self, enable: bool, weight_decay: float = 0.0) -> None:
        """Scale each tensor's update by its trust ratio ||p|| / ||u||; see include/ob.h."""
        _check(self.lib.ob_set_trust_ratio(self._ctx, 1 if enable else 0, float(weight_decay)),
               "ob_set_trust_ratio")

    def cltk_configure(self, density: float) -> List[int]:
        """Set up the cyclic local top-k codec; returns k_off[0..T] (K = k_off[T])."""
        K = _i64()
        _check(self.lib.ob_cltk_configure(self._ctx, float(density), ctypes.byref(K)), "ob_cltk_configure")
        out = (_i64 * (self.T + 1))()
        _check(self.lib.ob_cltk_layout(self._ctx, out), "ob_cltk_layout")
        self.K = K.value
        return list(out)

    def cltk_step(self, step, grads, memory, index, values, average, stream=None) -> None:
        """One cyclic-local-top-k exchange (see include/ob.h)."""
        f32 = (torch.float32,)
        st = self.lib.ob_cltk_step(
            self._ctx, int(step), self._grad_ptr(grads), _ptr(memory, f32, self.W * self.N, "memory"),
            _ptr(index, (torch.int32,), self.K, "index"), _ptr(values, f32, self.W * self.K, "values"),
            _ptr(average, f32, self.K, "average"), _stream(stream))
        _check(st, "ob_cltk_step")

    def set_server_chunks(self, chunks: int) -> None:
        """Partition the server C ways (one scale per tensor chunk); see include/ob.h."""
        _check(self.lib.ob_set_server_chunks(self._ctx, int(chunks)), "ob_set_server_chunks")
        self.S = self.lib.ob_server_scale_count(self._ctx)

    def close(self) -> None:
        if getattr(self, "_ctx", None):
            self.lib.ob_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- buffer allocation helpers (plumbing: torch owns the memory) ---------
    def alloc(self, device="cuda") -> Dict[str, torch.Tensor]:
        """Zero-filled message buffers for this tensor list."""
        d = torch.device(device)
        return {
            "packed_w": torch.zeros(self.W, self.Nw, dtype=torch.int64, device=d),
            "scale_w": torch.zeros(self.W, self.T, dtype=torch.float32, device=d),
            "packed_s": torch.zeros(self.Nw, dtype=torch.int64, device=d),
            "scale_s": torch.zeros(self.S, dtype=torch.float32, device=d),
        }

    def _grad_ptr(self, grads: torch.Tensor) -> int:
        want = (torch.bfloat16,) if self.grad_dtype == "bf16" else (torch.float32,)
        return _ptr(grads, want, self.W * self.N, "grads")

    # -- the C ABI calls -----------------------------------------------------
    def compress_worker(self, grads, m, err_w, packed_w, scale_w, w_begin=0, w_end=None,
                        stream=None) -> None:
        w_end = self.W if w_end is None else w_end
        f32 = (torch.float32,)
        st = self.lib.ob_compress_worker(
            self._ctx, w_begin, w_end, self._grad_ptr(grads), _ptr(m, f32, self.N, "m"),
            _ptr(err_w, f32, self.W * self.N, "err_w"),
            _ptr(packed_w, (torch.int64,), self.W * self.Nw, "packed_w"),
            _ptr(scale_w, f32, self.W * self.T, "scale_w"), _stream(stream))
        _check(st, "ob_compress_worker")

    def server_reduce(self, packed_w, scale_w, err_s, packed_s, scale_s, stream=None) -> None:
        f32 = (torch.float32,)
        st = self.lib.ob_server_reduce(
            self._ctx, _ptr(packed_w, (torch.int64,), self.W * self.Nw, "packed_w"),
            _ptr(scale_w, f32, self.W * self.T, "scale_w"), _ptr(err_s, f32, self.N, "err_s"),
            _ptr(packed_s, (torch.int64,), self.Nw, "packed_s"),
            _ptr(scale_s, f32, self.S, "scale_s"), _stream(stream))
        _check(st, "ob_server_reduce")

    def apply_update(self, packed_s, scale_s, v, m, params, lr, stream=None) -> None:
        f32 = (torch.float32,)
        st = self.lib.ob_apply_update(
            self._ctx, _ptr(packed_s, (torch.int64,), self.Nw, "packed_s"),
            _ptr(scale_s, f32, self.S, "scale_s"), _ptr(v, f32, self.N, "v"),
            _ptr(m, f32, self.N, "m"), _ptr(params, f32, self.N, "params"), float(lr),
            _stream(stream))
        _check(st, "ob_apply_update")

    def step(self, grads, m, v, params, err_w, err_s, packed_w, scale_w, packed_s, scale_s, lr,
             stream=None) -> None:
        f32 = (torch.float32,)
        st = self.lib.ob_step(
            self._ctx, self._grad_ptr(grads), _ptr(m, f32, self.N, "m"), _ptr(v, f32, self.N, "v"),
            _ptr(params, f32, self.N, "params"), _ptr(err_w, f32, self.W * self.N, "err_w"),
            _ptr(err_s, f32, self.N, "err_s"),
            _ptr(packed_w, (torch.int64,), self.W * self.Nw, "packed_w"),
            _ptr(scale_w, f32, self.W * self.T, "scale_w"),
            _ptr(packed_s, (torch.int64,), self.Nw, "packed_s"),
            _ptr(scale_s, f32, self.S, "scale_s"), float(lr), _stream(stream))
        _check(st, "ob_step")

    def step_residual(self, first, grads, m, v, params, err_w, err_s, packed_w, scale_w, packed_s,
                      scale_s, lr, stream=None, noalloc=False) -> None:
        """One step with err_w / err_s in residual form (see include/ob.h);
        noalloc=True calls ob_step_residual_noalloc (static scratch, no allocation)."""
        f32 = (torch.float32,)
        m_ptr = _ptr(m, f32, self.N, "m") if first else (None if m is None else _ptr(m, f32, self.N, "m"))
        name = "ob_step_residual_noalloc" if noalloc else "ob_step_residual"
        st = getattr(self.lib, name)(
            self._ctx, 1 if first else 0, self._grad_ptr(grads), m_ptr, _ptr(v, f32, self.N, "v"),
            _ptr(params, f32, self.N, "params"), _ptr(err_w, f32, self.W * self.N, "err_w"),
            _ptr(err_s, f32, self.N, "err_s"),
            _ptr(packed_w, (torch.int64,), self.W * self.Nw, "packed_w"),
            _ptr(scale_w, f32, self.W * self.T, "scale_w"),
            _ptr(packed_s, (torch.int64,), self.Nw, "packed_s"),
            _ptr(scale_s, f32, self.S, "scale_s"), float(lr), _stream(stream))
        _check(st, name)

    def materialize(self, x_w, scale_w, z, scale_s, err_w, err_s, m, stream=None) -> None:
        """Strict-form errors and momentum from a residual-form state (may be in place)."""
        f32 = (torch.float32,)
        st = self.lib.ob_materialize(
            self._ctx, _ptr(x_w, f32, self.W * self.N, "x_w"), _ptr(scale_w, f32, self.W * self.T, "scale_w"),
            _ptr(z, f32, self.N, "z"), _ptr(scale_s, f32, self.S, "scale_s"),
            _ptr(err_w, f32, self.W * self.N, "err_w"), _ptr(err_s, f32, self.N, "err_s"),
            _ptr(m, f32, self.N, "m"), _stream(stream))
        _check(st, "ob_materialize")

    def warmup_step(self, grads, m, v, params, beta2, lr, stream=None) -> None:
        """One uncompressed Adam step on the workers' average gradient."""
        f32 = (torch.float32,)
        st = self.lib.ob_warmup_step(
            self._ctx, self._grad_ptr(grads), _ptr(m, f32, self.N, "m"), _ptr(v, f32, self.N, "v"),
            _ptr(params, f32, self.N, "params"), float(beta2), float(lr), _stream(stream))
        _check(st, "ob_warmup_step")

    def begin_compression(self, err_w, err_s, stream=None) -> None:
        """Zero the error buffers at the switch from warmup to compression."""
        f32 = (torch.float32,)
        st = self.lib.ob_begin_compression(
            self._ctx, _ptr(err_w, f32, self.W * self.N, "err_w"), _ptr(err_s, f32, self.N, "err_s"),
            _stream(stream))
        _check(st, "ob_begin_compression")

    # -- kernel timing -------------------------------------------------------
    def profile(self, enable: bool) -> None:
        _check(self.lib.ob_profile_enable(self._ctx, 1 if enable else 0), "ob_profile_enable")

    def profile_read(self, reset: bool = True) -> Dict[str, tuple]:
        """{kernel kind: (total ms, launches)}; waits for the recorded events."""
        k = self.lib.ob_profile_kinds()
        ms = (_f64 * k)()
        n = (_i64 * k)()
        _check(self.lib.ob_profile_read(self._ctx, ms, n, 1 if reset else 0), "ob_profile_read")
        return {self.lib.ob_profile_kind_name(i).decode(): (ms[i], n[i]) for i in range(k)}
