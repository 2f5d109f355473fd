"""Overlap-save FIR filtering on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libfirols.so``: the functions below carry the C
names of ``include/firols.h`` and only marshal arguments (pointers, sizes,
streams).  Every step of the filtering runs in the library's HIP kernels.
If the library is not built, loading raises ``FirOlsError``: there is no
fallback of any kind.

Pointers may be given as integers or as torch tensors (their ``data_ptr``);
streams as integers, torch streams, or ``None`` (torch's current stream on
the current device when torch has CUDA/HIP, else the null stream).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from .build import LIB as LIBRARY_PATH

__all__ = [
    "FirOlsError", "Plan", "load_library", "LIBRARY_PATH", "EXPORTED",
    "fir_ols_plan", "fir_ols_set_taps", "fir_ols_set_freq_response",
    "fir_ols_execute", "fir_ols_execute_host", "fir_ols_execute_real", "fir_ols_execute_static",
    "fir_ols_static_scratch_bytes", "fir_ols_set_state",
    "fir_ols_get_state", "fir_ols_check", "fir_ols_destroy", "fir_ols_block_length",
    "fir_ols_choose_n", "fir_ols_status_string", "Channelizer", "fir_pfb_plan", "fir_pfb_set_taps",
    "fir_pfb_execute", "fir_pfb_set_state", "fir_pfb_get_state", "fir_pfb_destroy",
]

# Every symbol include/firols.h and include/firpfb.h declare.
EXPORTED = (
    "fir_ols_plan", "fir_ols_set_taps", "fir_ols_set_freq_response",
    "fir_ols_execute", "fir_ols_execute_host", "fir_ols_execute_real", "fir_ols_execute_static",
    "fir_ols_static_scratch_bytes", "fir_ols_set_state",
    "fir_ols_get_state", "fir_ols_check", "fir_ols_destroy", "fir_ols_block_length",
    "fir_ols_choose_n", "fir_ols_status_string", "fir_pfb_plan", "fir_pfb_set_taps", "fir_pfb_execute",
    "fir_pfb_set_state", "fir_pfb_get_state", "fir_pfb_destroy",
)

STATUS = {
    0: "FIR_OLS_OK", -1: "FIR_OLS_ERR_INVALID_ARG", -2: "FIR_OLS_ERR_UNSUPPORTED",
    -3: "FIR_OLS_ERR_NO_FILTER", -4: "FIR_OLS_ERR_ALIAS", -5: "FIR_OLS_ERR_ALIGN",
    -6: "FIR_OLS_ERR_OOM", -7: "FIR_OLS_ERR_HIP", -8: "FIR_OLS_ERR_DEVICE",
    -9: "FIR_OLS_ERR_TIMEOUT",
}


class FirOlsError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = self.name if status in STATUS else f"status {status}"
        if _lib is not None and status in STATUS:
            msg += ": " + _lib.fir_ols_status_string(status).decode()
        super().__init__(f"{where}: {msg}" if where else msg)


_lib = None
_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int


def load_library(path: Optional[str] = None):
    """Load libfirols.so (built in-tree by order_fir_filtering_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIBRARY_PATH
    if not os.path.exists(path):
        raise FirOlsError(-7, f"{path} is not built (run order_fir_filtering_amd.build.build())")
    lib = ctypes.CDLL(path)
    sig = {
        "fir_ols_plan": (_int, [ctypes.POINTER(_vp), _i64, _i64, _i64]),
        "fir_ols_set_taps": (_int, [_vp, _vp, _i64, _int, _vp]),
        "fir_ols_set_freq_response": (_int, [_vp, _vp, _i64, _vp]),
        "fir_ols_execute": (_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
        "fir_ols_execute_host": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
        "fir_ols_execute_real": (_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
        "fir_ols_execute_static": (_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
        "fir_ols_static_scratch_bytes": (_i64, []),
        "fir_ols_set_state": (_int, [_vp, _vp, _vp]),
        "fir_ols_get_state": (_int, [_vp, _vp, _vp]),
        "fir_ols_check": (_int, [_vp, _vp]),
        "fir_ols_destroy": (_int, [_vp]),
        "fir_ols_block_length": (_i64, [_vp]),
        "fir_ols_choose_n": (_i64, [_i64]),
        "fir_ols_status_string": (ctypes.c_char_p, [_int]),
        "fir_pfb_plan": (_int, [ctypes.POINTER(_vp), _i64, _i64, _i64]),
        "fir_pfb_set_taps": (_int, [_vp, _vp, _i64, _vp]),
        "fir_pfb_execute": (_int, [_vp, _vp, _vp, _i64, _vp]),
        "fir_pfb_set_state": (_int, [_vp, _vp, _i64, _vp]),
        "fir_pfb_get_state": (_int, [_vp, _vp, ctypes.POINTER(_i64), _vp]),
        "fir_pfb_destroy": (_int, [_vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    if path == LIBRARY_PATH:
        _lib = lib
    return lib


def _ptr(p) -> Optional[int]:
    if p is None:
        return None
    if hasattr(p, "data_ptr"):
        return int(p.data_ptr())
    return int(p)


def _stream(s) -> Optional[int]:
    if s is None:
        try:
            import torch
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream) or None
        except ImportError:
            pass
        return None
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream) or None
    return int(s) or None


def _check(status: int, where: str) -> None:
    if status != 0:
        raise FirOlsError(status, where)


def fir_ols_plan(M: int, N: int, nchan: int = 1) -> int:
    """Create a plan; returns the opaque handle as an integer."""
    lib = load_library()
    h = _vp()
    _check(lib.fir_ols_plan(ctypes.byref(h), M, N, nchan), "fir_ols_plan")
    return h.value


def fir_ols_set_taps(plan: int, h, stream=None) -> None:
    """Taps from host memory: real float32 or complex64 array of length M."""
    lib = load_library()
    h = np.asarray(h)
    is_complex = np.iscomplexobj(h)
    arr = np.ascontiguousarray(h, dtype=np.complex64 if is_complex else np.float32)
    _check(lib.fir_ols_set_taps(plan, arr.ctypes.data, arr.size, int(is_complex), _stream(stream)),
           "fir_ols_set_taps")


def fir_ols_set_freq_response(plan: int, H, stream=None) -> None:
    """Unscaled N-point response from host memory (complex64, bin 0 first)."""
    lib = load_library()
    arr = np.ascontiguousarray(np.asarray(H), dtype=np.complex64)
    _check(lib.fir_ols_set_freq_response(plan, arr.ctypes.data, arr.size, _stream(stream)),
           "fir_ols_set_freq_response")


def fir_ols_execute(plan: int, x, y, nsamples: int, chan_stride: int, stream=None) -> None:
    """Enqueue one call on device buffers x -> y ([nchan][chan_stride] complex64)."""
    lib = load_library()
    _check(lib.fir_ols_execute(plan, _ptr(x), _ptr(y), nsamples, chan_stride, _stream(stream)),
           "fir_ols_execute")


def fir_ols_execute_real(plan: int, x, y, nsamples: int, row_stride: int, stream=None) -> None:
    """Enqueue one call on real float32 rows ([2 nchan][row_stride] device buffers)."""
    lib = load_library()
    _check(lib.fir_ols_execute_real(plan, _ptr(x), _ptr(y), nsamples, row_stride,
                                    _stream(stream)), "fir_ols_execute_real")


def fir_ols_execute_static(plan: int, x, y, nsamples: int, chan_stride: int,
                           stream=None) -> None:
    """fir_ols_execute with the kernels' scratch in the library's fixed device
    array (no allocation in the call)."""
    lib = load_library()
    _check(lib.fir_ols_execute_static(plan, _ptr(x), _ptr(y), nsamples, chan_stride,
                                      _stream(stream)), "fir_ols_execute_static")


def fir_ols_static_scratch_bytes() -> int:
    """Size of the fixed device array fir_ols_execute_static works in."""
    return int(load_library().fir_ols_static_scratch_bytes())


def fir_ols_execute_host(plan: int, x, y, nsamples: int, chan_stride: int, chunk: int = 0,
                         stream=None) -> None:
    """Enqueue the host-resident streaming call: x, y are host addresses (or
    CPU tensors) of [nchan][chan_stride] complex64; `stream` passes the call
    after the last output copy."""
    lib = load_library()
    _check(lib.fir_ols_execute_host(plan, _ptr(x), _ptr(y), nsamples, chan_stride, chunk,
                                    _stream(stream)), "fir_ols_execute_host")


def fir_ols_set_state(plan: int, s0=None, stream=None) -> None:
    lib = load_library()
    _check(lib.fir_ols_set_state(plan, _ptr(s0), _stream(stream)), "fir_ols_set_state")


def fir_ols_get_state(plan: int, out, stream=None) -> None:
    lib = load_library()
    _check(lib.fir_ols_get_state(plan, _ptr(out), _stream(stream)), "fir_ols_get_state")


def fir_ols_check(plan: int, stream=None) -> None:
    """Synchronize the stream and raise FirOlsError(FIR_OLS_ERR_TIMEOUT) if
    a kernel wait of the plan's calls ran out (the word is then cleared)."""
    lib = load_library()
    _check(lib.fir_ols_check(plan, _stream(stream)), "fir_ols_check")


def fir_ols_destroy(plan: Optional[int]) -> None:
    lib = load_library()
    _check(lib.fir_ols_destroy(plan), "fir_ols_destroy")


def fir_ols_block_length(plan: int) -> int:
    lib = load_library()
    L = lib.fir_ols_block_length(plan)
    if L < 0:
        raise FirOlsError(int(L), "fir_ols_block_length")
    return int(L)


def fir_ols_choose_n(M: int) -> int:
    """Planner choice of the FFT length N for M taps (see include/firols.h)."""
    N = load_library().fir_ols_choose_n(M)
    if N < 0:
        raise FirOlsError(int(N), "fir_ols_choose_n")
    return int(N)


def fir_ols_status_string(status: int) -> str:
    return load_library().fir_ols_status_string(status).decode()


class Plan:
    """Owning wrapper of a plan that works on torch complex64 device tensors."""

    def __init__(self, M: int, N: int, nchan: int = 1):
        self.M, self.N, self.nchan = int(M), int(N), int(nchan)
        self.handle = fir_ols_plan(self.M, self.N, self.nchan)
        self.L = fir_ols_block_length(self.handle)

    def set_taps(self, h, stream=None) -> "Plan":
        fir_ols_set_taps(self.handle, h, stream)
        return self

    def set_freq_response(self, H, stream=None) -> "Plan":
        fir_ols_set_freq_response(self.handle, H, stream)
        return self

    def _layout(self, x):
        import torch
        if x.dtype != torch.complex64 or not x.is_cuda:
            raise FirOlsError(-1, "execute: x must be a complex64 device tensor")
        if x.dim() == 1:
            if self.nchan != 1:
                raise FirOlsError(-1, "execute: x must be [nchan, n]")
            return x.shape[0], max(x.shape[0], 1)
        if x.dim() != 2 or x.shape[0] != self.nchan or (x.shape[1] > 1 and x.stride(1) != 1):
            raise FirOlsError(-1, "execute: x must be [nchan, n] with unit inner stride")
        return x.shape[1], max(x.stride(0), x.shape[1])

    def execute(self, x, y=None, stream=None):
        """Filter x (shape [n] or [nchan, n]); returns y (same shape/strides)."""
        import torch
        n, stride = self._layout(x)
        if y is None:
            y = torch.empty_strided(x.shape, x.stride(), dtype=x.dtype, device=x.device)
        elif y.shape != x.shape or y.stride() != x.stride() or y.dtype != x.dtype:
            raise FirOlsError(-1, "execute: y must match x in shape, strides and dtype")
        fir_ols_execute(self.handle, x, y, n, stride, stream)
        return y

    def execute_host(self, x, y=None, chunk: int = 0, stream=None):
        """Filter a host (CPU, ideally pinned) complex64 tensor x of shape [n]
        or [nchan, n] through the host-resident streaming call; returns y
        (a pinned CPU tensor unless given) once the stream has passed it."""
        import torch
        if x.dtype != torch.complex64 or x.is_cuda:
            raise FirOlsError(-1, "execute_host: x must be a complex64 CPU tensor")
        if x.dim() == 1:
            if self.nchan != 1:
                raise FirOlsError(-1, "execute_host: x must be [nchan, n]")
            n, stride = x.shape[0], max(x.shape[0], 1)
        elif x.dim() == 2 and x.shape[0] == self.nchan and (x.shape[1] <= 1 or x.stride(1) == 1):
            n, stride = x.shape[1], max(x.stride(0), x.shape[1])
        else:
            raise FirOlsError(-1, "execute_host: x must be [nchan, n] with unit inner stride")
        if y is None:
            y = torch.empty_strided(x.shape, x.stride(), dtype=x.dtype, pin_memory=True)
        elif y.shape != x.shape or y.stride() != x.stride() or y.dtype != x.dtype or y.is_cuda:
            raise FirOlsError(-1, "execute_host: y must be a CPU tensor matching x")
        fir_ols_execute_host(self.handle, x, y, n, stride, chunk, stream)
        s = stream if stream is not None else torch.cuda.current_stream()
        (s if hasattr(s, "synchronize") else torch.cuda.current_stream()).synchronize()
        return y

    def set_state(self, s0=None, stream=None) -> None:
        fir_ols_set_state(self.handle, s0, stream)

    def get_state(self, stream=None):
        import torch
        out = torch.empty((self.nchan, self.M - 1), dtype=torch.complex64, device="cuda")
        fir_ols_get_state(self.handle, out, stream)
        return out

    def check(self, stream=None) -> None:
        fir_ols_check(self.handle, stream)

    def close(self) -> None:
        if getattr(self, "handle", None):
            fir_ols_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


# Polyphase filter-bank channelizer (include/firpfb.h).

def fir_pfb_plan(K: int, D: int, Nh: int) -> int:
    """Create a channelizer plan; returns the opaque handle as an integer."""
    lib = load_library()
    h = _vp()
    _check(lib.fir_pfb_plan(ctypes.byref(h), K, D, Nh), "fir_pfb_plan")
    return h.value


def fir_pfb_set_taps(plan: int, h, stream=None) -> None:
    """Real prototype taps from host memory (float32, length Nh)."""
    lib = load_library()
    arr = np.ascontiguousarray(np.asarray(h), dtype=np.float32)
    _check(lib.fir_pfb_set_taps(plan, arr.ctypes.data, arr.size, _stream(stream)),
           "fir_pfb_set_taps")


def fir_pfb_execute(plan: int, x, y, nsamples: int, stream=None) -> None:
    _check(load_library().fir_pfb_execute(plan, _ptr(x), _ptr(y), nsamples, _stream(stream)),
           "fir_pfb_execute")


def fir_pfb_set_state(plan: int, s=None, t_next: int = 0, stream=None) -> None:
    _check(load_library().fir_pfb_set_state(plan, _ptr(s), t_next, _stream(stream)),
           "fir_pfb_set_state")


def fir_pfb_get_state(plan: int, out=None, stream=None) -> int:
    """Copies the state to out (if given); returns the next stream time."""
    t = _i64(0)
    _check(load_library().fir_pfb_get_state(plan, _ptr(out), ctypes.byref(t), _stream(stream)),
           "fir_pfb_get_state")
    return int(t.value)


def fir_pfb_destroy(plan: Optional[int]) -> None:
    if plan:
        _check(load_library().fir_pfb_destroy(plan), "fir_pfb_destroy")


class Channelizer:
    """Owning wrapper of a channelizer plan on torch complex64 device tensors."""

    def __init__(self, K: int, D: int, Nh: int):
        self.K, self.D, self.Nh = int(K), int(D), int(Nh)
        self.handle = fir_pfb_plan(self.K, self.D, self.Nh)

    def set_taps(self, h, stream=None) -> "Channelizer":
        fir_pfb_set_taps(self.handle, h, stream)
        return self

    def execute(self, x, y=None, stream=None):
        """Channelize x (complex64 [n], n a multiple of D); returns y [n / D, K]."""
        import torch
        if x.dtype != torch.complex64 or not x.is_cuda or x.dim() != 1 or (
                x.shape[0] > 1 and x.stride(0) != 1):
            raise FirOlsError(-1, "execute: x must be a contiguous complex64 device vector")
        n = x.shape[0]
        if y is None:
            y = torch.empty((n // self.D, self.K), dtype=x.dtype, device=x.device)
        elif y.shape != (n // self.D, self.K) or not y.is_contiguous() or y.dtype != x.dtype:
            raise FirOlsError(-1, "execute: y must be a contiguous [n / D, K] complex64 tensor")
        fir_pfb_execute(self.handle, x, y, n, stream)
        return y

    def set_state(self, s=None, t_next: int = 0, stream=None) -> None:
        fir_pfb_set_state(self.handle, s, t_next, stream)

    def get_state(self, stream=None):
        """(state tensor [Nh - 1], next stream time)."""
        import torch
        out = torch.empty((max(self.Nh - 1, 1),), dtype=torch.complex64, device="cuda")
        t = fir_pfb_get_state(self.handle, out, stream)
        return out[:self.Nh - 1], t

    def close(self) -> None:
        if getattr(self, "handle", None):
            fir_pfb_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
