"""Float64 CPU oracle for overlap-save FIR filtering.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  The product
library never calls it, and it shares no code with the HIP path.

Source of truth: the method page "一种基于GPU的高阶数字FIR滤波器频域并行处理实现
方法" (a GPU frequency-domain parallel method for high-order FIR filters),
abstract and claim 1, steps 1-6.

* ``fir_direct`` — the plain definition the method reaches exactly: linear
  convolution of the taps with the stream {S0, X} (claim 1, steps 3-5; the
  abstract says the method is FIR filtering).  Plain float64 loops in C
  (``direct_form.c``).
* ``state_next`` — the state handed to the next call: the last M-1 samples of
  {S0, X} (claim 1, step 3: D_{k-1} is moved into S0).
* ``fir_ols_blocks`` — the method's own steps, for the frequency-response
  entry with an arbitrary H that need not come from an M-tap filter (claim 1,
  step 1 second case, then steps 3-5).  There the result is a per-block
  circular convolution and has no simpler definition.  numpy's FFT serves as
  the N-point transform; the inverse carries the 1/N factor.
* ``parity_bound`` — the accepted error of a complex64 result:
  1e-5 * max|xt| * sum|h|.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "direct_form.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile direct_form.c into liboracle.so with gcc (float64, OpenMP)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
             "-o", tmp, _SRC])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_SO)
        lib.oracle_fir_direct.restype = ctypes.c_int
        lib.oracle_fir_direct.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_int]
        _lib = lib
    return _lib


def _taps128(h) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(h).astype(np.complex128).ravel())


def fir_direct(h, x, s0=None, idx=None, threads: int = 1) -> np.ndarray:
    """y[t] = sum_m h[m] xt[t-m] in float64 for one stream.

    h: M taps (real or complex, any float dtype); x: complex64 samples;
    s0: complex64 state of M-1 samples (oldest first) or None for zeros;
    idx: output indices to compute (default: all).  Returns complex128.
    """
    lib = _load()
    hh = _taps128(h)
    M = hh.size
    xx = np.ascontiguousarray(np.asarray(x, dtype=np.complex64).ravel())
    n = xx.size
    if s0 is not None:
        ss = np.ascontiguousarray(np.asarray(s0, dtype=np.complex64).ravel())
        if ss.size != M - 1:
            raise ValueError("state must hold M-1 samples")
        s_ptr = ss.ctypes.data if M > 1 else None
    else:
        ss, s_ptr = None, None
    if idx is None:
        ii, i_ptr, count = None, None, n
    else:
        ii = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).ravel())
        i_ptr, count = ii.ctypes.data, ii.size
    y = np.empty(count, dtype=np.complex128)
    rc = lib.oracle_fir_direct(hh.ctypes.data, M, s_ptr,
                               xx.ctypes.data if n else None, n, i_ptr,
                               count, y.ctypes.data if count else None, threads)
    if rc != 0:
        raise ValueError("oracle_fir_direct rejected its arguments")
    return y


def fir_direct_multi(h, x, s0=None, idx=None, threads: int = 1) -> np.ndarray:
    """fir_direct over channels: x [nchan, n], s0 [nchan, M-1] or None."""
    x = np.asarray(x)
    out = []
    for c in range(x.shape[0]):
        out.append(fir_direct(h, x[c], None if s0 is None else s0[c], idx, threads))
    return np.stack(out) if out else np.zeros((0, 0), np.complex128)


def state_next(x, s0, M: int) -> np.ndarray:
    """Last M-1 samples of the stream {S0, X} (complex64, oldest first)."""
    x = np.asarray(x, dtype=np.complex64).ravel()
    s0 = (np.zeros(M - 1, np.complex64) if s0 is None
          else np.asarray(s0, dtype=np.complex64).ravel())
    stream = np.concatenate([s0, x])
    return stream[stream.size - (M - 1):].copy()


def fir_ols_blocks(H, x, s0, M: int) -> np.ndarray:
    """The method's steps 3-5 for a given N-point response H (float64).

    N = len(H), L = N - M + 1.  The stream xt = {S0, X, zeros}; block i is
    E_i = xt[iL : iL + N] (E_0 = {S0, B_0}, E_i = {D_(i-1), B_i});
    F_i = FFT(E_i); I_i = F_i * H; R_i = IFFT(I_i) with the 1/N factor;
    Y_i = R_i[M-1 : M-1+L].  Returns the first len(x) outputs.
    """
    H = np.asarray(H, dtype=np.complex128).ravel()
    N = H.size
    L = N - M + 1
    if L < 1:
        raise ValueError("need N >= M")
    x = np.asarray(x, dtype=np.complex64).ravel().astype(np.complex128)
    n = x.size
    s0 = (np.zeros(M - 1) if s0 is None
          else np.asarray(s0, dtype=np.complex64).ravel().astype(np.complex128))
    k = -(-n // L)
    xt = np.concatenate([s0, x, np.zeros(k * L + N - (M - 1) - n + L)])
    y = np.empty(k * L, dtype=np.complex128)
    for i in range(k):
        E = xt[i * L: i * L + N]
        F = np.fft.fft(E)
        R = np.fft.ifft(F * H)
        y[i * L:(i + 1) * L] = R[M - 1:M - 1 + L]
    return y[:n]


def parity_bound(h, x, s0=None, rel: float = 1e-5) -> float:
    """rel * max|xt| * sum|h|, xt = the samples and state used by the run."""
    hh = np.asarray(h).astype(np.complex128).ravel()
    mx = 0.0
    if np.size(x):
        mx = float(np.abs(np.asarray(x)).max())
    if s0 is not None and np.size(s0):
        mx = max(mx, float(np.abs(np.asarray(s0)).max()))
    return rel * mx * float(np.abs(hh).sum())
