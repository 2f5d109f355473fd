"""Float64 CPU oracle of the polyphase filter-bank channelizer.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
``bench.py`` may import this module.  The product library never calls it,
and it shares no code with the HIP path.

Source: the polyphase-channelizer page ("GPU polyphase filter bank
channelizer", sections 2.1 and 2.2).  Section 2.1 describes each sub-band
as the wide-band input shifted down to baseband, low-pass filtered by the
prototype h and decimated by D; its three steps (decimate into branches,
filter each branch with its polyphase component h(nK + k), DFT across the
branches) are a fast way to compute that.  Section 2.2 gives the 50 %
overlapping design, K channels at decimation D = K / 2; the page's kernels
use D = K (one branch per channel, critically sampled).  This oracle is
the definition, written out:

    y_c(m) = sum_{p=0}^{Nh-1} h(p) * xt(t_m - p) * exp(-2 pi j c (t_m - p) / K)

for channel c in [0, K), output m of a call, t_m = t0 + m D + D - 1 the
stream time of the last input sample of output m's hop, t0 the stream time
of the call's first sample, and xt the stream: the call's samples at
times t0 .. t0 + n - 1, the state (the Nh - 1 samples before t0, oldest
first) before them, zeros before that.  The phase uses the absolute stream
time, so channel c comes out at baseband.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def channel_table(K: int) -> np.ndarray:
    """W[c, e] = exp(-2 pi j c e / K) in float64 (c, e in [0, K))."""
    c = np.arange(K)
    return np.exp(-2j * np.pi * np.outer(c, c) / K)


def pfb_channelize(h, x, K: int, D: int, state=None, t0: int = 0,
                   idx: Optional[np.ndarray] = None) -> np.ndarray:
    """Outputs y[m, c] of one call (complex128, [n/D, K], or [len(idx), K]).

    h: real or complex prototype taps (Nh); x: the call's n samples (n a
    multiple of D); state: the Nh - 1 samples before the call (None: zeros);
    t0: stream time of x[0]; idx: the output indices m to compute (default
    all).  Every output is the sum over p of the definition, one output at
    a time.
    """
    h = np.asarray(h).astype(np.complex128).ravel()
    x = np.asarray(x, dtype=np.complex64).ravel().astype(np.complex128)
    Nh = h.size
    n = x.size
    if K < 1 or D < 1 or n % D:
        raise ValueError("need K, D >= 1 and a multiple of D samples")
    st = (np.zeros(Nh - 1) if state is None
          else np.asarray(state, dtype=np.complex64).ravel().astype(np.complex128))
    if st.size != Nh - 1:
        raise ValueError("state must hold Nh - 1 samples")
    xt = np.concatenate([st, x])            # xt[j + Nh - 1] is the sample at time t0 + j
    W = channel_table(K)
    ms = np.arange(n // D) if idx is None else np.asarray(idx, dtype=np.int64)
    y = np.empty((ms.size, K), dtype=np.complex128)
    p = np.arange(Nh)
    for row, m in enumerate(ms):
        j = m * D + D - 1 - p                # time of each tap's sample, relative to t0
        samples = xt[j + Nh - 1]             # j >= -(Nh - 1) always
        e = (t0 + j) % K                     # absolute time mod K
        y[row] = W[:, e] @ (h * samples)
    return y


def pfb_state_next(x, state, Nh: int) -> np.ndarray:
    """The last Nh - 1 samples of {state, x} (complex64, oldest first)."""
    x = np.asarray(x, dtype=np.complex64).ravel()
    st = (np.zeros(Nh - 1, np.complex64) if state is None
          else np.asarray(state, dtype=np.complex64).ravel())
    s = np.concatenate([st, x])
    return s[s.size - (Nh - 1):].copy()


def pfb_parity_bound(h, x, state=None, rel: float = 1e-5) -> float:
    """rel * max|xt| * sum|h|: every output is a sum of Nh products of a
    tap, a sample and a unit phase, so its float32 rounding error scales
    with max|xt| * sum|h|."""
    hh = np.abs(np.asarray(h).astype(np.complex128)).sum()
    mx = float(np.abs(np.asarray(x)).max()) if np.size(x) else 0.0
    if state is not None and np.size(state):
        mx = max(mx, float(np.abs(np.asarray(state)).max()))
    return rel * mx * float(hh)
