"""Pins of the channelizer oracle against facts it does not compute itself.

Source: the polyphase-channelizer page ("GPU polyphase filter bank
channelizer", section 2.1: shift each sub-band to baseband, low-pass filter
with the prototype, decimate; section 2.2: K channels at D = K / 2).  The
checks: hand-worked outputs (tests/golden/pfb_hand_worked.txt), the
one-channel case reducing to numpy's convolution, the explicit
shift-filter-decimate route per channel through numpy's convolution, a
tone's closed form (the prototype's response at the frequency offset,
evaluated by Horner's rule), and streaming with carried state and time.
"""
import os

import numpy as np
import pytest

from oracle import pfb_channelize, pfb_parity_bound, pfb_state_next

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pfb_hand_worked.txt")


def load_golden():
    cases, cur = {}, None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "case":
                cur = cases.setdefault(vals[0], {})
            else:
                cur[key] = np.array([complex(v) for v in vals])
    return cases


def rand_c64(rng, n):
    return (rng.standard_normal(n) + 1j * rng.standard_normal(n)).astype(np.complex64)


@pytest.mark.parametrize("name", ["k2d1", "k2d2"])
def test_golden(name):
    c = load_golden()[name]
    K, D = int(c["K"][0].real), int(c["D"][0].real)
    y = pfb_channelize(c["h"].real, c["x"], K, D)
    np.testing.assert_allclose(y[:, 0], c["y0"], atol=1e-12)
    np.testing.assert_allclose(y[:, 1], c["y1"], atol=1e-12)


def test_one_channel_is_numpy_convolution():
    rng = np.random.default_rng(1)
    h = rng.standard_normal(37)
    x = rand_c64(rng, 500)
    y = pfb_channelize(h, x, 1, 1)
    want = np.convolve(h, x.astype(np.complex128))[:x.size]
    np.testing.assert_allclose(y[:, 0], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("K,D,Nh,t0", [(8, 4, 40, 0), (16, 16, 64, 5), (32, 16, 100, 77),
                                       (4, 2, 9, 3)])
def test_shift_filter_decimate_route(K, D, Nh, t0):
    """Each channel by the explicit route: multiply the stream (state
    included) by exp(-2 pi j c t / K) at its absolute times, convolve with h
    (numpy), keep the samples at t_m."""
    rng = np.random.default_rng(K * 100 + Nh)
    h = rng.standard_normal(Nh)
    n = 12 * D
    x = rand_c64(rng, n)
    st = rand_c64(rng, Nh - 1)
    y = pfb_channelize(h, x, K, D, state=st, t0=t0)
    stream = np.concatenate([st, x]).astype(np.complex128)
    times = t0 - (Nh - 1) + np.arange(stream.size)
    for c in range(K):
        shifted = stream * np.exp(-2j * np.pi * c * (times % K) / K)
        full = np.convolve(h, shifted)                   # full[i] pairs with stream[i]
        keep = (Nh - 1) + np.arange(n // D) * D + D - 1
        np.testing.assert_allclose(y[:, c], full[keep], rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("c0", [0, 3, 7])
def test_tone_closed_form(c0):
    """x(t) = exp(2 pi j c0 t / K) on both sides of t0: channel c sees
    exp(2 pi j (c0 - c) t_m / K) times the prototype's response
    sum_p h(p) z^p at z = exp(-2 pi j (c0 - c) / K)."""
    K, D, Nh, t0 = 8, 4, 24, 11
    rng = np.random.default_rng(c0)
    h = rng.standard_normal(Nh)
    n = 10 * D
    t = np.arange(t0 - (Nh - 1), t0 + n)
    tone = np.exp(2j * np.pi * c0 * t / K)
    st, x = tone[:Nh - 1], tone[Nh - 1:]
    y = pfb_channelize(h, x.astype(np.complex64), K, D, state=st.astype(np.complex64), t0=t0)
    tm = t0 + np.arange(n // D) * D + D - 1
    for c in range(K):
        z = np.exp(-2j * np.pi * (c0 - c) / K)
        gain = np.polyval(h[::-1], z)
        want = np.exp(2j * np.pi * (c0 - c) * tm / K) * gain
        np.testing.assert_allclose(y[:, c], want, rtol=1e-6, atol=1e-6)


def test_streaming_equals_one_shot():
    K, D, Nh = 16, 8, 70
    rng = np.random.default_rng(5)
    h = rng.standard_normal(Nh)
    x = rand_c64(rng, 40 * D)
    st = rand_c64(rng, Nh - 1)
    one = pfb_channelize(h, x, K, D, state=st, t0=3)
    parts, s, t0, pos = [], st, 3, 0
    for n in (5 * D, D, 34 * D):
        parts.append(pfb_channelize(h, x[pos:pos + n], K, D, state=s, t0=t0))
        s = pfb_state_next(x[pos:pos + n], s, Nh)
        pos += n
        t0 += n
    np.testing.assert_allclose(np.concatenate(parts), one, rtol=1e-12, atol=1e-12)


def test_index_subset_and_bound():
    K, D, Nh = 8, 8, 16
    rng = np.random.default_rng(9)
    h = rng.standard_normal(Nh)
    x = rand_c64(rng, 20 * D)
    full = pfb_channelize(h, x, K, D)
    idx = np.array([0, 3, 19])
    np.testing.assert_array_equal(pfb_channelize(h, x, K, D, idx=idx), full[idx])
    b = pfb_parity_bound(h, x)
    assert b == pytest.approx(1e-5 * np.abs(x).max() * np.abs(h).sum())
    with pytest.raises(ValueError):
        pfb_channelize(h, x[:D + 1], K, D)
