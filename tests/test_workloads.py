"""Pins of the seeded workload generators (CPU only)."""
import numpy as np
import pytest
import scipy.signal

import workloads as W


@pytest.mark.parametrize("M", [65, 257, 1025])
def test_hamming_sinc_matches_firwin(M):
    h = W.hamming_sinc(M)
    ref = scipy.signal.firwin(M, 0.25, window="hamming")     # cutoff rel. to Nyquist
    assert h.dtype == np.float32
    np.testing.assert_allclose(h, ref.astype(np.float32), rtol=0, atol=2e-9)
    assert abs(float(h.astype(np.float64).sum()) - 1.0) < 1e-6
    np.testing.assert_allclose(h, h[::-1], rtol=0, atol=1e-9)
    # gain at the cutoff (0.25 pi rad/sample) of a windowed-sinc design is ~ -6 dB
    g = np.abs(np.sum(h.astype(np.float64) * np.exp(-1j * 0.25 * np.pi * np.arange(M))))
    assert abs(g - 0.5) < 0.01


def test_complex_normal_layout_and_determinism():
    a = W.complex_normal(np.random.default_rng(5), (3, 1000))
    b = W.complex_normal(np.random.default_rng(5), (3, 1000))
    np.testing.assert_array_equal(a, b)
    assert a.dtype == np.complex64 and a.shape == (3, 1000)
    g = np.random.default_rng(5)
    re = g.standard_normal(3000, dtype=np.float32)
    im = g.standard_normal(3000, dtype=np.float32)
    np.testing.assert_array_equal(a.ravel().real, re)
    np.testing.assert_array_equal(a.ravel().imag, im)
    big = W.complex_normal(np.random.default_rng(6), 200000)
    assert abs(big.real.var() - 1) < 0.02 and abs(big.imag.mean()) < 0.01


def test_freq_response_input_is_dft_of_padded_taps():
    rng = np.random.default_rng(3)
    h = W.complex_taps(rng, 5)
    H = W.freq_response_input(h, 16)
    q = np.arange(16)
    want = np.array([np.sum(h * np.exp(-2j * np.pi * k * np.arange(5) / 16)) for k in q])
    np.testing.assert_allclose(H, want, rtol=0, atol=1e-6)
    assert H.dtype == np.complex64


@pytest.mark.parametrize("key", sorted(W.WORKLOADS))
def test_workload_shapes(key):
    w = W.WORKLOADS[key]
    assert w.N == w.L + w.M - 1
    assert sum(w.calls) == w.samples
    inp = W.make_inputs(key, samples=min(w.samples, 5000))
    assert inp.x.shape == (w.nchan, min(w.samples, 5000))
    assert inp.s0.shape == (w.nchan, w.M - 1)
    assert (inp.H is None) == (w.taps != "complex_H")
    if w.state == "zero":
        assert not inp.s0.any()
    # seeded: same call, same numbers
    again = W.make_inputs(key, samples=min(w.samples, 5000))
    np.testing.assert_array_equal(inp.x, again.x)


def test_sample_indices():
    i = W.sample_indices(1, 1000, 50)
    assert i.size == 50 and np.all(np.diff(i) > 0) and i.min() >= 0 and i.max() < 1000


@pytest.mark.parametrize("key", sorted(W.PFB_WORKLOADS))
def test_channelizer_prototype_is_the_pages_design_call(key):
    """The channelizer workloads' prototype is the window-method design the
    channelizer page gives (section 2.2: a Hamming window, cutoff 1/D of
    Nyquist), i.e. scipy's firwin(Nh, 1/D, window='hamming'); the input is
    seeded and reproducible."""
    w = W.PFB_WORKLOADS[key]
    h, x = W.make_pfb_inputs(key, samples=4096)
    ref = scipy.signal.firwin(w["Nh"], 1.0 / w["D"], window="hamming")
    assert h.dtype == np.float32 and h.size == w["Nh"]
    np.testing.assert_allclose(h, ref.astype(np.float32), rtol=0, atol=2e-9)
    assert x.dtype == np.complex64 and x.shape == (4096,)
    h2, x2 = W.make_pfb_inputs(key, samples=4096)
    np.testing.assert_array_equal(x, x2)
    assert w["K"] % w["D"] == 0 and w["samples"] % w["D"] == 0
