"""Pins of the float64 oracle against facts it does not compute itself.

Each test checks the oracle against something fixed independently of its
code: hand-worked values, closed-form sums, numpy's convolution, the
method's own steps written with explicit DFT matrices, and invariants
(streaming with carried state, linearity, time invariance).  Method page:
"一种基于GPU的高阶数字FIR滤波器频域并行处理实现方法", claim 1.
"""
import os

import numpy as np
import pytest

from oracle import fir_direct, fir_ols_blocks, parity_bound, state_next

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.txt")


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


def dft_matrix(N):
    q = np.arange(N)
    return np.exp(-2j * np.pi * np.outer(q, q) / N)


def rand_c64(rng, n):
    return (rng.standard_normal(n) + 1j * rng.standard_normal(n)).astype(np.complex64)


def test_golden_real3():
    c = load_golden()["real3"]
    M, N = int(c["M"][0].real), int(c["N"][0].real)
    h = c["h"].real
    s0 = c["s0"].astype(np.complex64)
    x = c["x"].astype(np.complex64)
    y = fir_direct(h, x, s0)
    np.testing.assert_array_equal(y, c["y"])
    np.testing.assert_array_equal(state_next(x, s0, M), c["s0_next"].astype(np.complex64))
    # the page's block steps with H = DFT of the zero-padded taps
    F = dft_matrix(N)
    H = F @ np.concatenate([h, np.zeros(N - M)])
    np.testing.assert_allclose(fir_ols_blocks(H, x, s0, M), c["y"], atol=1e-12)
    # dropped points Z_0: circular convolution of E_0 = {S0, B_0} with h
    E0 = np.concatenate([c["s0"], c["x"][: N - (M - 1)]])
    R0 = [sum(h[m] * E0[(t - m) % N] for m in range(M)) for t in range(N)]
    np.testing.assert_allclose(R0[: M - 1], c["z0"], atol=0)
    np.testing.assert_allclose(R0[M - 1:], c["y"][: N - M + 1], atol=0)


def test_golden_complex2_two_calls():
    c = load_golden()["complex2"]
    M = int(c["M"][0].real)
    h = c["h"]
    s0 = c["s0"].astype(np.complex64)
    x = c["x"].astype(np.complex64)
    np.testing.assert_array_equal(fir_direct(h, x, s0), c["y"])
    s1 = state_next(x, s0, M)
    np.testing.assert_array_equal(s1, c["s0_next"].astype(np.complex64))
    x2 = c["x2"].astype(np.complex64)
    np.testing.assert_array_equal(fir_direct(h, x2, s1), c["y2"])
    np.testing.assert_array_equal(state_next(x2, s1, M), c["s0_next2"].astype(np.complex64))


@pytest.mark.parametrize("M", [1, 2, 7, 64, 65])
def test_impulse_returns_taps(M):
    rng = np.random.default_rng(M)
    h = rng.standard_normal(M) + 1j * rng.standard_normal(M)
    n = M + 9
    x = np.zeros(n, np.complex64)
    x[0] = 1
    y = fir_direct(h, x)
    np.testing.assert_array_equal(y[:M], h)
    np.testing.assert_array_equal(y[M:], 0)


@pytest.mark.parametrize("d", [-5, -1, 0, 3, 17])
def test_shifted_impulse_in_input_and_state(d):
    M, n = 6, 30
    rng = np.random.default_rng(100 + d)
    h = rng.standard_normal(M)
    x = np.zeros(n, np.complex64)
    s0 = np.zeros(M - 1, np.complex64)
    if d >= 0:
        x[d] = 1
    else:
        s0[M - 1 + d] = 1          # S0[M-1+d] is stream sample d
    y = fir_direct(h, x, s0)
    want = np.zeros(n, np.complex128)
    for t in range(n):
        if 0 <= t - d < M:
            want[t] = h[t - d]
    np.testing.assert_array_equal(y, want)


@pytest.mark.parametrize("omega", [2 * np.pi * 5 / 64, 0.3, 1.9, -2.2])
def test_geometric_taps_sinusoid_closed_form(omega):
    # h[m] = a^m: the response to e^{j w t} is e^{j w t} (1-(a e^{-jw})^M)/(1-a e^{-jw})
    M, n = 40, 300
    a = 0.93 * np.exp(0.4j)
    h = a ** np.arange(M)
    t = np.arange(-(M - 1), n)
    xt = np.exp(1j * omega * t).astype(np.complex64)
    y = fir_direct(h, xt[M - 1:], xt[: M - 1])
    r = a * np.exp(-1j * omega)
    gain = (1 - r ** M) / (1 - r)
    want = gain * np.exp(1j * omega * np.arange(n))
    scale = np.abs(h).sum()
    assert np.abs(y - want).max() < 2e-7 * scale


@pytest.mark.parametrize("q,N", [(3, 64), (0, 16), (7, 32)])
def test_boxcar_sinusoid_dirichlet(q, N):
    # h = 1 (M taps): gain = e^{-jw(M-1)/2} sin(wM/2)/sin(w/2), gain(0) = M
    M, n = 11, 100
    omega = 2 * np.pi * q / N + 0.01
    h = np.ones(M)
    t = np.arange(-(M - 1), n)
    xt = np.exp(1j * omega * t).astype(np.complex64)
    y = fir_direct(h, xt[M - 1:], xt[: M - 1])
    gain = np.exp(-1j * omega * (M - 1) / 2) * np.sin(omega * M / 2) / np.sin(omega / 2)
    want = gain * np.exp(1j * omega * np.arange(n))
    assert np.abs(y - want).max() < 2e-7 * M


def test_random_vs_numpy_convolve():
    rng = np.random.default_rng(7)
    for trial in range(60):
        M = int(rng.integers(1, 80))
        n = int(rng.choice([0, 1, 2, max(M - 2, 0), M, int(rng.integers(1, 400))]))
        complex_taps = trial % 2 == 0
        h = rng.standard_normal(M) + (1j * rng.standard_normal(M) if complex_taps else 0)
        x = rand_c64(rng, n)
        s0 = rand_c64(rng, M - 1)
        y = fir_direct(h, x, s0)
        full = np.convolve(h, np.concatenate([s0, x]).astype(np.complex128))
        want = full[M - 1: M - 1 + n]
        assert y.shape == (n,)
        if n:
            np.testing.assert_allclose(y, want, rtol=0, atol=1e-12 * max(1, np.abs(h).sum()) * 10)


@pytest.mark.parametrize("N", [4, 8, 16, 32, 64])
def test_literal_ols_steps_with_dft_matrices(N):
    """The method's steps 2-5 with explicit DFT matrices equal the oracle."""
    rng = np.random.default_rng(N)
    F = dft_matrix(N)
    Finv = np.conj(F) / N
    for M in sorted({1, 2, N // 4 + 1, N // 2, N}):
        L = N - M + 1
        h = rng.standard_normal(M) + 1j * rng.standard_normal(M)
        for n in (1, L, 3 * L + 1, 5 * L):
            x = rand_c64(rng, n)
            s0 = rand_c64(rng, M - 1)
            k = -(-n // L)
            xt = np.concatenate([s0, x, np.zeros(k * L + N)]).astype(np.complex128)
            H = F @ np.concatenate([h, np.zeros(N - M)])
            ys = []
            for i in range(k):
                E = xt[i * L: i * L + N]            # {D_(i-1), B_i}; E_0 = {S0, B_0}
                R = Finv @ ((F @ E) * H)
                ys.append(R[M - 1: M - 1 + L])      # drop Z_i (M-1 points), keep Y_i
            y_lit = np.concatenate(ys)[:n]
            y = fir_direct(h, x, s0)
            tol = 1e-11 * np.abs(h).sum() * max(1.0, np.abs(xt).max())
            np.testing.assert_allclose(y, y_lit, rtol=0, atol=tol)
            np.testing.assert_allclose(fir_ols_blocks(H, x, s0, M), y_lit, rtol=0, atol=tol)


@pytest.mark.parametrize("N,M", [(4, 2), (8, 3), (16, 16), (16, 1)])
def test_ols_blocks_arbitrary_response_is_circular_convolution(N, M):
    """For an H that is no M-tap filter, each kept point is circular."""
    rng = np.random.default_rng(N * 100 + M)
    H = rng.standard_normal(N) + 1j * rng.standard_normal(N)
    F = dft_matrix(N)
    g = (np.conj(F) @ H) / N                          # g = IDFT(H)
    L = N - M + 1
    n = 3 * L + 2
    x = rand_c64(rng, n)
    s0 = rand_c64(rng, M - 1)
    xt = np.concatenate([s0, x, np.zeros(4 * L + N)]).astype(np.complex128)
    want = np.empty(n, np.complex128)
    for t_all in range(n):
        i, t = divmod(t_all, L)
        E = xt[i * L: i * L + N]
        want[t_all] = sum(g[m] * E[(M - 1 + t - m) % N] for m in range(N))
    y = fir_ols_blocks(H, x, s0, M)
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-11 * np.abs(g).sum() * 5)


def test_chunked_streaming_equals_one_shot():
    rng = np.random.default_rng(11)
    for M in (1, 2, 9, 33):
        h = rng.standard_normal(M) + 1j * rng.standard_normal(M)
        x = rand_c64(rng, 500)
        s0 = rand_c64(rng, M - 1)
        once = fir_direct(h, x, s0)
        cuts = [1, max(M - 2, 1), 0, 7, 64, 3, 1]
        parts, state, pos = [], s0, 0
        for c in cuts + [x.size]:
            c = min(c, x.size - pos)
            chunk = x[pos: pos + c]
            parts.append(fir_direct(h, chunk, state))
            state = state_next(chunk, state, M)
            pos += c
            if pos == x.size:
                break
        np.testing.assert_array_equal(np.concatenate(parts), once)
        np.testing.assert_array_equal(state, state_next(x, s0, M))


def test_linearity_and_time_invariance():
    rng = np.random.default_rng(12)
    M, n = 17, 200
    h = rng.standard_normal(M) + 1j * rng.standard_normal(M)
    # values on a 2^-8 grid, so a*x1 + b*x2 is exact in complex64
    q = lambda v: (np.round(v * 256) / 256).astype(np.complex64)
    x1, x2 = q(rand_c64(rng, n)), q(rand_c64(rng, n))
    s1, s2 = q(rand_c64(rng, M - 1)), q(rand_c64(rng, M - 1))
    a, b = 0.5, -2.0
    y = fir_direct(h, (a * x1 + b * x2).astype(np.complex64),
                   (a * s1 + b * s2).astype(np.complex64))
    np.testing.assert_allclose(y, a * fir_direct(h, x1, s1) + b * fir_direct(h, x2, s2),
                               rtol=0, atol=1e-12 * np.abs(h).sum() * 10)
    d = 23
    xs = np.concatenate([np.zeros(d, np.complex64), x1])
    np.testing.assert_array_equal(fir_direct(h, xs)[d:], fir_direct(h, x1))


def test_index_subset_and_threads_agree():
    rng = np.random.default_rng(13)
    M, n = 50, 3000
    h = rng.standard_normal(M)
    x = rand_c64(rng, n)
    s0 = rand_c64(rng, M - 1)
    full = fir_direct(h, x, s0)
    idx = np.array([0, 1, M - 2, M - 1, 1234, n - 1])
    np.testing.assert_array_equal(fir_direct(h, x, s0, idx=idx), full[idx])
    np.testing.assert_array_equal(fir_direct(h, x, s0, threads=4), full)


def test_bad_arguments_rejected():
    h = np.ones(4)
    x = np.zeros(10, np.complex64)
    with pytest.raises(ValueError):
        fir_direct(h, x, idx=[10])
    with pytest.raises(ValueError):
        fir_direct(h, x, idx=[-1])
    with pytest.raises(ValueError):
        fir_direct(h, x, s0=np.zeros(2, np.complex64))


def test_state_next_cases():
    s0 = np.array([1, 2, 3], np.complex64)
    np.testing.assert_array_equal(state_next(np.array([9, 8, 7, 6], np.complex64), s0, 4), [8, 7, 6])
    np.testing.assert_array_equal(state_next(np.array([9], np.complex64), s0, 4), [2, 3, 9])
    np.testing.assert_array_equal(state_next(np.array([], np.complex64), s0, 4), [1, 2, 3])
    assert state_next(np.array([5], np.complex64), None, 1).size == 0


def test_parity_bound_value():
    h = np.array([1.0, -2.0, 0.5])
    x = np.array([3 + 4j, 1], np.complex64)
    s0 = np.array([0, 1j], np.complex64)
    assert parity_bound(h, x, s0) == pytest.approx(1e-5 * 5.0 * 3.5)
