"""fir_ols_execute_host (host-resident streaming) and fir_ols_choose_n through the C ABI.

The host call cuts the stream into chunks and runs one filtering call per
chunk, so its output must equal, bit for bit, fir_ols_execute over the same
chunks on device copies of the data; and, like every path, the float64
oracle within the parity bound.  Pinned and pageable host memory, padded
channel strides, several calls in a row (the state carried), and the
argument checks.
"""
import os

import numpy as np
import pytest

import workloads as W
import order_fir_filtering_amd as fo
import oracle
from gpu_util import say, to_dev, check

THREADS = min(16, len(os.sched_getaffinity(0)))

pytestmark = pytest.mark.gpu


def _filter(p, h, N):
    if N == 65536:
        p.set_freq_response(W.freq_response_input(h, N))
    else:
        p.set_taps(h)


def _device_chunked(N, M, h, x, s0, chunk, stride):
    """fir_ols_execute over the chunks the host call uses, on device copies."""
    import torch
    nchan, n = x.shape
    xp = np.zeros((nchan, stride), np.complex64)
    xp[:, :n] = x
    xd = to_dev(xp)
    yd = torch.zeros_like(xd)
    with fo.Plan(M, N, nchan) as p:
        _filter(p, h, N)
        p.set_state(to_dev(s0))
        eff = min(chunk, n)
        for c0 in range(0, n, eff):
            c = min(eff, n - c0)
            fo.fir_ols_execute(p.handle, xd.data_ptr() + 8 * c0, yd.data_ptr() + 8 * c0, c,
                               stride, None)
        torch.cuda.synchronize()
    return yd.cpu().numpy()[:, :n]


CASES = [(1024, 257, 3, 20000), (4096, 1025, 1, 100000), (32768, 8193, 1, 120000),
         (65536, 16385, 1, 150000), (131072, 32769, 2, 300000)]


@pytest.mark.parametrize("N,M,nchan,n", CASES)
@pytest.mark.parametrize("chunk_kind", ["short", "odd", "default"])
def test_host_stream_equals_device_chunks(N, M, nchan, n, chunk_kind):
    import torch
    L = N - M + 1
    chunk = {"short": max(L - 1, 1), "odd": 3 * L + 5, "default": 0}[chunk_kind]
    eff = chunk if chunk else -(-((1 << 22) // nchan) // L) * L
    say(f"host stream: N={N} M={M} nchan={nchan} n={n} chunk={chunk} ({eff})")
    rng = np.random.default_rng(N + M + n + chunk)
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (nchan, n))
    s0 = W.complex_normal(rng, (nchan, M - 1))
    stride = n + 9
    xh = torch.zeros((nchan, stride), dtype=torch.complex64, pin_memory=True)
    xh[:, :n] = torch.from_numpy(x)
    yh = torch.full((nchan, stride), complex(5.0, 5.0), dtype=torch.complex64, pin_memory=True)
    stream = torch.cuda.Stream()
    with fo.Plan(M, N, nchan) as p:
        _filter(p, h, N)
        p.set_state(to_dev(s0), stream)
        fo.fir_ols_execute_host(p.handle, xh.data_ptr(), yh.data_ptr(), n, stride, chunk, stream)
        stream.synchronize()
        st = p.get_state(stream)
        stream.synchronize()
        st = st.cpu().numpy()
    y = yh.numpy()
    assert np.all(y[:, n:] == np.complex64(complex(5.0, 5.0)))      # padding untouched
    want = _device_chunked(N, M, h, x, s0, eff, stride)
    np.testing.assert_array_equal(y[:, :n], want)
    idx = np.unique(np.concatenate([np.arange(0, n, max(n // 3000, 1)), [n - 1]]))
    ref = oracle.fir_direct_multi(h, x, s0, idx=idx, threads=THREADS)
    check(y[:, idx], ref, h, x, s0, f"host stream N={N} chunk={chunk}")
    for c in range(nchan):
        np.testing.assert_array_equal(st[c], oracle.state_next(x[c], s0[c], M))


def test_host_stream_calls_in_a_row_and_pageable_memory():
    import torch
    N, M, n1, n2 = 4096, 1025, 50001, 33333
    rng = np.random.default_rng(5)
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (1, n1 + n2))
    s0 = np.zeros((1, M - 1), np.complex64)
    # pageable host memory (numpy arrays), two calls carrying the state
    y = np.zeros_like(x)
    with fo.Plan(M, N, 1) as p:
        p.set_taps(h)
        fo.fir_ols_execute_host(p.handle, x.ctypes.data, y.ctypes.data, n1, n1 + n2, 7000, None)
        fo.fir_ols_execute_host(p.handle, x.ctypes.data + 8 * n1, y.ctypes.data + 8 * n1, n2,
                                n1 + n2, 0, None)
        torch.cuda.synchronize()
    idx = np.unique(np.concatenate([np.arange(0, n1 + n2, 17), [n1 - 1, n1, n1 + 1]]))
    ref = oracle.fir_direct_multi(h, x, s0, idx=idx, threads=THREADS)
    check(y[:, idx], ref, h, x, s0, "two host calls, pageable")
    # the Plan wrapper on a pinned tensor equals the raw call
    xt = torch.from_numpy(x[0, :n1].copy()).pin_memory()
    with fo.Plan(M, N, 1) as p:
        p.set_taps(h)
        yt = p.execute_host(xt, chunk=7000)
    np.testing.assert_array_equal(yt.numpy(), y[0, :n1])


def test_host_stream_argument_checks():
    import torch
    x = torch.zeros(1000, dtype=torch.complex64, pin_memory=True)
    with fo.Plan(257, 1024, 1) as p:
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_host(p.handle, x.data_ptr(), x.data_ptr() + 8, 100, 100, 0, None)
        assert e.value.status == -3                 # no filter yet
        p.set_taps(np.ones(257, np.float32))
        fo.fir_ols_execute_host(p.handle, x.data_ptr(), x.data_ptr(), 0, 0, 0, None)   # no-op
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_host(p.handle, x.data_ptr(), x.data_ptr() + 8 * 50, 100, 100, 0,
                                    None)
        assert e.value.status == -4                 # overlapping host ranges
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_host(p.handle, x.data_ptr(), x.data_ptr() + 8 * 500, 100, 100,
                                    -1, None)
        assert e.value.status == -1                 # negative chunk
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_host(p.handle, x.data_ptr(), x.data_ptr() + 8 * 500, 100, 99, 0,
                                    None)
        assert e.value.status == -1                 # stride below nsamples
        torch.cuda.synchronize()


@pytest.mark.parametrize("M", [1, 203, 1025, 5000, 70000])
def test_planner_choice_runs_and_matches_the_oracle(M):
    """A plan with the N that fir_ols_choose_n picks filters correctly."""
    N = fo.fir_ols_choose_n(M)
    say(f"planner: M={M} -> N={N}")
    rng = np.random.default_rng(M)
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (1, 3 * N + 17))
    s0 = W.complex_normal(rng, (1, M - 1))
    from gpu_util import run_calls
    with fo.Plan(M, N, 1) as p:
        p.set_taps(h)
        y = run_calls(p, x, [x.shape[1]], s0)
    n = x.shape[1]
    idx = np.unique(np.concatenate([np.arange(min(n, 2000)), np.arange(0, n, max(7, n // 3000)),
                                    [n - 1]]))
    ref = oracle.fir_direct_multi(h, x, s0, idx=idx, threads=THREADS)
    check(y[:, idx], ref, h, x, s0, f"planner M={M} N={N}")
