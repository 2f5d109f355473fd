"""fir_ols_execute_real: real float32 rows filtered two at a time.

Each real row is checked against the float64 oracle run on that row alone
(as a complex stream with zero imaginary part, whose output's real part is
the row's filtered stream), so the packing of two rows into one complex
channel is checked, not assumed.  Sizes cover every fused-kernel form
(several blocks per wave, one wave per block, register-held and table-fed
twiddles, pointer I/O at N = 16384), the half-resident (N = 32768), split
(N = 65536) and multi-pass (N = 2^17, 2^18) kernels, ragged lengths,
padded row strides, calls carrying the state, calls shorter than the
state, and the argument checks.
"""
import os

import numpy as np
import pytest

import workloads as W
import order_fir_filtering_amd as fo
import oracle
from gpu_util import say, to_dev, check

pytestmark = pytest.mark.gpu
THREADS = max(1, min(16, os.cpu_count() or 1))


def _run_real(M, N, rows, calls, s0c=None, stride_pad=5):
    """Feed float32 rows [2 nchan, n] as consecutive calls; returns y rows and the state."""
    import torch
    nrow, n = rows.shape
    stride = n + stride_pad
    xp = np.zeros((nrow, stride), np.float32)
    xp[:, :n] = rows
    xd = to_dev(xp)
    yd = torch.full_like(xd, 3.0)
    with fo.Plan(M, N, nrow // 2) as p:
        p.set_taps(HREAL[(M, N)])
        if s0c is not None:
            p.set_state(to_dev(s0c))
        pos = 0
        for c in calls:
            fo.fir_ols_execute_real(p.handle, xd.data_ptr() + 4 * pos, yd.data_ptr() + 4 * pos, c,
                                    stride, None)
            pos += c
        st = p.get_state()
        torch.cuda.synchronize()
        st = st.cpu().numpy()
    y = yd.cpu().numpy()
    assert np.all(y[:, n:] == 3.0)            # padding between rows untouched
    return y[:, :n], st


HREAL = {}
CASES = [(65, 256, 2, [12288]), (257, 1024, 4, [30001, 7, 2000]), (1025, 4096, 2, [50000, 1, 9999]),
         (2049, 8192, 2, [40000]), (4097, 16384, 2, [70000, 3]), (3, 8, 2, [100, 5]),
         # the half-resident, split and multi-pass kernels
         (8193, 32768, 2, [80000, 5, 30001]), (1, 32768, 2, [40000]),
         (16385, 65536, 2, [150000, 7, 20000]), (30000, 65536, 4, [20000]),
         (32769, 131072, 2, [250000, 3]), (100001, 262144, 2, [50000, 300000])]


@pytest.mark.parametrize("M,N,nrow,calls", CASES)
def test_real_rows_match_the_oracle_per_row(M, N, nrow, calls):
    say(f"real rows: M={M} N={N} rows={nrow} calls={calls}")
    rng = np.random.default_rng(M * 7 + N)
    h = (rng.standard_normal(M) / np.sqrt(M)).astype(np.float32)
    HREAL[(M, N)] = h
    n = sum(calls)
    rows = rng.standard_normal((nrow, n)).astype(np.float32)
    s1 = rng.standard_normal((nrow, M - 1)).astype(np.float32)
    s0c = (s1[0::2] + 1j * s1[1::2]).astype(np.complex64)      # packed states of the pairs
    y, st = _run_real(M, N, rows, calls, s0c)
    idx = np.unique(np.concatenate([np.arange(0, n, 11), [n - 1]]))
    for r in range(nrow):
        xr = rows[r:r + 1].astype(np.complex64)
        sr = s1[r:r + 1].astype(np.complex64)
        ref = oracle.fir_direct_multi(h, xr, sr, idx=idx, threads=THREADS)
        check(y[r:r + 1, idx], ref.real, h, xr, sr, f"row {r}")
    # the carried state: the last M-1 samples of each pair, packed
    for c in range(nrow // 2):
        want = oracle.state_next(rows[2 * c] + 1j * rows[2 * c + 1], s0c[c], M)
        np.testing.assert_array_equal(st[c], want.astype(np.complex64))


def test_real_rows_equal_complex_channel_bitwise():
    """Two real rows give, bit for bit, the real and imaginary parts of the
    complex path on the packed channel (same kernels, same arithmetic)."""
    import torch
    M, N, n = 1025, 4096, 77777
    rng = np.random.default_rng(3)
    h = (rng.standard_normal(M) / np.sqrt(M)).astype(np.float32)
    HREAL[(M, N)] = h
    rows = rng.standard_normal((2, n)).astype(np.float32)
    y, _ = _run_real(M, N, rows, [n], stride_pad=0)
    z = to_dev((rows[0] + 1j * rows[1]).astype(np.complex64)[None, :])
    with fo.Plan(M, N, 1) as p:
        p.set_taps(h)
        yz = p.execute(z)
        torch.cuda.synchronize()
    yz = yz.cpu().numpy()[0]
    np.testing.assert_array_equal(y[0], yz.real)
    np.testing.assert_array_equal(y[1], yz.imag)


def test_real_argument_checks():
    import torch
    x = torch.zeros((2, 100), dtype=torch.float32, device="cuda")
    y = torch.zeros_like(x)
    with fo.Plan(65, 256, 1) as p:
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_real(p.handle, x, y, 100, 100)
        assert e.value.status == -3                       # no filter yet
        p.set_taps(np.ones(65, np.complex64))             # complex taps
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_real(p.handle, x, y, 100, 100)
        assert e.value.status == -2
        p.set_freq_response(np.ones(256, np.complex64))   # a response, not real taps
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_real(p.handle, x, y, 100, 100)
        assert e.value.status == -2
        p.set_taps(np.ones(65, np.float32))
        fo.fir_ols_execute_real(p.handle, x, y, 0, 0)     # no-op
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_real(p.handle, x, x, 100, 100)
        assert e.value.status == -4                       # overlap
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_real(p.handle, x.data_ptr() + 2, y, 10, 100)
        assert e.value.status == -5                       # alignment
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_real(p.handle, x, y, 100, 99)
        assert e.value.status == -1                       # stride below nsamples
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,blocks", [(4097, 16384, 700), (8193, 32768, 3), (16385, 65536, 3),
                                        (32769, 131072, 3)])
def test_real_rows_equal_complex_channel_bitwise_large(M, N, blocks):
    """As above for the large-N kernels: the real-pair forms compute what the
    complex forms do on the packed channel, bit for bit (at N = 16384 with
    more blocks than resident workgroups, so each runs several)."""
    import torch
    rng = np.random.default_rng(M)
    h = (rng.standard_normal(M) / np.sqrt(M)).astype(np.float32)
    HREAL[(M, N)] = h
    n = blocks * (N - M + 1) + 777
    rows = rng.standard_normal((2, n)).astype(np.float32)
    y, _ = _run_real(M, N, rows, [n], stride_pad=0)
    z = to_dev((rows[0] + 1j * rows[1]).astype(np.complex64)[None, :])
    with fo.Plan(M, N, 1) as p:
        p.set_taps(h)
        yz = p.execute(z)
        torch.cuda.synchronize()
    yz = yz.cpu().numpy()[0]
    np.testing.assert_array_equal(y[0], yz.real)
    np.testing.assert_array_equal(y[1], yz.imag)


@pytest.mark.parametrize("N,Mm1", [(16384, 1769), (16384, 1770), (16384, 1771),
                                   (32768, 2997), (32768, 2998), (32768, 2999),
                                   (65536, 9001), (65536, 9002), (65536, 9003)])
def test_real_rows_with_state_length_not_a_multiple_of_four(N, Mm1):
    """Every output near the start of each call, at M - 1 = 1, 2, 3 (mod 4)
    and N = 16384, 32768, 65536.  In the first block of a call, the threads
    below M - 1 index the input at negative positions (the state lies
    there) while their neighbours read x[0], x[1], ...; with 4-byte rows
    the neighbours' offsets 0, 4, 8 sit next to wrapped negative ones, and
    the outputs that hold x[0] .. x[2] (and, in the paired kernel, the
    stores of outputs 0 and 1) must still be right.  The complex channel of
    the same rows must agree bit for bit."""
    import torch
    M = Mm1 + 1
    say(f"real rows, M-1 mod 4 = {Mm1 % 4}: M={M} N={N}")
    rng = np.random.default_rng(Mm1)
    h = (rng.standard_normal(M) / np.sqrt(M)).astype(np.float32)
    HREAL[(M, N)] = h
    L = N - Mm1
    calls = [2 * L + 501, 3 * L + 77]
    n = sum(calls)
    rows = rng.standard_normal((2, n)).astype(np.float32)
    s1 = rng.standard_normal((2, Mm1)).astype(np.float32)
    s0c = (s1[0::2] + 1j * s1[1::2]).astype(np.complex64)
    y, st = _run_real(M, N, rows, calls, s0c)
    starts = np.concatenate([np.arange(0, M + 256), calls[0] + np.arange(0, M + 256)])
    idx = np.unique(np.concatenate([starts, np.arange(0, n, 13), [n - 1]]))
    for r in range(2):
        xr = rows[r:r + 1].astype(np.complex64)
        sr = s1[r:r + 1].astype(np.complex64)
        ref = oracle.fir_direct_multi(h, xr, sr, idx=idx, threads=THREADS)
        check(y[r:r + 1, idx], ref.real, h, xr, sr, f"row {r}")
    want = oracle.state_next(rows[0] + 1j * rows[1], s0c[0], M)
    np.testing.assert_array_equal(st[0], want.astype(np.complex64))
    # the packed complex channel, same calls, same state
    z = to_dev((rows[0] + 1j * rows[1]).astype(np.complex64)[None, :])
    yz = torch.empty_like(z)
    with fo.Plan(M, N, 1) as p:
        p.set_taps(h)
        p.set_state(to_dev(s0c))
        pos = 0
        for c in calls:
            yz[:, pos:pos + c] = p.execute(z[:, pos:pos + c].contiguous())
            pos += c
        torch.cuda.synchronize()
    yz = yz.cpu().numpy()[0]
    np.testing.assert_array_equal(y[0], yz.real)
    np.testing.assert_array_equal(y[1], yz.imag)
