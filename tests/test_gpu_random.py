"""Seeded random sweeps over every kernel family and entry point, every
output checked.

Each case draws N (8 .. 2^20, so the fused, 16384, 32768, paired/split and
multi-pass kernels all appear), M (1, 2, small, up to N/2, up to N, and a
few values of M - 1 near a multiple of 4 or 64), the channel count, a
ragged length of up to a dozen blocks cut into one to three calls, complex
or real-pair input, a padded row stride, and at N = 65536 whether the
filter comes as taps or as its response.  Every output of every channel
is compared with the oracle's float64 block overlap-save (the method
page, claim 1, steps 3-5), and the carried state with the last M - 1
samples (step 6).  Fixed cases chose M - 1 as a multiple of 4 at the
large sizes and so missed the negative-offset bug of the real-pair
gathers; random draws are what found it.
"""
import numpy as np
import pytest

import workloads as W
import order_fir_filtering_amd as fo
import oracle
from gpu_util import say, to_dev, check

pytestmark = pytest.mark.gpu

NCASES = 40
SAMPLE_CAP = 3_000_000          # samples per channel
TOTAL_CAP = 4_000_000           # samples over all channels


def _draw(k):
    rng = np.random.default_rng(20_000 + k)
    logn = int(rng.choice([3, 5, 8, 10, 12, 13, 14, 14, 15, 15, 16, 16, 16, 17, 18, 20]))
    N = 1 << logn
    kind = int(rng.integers(0, 6))
    if kind == 0:
        M = int(rng.choice([1, 2]))
    elif kind == 1:
        M = int(rng.integers(2, min(64, N) + 1))
    elif kind == 2:
        M = int(rng.integers(2, N // 2 + 1))
    elif kind == 3:
        M = int(rng.integers(N // 2, N + 1))
    else:
        # M - 1 just off a multiple of 4 or 64
        base = int(rng.integers(1, max(2, N // 128))) * int(rng.choice([4, 64]))
        M = min(N, max(1, base + int(rng.integers(-3, 4)) + 1))
    L = N - M + 1
    nchan = int(rng.integers(1, 4))
    nblk = int(rng.integers(1, 13 if L > 64 else 40))
    n = max(1, nblk * L + int(rng.integers(-L + 1, L)))
    n = min(n, SAMPLE_CAP, TOTAL_CAP // nchan)
    real = bool(rng.integers(0, 2))
    ncalls = int(rng.integers(1, 4))
    cuts = (sorted(rng.choice(np.arange(1, n), size=min(ncalls - 1, n - 1), replace=False))
            if n > 1 else [])
    calls = [int(c) for c in np.diff([0] + [int(c) for c in cuts] + [n])]
    pad = int(rng.choice([0, 0, 3, 64]))
    use_h = N == 65536 and not real and bool(rng.integers(0, 2))
    return rng, N, M, nchan, n, real, calls, pad, use_h


@pytest.mark.parametrize("k", range(NCASES))
def test_random_case_matches_block_ols(k):
    import torch
    rng, N, M, nchan, n, real, calls, pad, use_h = _draw(k)
    say(f"random case {k}: N={N} M={M} nchan={nchan} n={n} real={real} calls={calls} "
        f"pad={pad} response={use_h}")
    stride = n + pad
    if real:
        h = (rng.standard_normal(M) / np.sqrt(M)).astype(np.float32)
        rows = rng.standard_normal((2 * nchan, n)).astype(np.float32)
        s0 = W.complex_normal(rng, (nchan, M - 1))
        xp = np.zeros((2 * nchan, stride), np.float32)
        xp[:, :n] = rows
        x = (rows[0::2] + 1j * rows[1::2]).astype(np.complex64)
    else:
        h = W.complex_taps(rng, M).astype(np.complex64)
        x = W.complex_normal(rng, (nchan, n))
        s0 = W.complex_normal(rng, (nchan, M - 1))
        xp = np.zeros((nchan, stride), np.complex64)
        xp[:, :n] = x
    xd = to_dev(xp)
    yd = torch.full_like(xd, 7.0)
    item = xd.element_size()
    with fo.Plan(M, N, nchan) as p:
        if use_h:
            p.set_freq_response(W.freq_response_input(h, N))
        else:
            p.set_taps(h)
        p.set_state(to_dev(s0))
        pos = 0
        for c in calls:
            f = fo.fir_ols_execute_real if real else fo.fir_ols_execute
            f(p.handle, xd.data_ptr() + item * pos, yd.data_ptr() + item * pos, c, stride, None)
            pos += c
        st = p.get_state().cpu().numpy()
        p.check()
    y = yd.cpu().numpy()
    assert np.all(y[:, n:] == 7.0)                    # the padding is never written
    y = y[:, :n]
    got = y[0::2] + 1j * y[1::2] if real else y
    H = np.fft.fft(np.asarray(h, np.complex128), N)
    for c in range(nchan):
        ref = oracle.fir_ols_blocks(H, x[c], s0[c], M)
        check(got[c], ref, h, x[c:c + 1], s0[c:c + 1], f"case {k} ch {c}")
        np.testing.assert_array_equal(st[c], oracle.state_next(x[c], s0[c], M))


NMIXED = 16


@pytest.mark.parametrize("k", range(NMIXED))
def test_random_mixed_entry_points_carry_one_stream(k):
    """Consecutive calls on one plan through fir_ols_execute,
    fir_ols_execute_static (no allocation) and fir_ols_execute_host
    (host-resident, random chunk sizes) in random order: together they must
    filter the stream as one pass does, every output and the final state."""
    import torch
    rng = np.random.default_rng(30_000 + k)
    N = 1 << int(rng.choice([5, 8, 10, 12, 14, 15, 16, 17]))
    M = int(rng.choice([1, int(rng.integers(2, N // 2 + 1)), int(rng.integers(N // 2, N + 1))]))
    L = N - M + 1
    nchan = int(rng.integers(1, 4))
    n = max(1, min(int(rng.integers(1, 7)) * L + int(rng.integers(-L + 1, L)), 600_000 // nchan))
    ncalls = int(rng.integers(2, 7))
    cuts = (sorted(rng.choice(np.arange(1, n), size=min(ncalls - 1, n - 1), replace=False))
            if n > 1 else [])
    calls = [int(c) for c in np.diff([0] + [int(c) for c in cuts] + [n])]
    kinds = [str(rng.choice(["dev", "static", "host"])) for _ in calls]
    pad = int(rng.choice([0, 5]))
    say(f"mixed case {k}: N={N} M={M} nchan={nchan} n={n} calls={calls} kinds={kinds}")
    stride = n + pad
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (nchan, n))
    s0 = W.complex_normal(rng, (nchan, M - 1))
    xp = np.zeros((nchan, stride), np.complex64)
    xp[:, :n] = x
    xd = to_dev(xp)
    yd = torch.full_like(xd, 7.0)
    xh = torch.from_numpy(xp).pin_memory()
    yh = torch.full_like(xh, 7.0).pin_memory()
    on_host = np.zeros(n, bool)
    with fo.Plan(M, N, nchan) as p:
        p.set_taps(h)
        p.set_state(to_dev(s0))
        pos = 0
        for c, kd in zip(calls, kinds):
            off = 8 * pos
            if kd == "dev":
                fo.fir_ols_execute(p.handle, xd.data_ptr() + off, yd.data_ptr() + off, c, stride)
            elif kd == "static":
                fo.fir_ols_execute_static(p.handle, xd.data_ptr() + off, yd.data_ptr() + off, c,
                                          stride)
            else:
                # (one-sample chunks, one launch per sample, on short calls only)
                chunk = int(rng.choice([0, 1 if c <= 200 else L, L, 3 * L + 5]))
                fo.fir_ols_execute_host(p.handle, xh.data_ptr() + off, yh.data_ptr() + off, c,
                                        stride, chunk)
                on_host[pos:pos + c] = True
            pos += c
        st = p.get_state().cpu().numpy()
        torch.cuda.synchronize()
        p.check()
    y = yd.cpu().numpy().copy()
    yhost = yh.numpy()
    assert np.all(y[:, n:] == 7.0) and np.all(yhost[:, n:] == 7.0)
    y = y[:, :n]
    y[:, on_host] = yhost[:, :n][:, on_host]
    H = np.fft.fft(np.asarray(h, np.complex128), N)
    for c in range(nchan):
        ref = oracle.fir_ols_blocks(H, x[c], s0[c], M)
        check(y[c], ref, h, x[c:c + 1], s0[c:c + 1], f"mixed case {k} ch {c}")
        np.testing.assert_array_equal(st[c], oracle.state_next(x[c], s0[c], M))
