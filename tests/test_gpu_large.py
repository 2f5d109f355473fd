"""GPU parity of the large-N paths, N = 32768 and 65536.

Full-size workloads are checked on sampled outputs the float64 direct-form
oracle computes one by one (four whole blocks: first, second, middle,
last, plus 65536 seeded random indices), and on every output against the
oracle's float64 block overlap-save (numpy FFTs), which the CPU tests pin
to the direct form.  Small cases cover every output with the direct form.
"""
import os

import numpy as np
import pytest

import oracle
import order_fir_filtering_amd as fo
import workloads as W
from gpu_util import check, run_calls, say, to_dev

pytestmark = pytest.mark.gpu
THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    fo.load_library()
    yield
    torch.cuda.synchronize()


def sampled_indices(w, seed):
    L, k = w.L, w.samples // w.L
    blocks = [np.arange(b * L, (b + 1) * L) for b in (0, 1, k // 2, k - 1)]
    return np.unique(np.concatenate(blocks + [W.sample_indices(seed, w.samples, 65536)]))


def test_cfg3_sampled():
    inp = W.make_inputs("cfg3")
    w = inp.workload
    say(f"cfg3: M={w.M} N={w.N} n={w.samples}")
    with fo.Plan(w.M, w.N) as p:
        p.set_taps(inp.taps)
        y = run_calls(p, inp.x, w.calls)
        st = p.get_state().cpu().numpy()
    idx = sampled_indices(w, 33)
    ref = oracle.fir_direct(inp.h_ref, inp.x[0], inp.s0[0], idx=idx, threads=THREADS)
    check(y[0, idx], ref, inp.h_ref, inp.x, inp.s0, f"cfg3 ({idx.size} outputs)")
    np.testing.assert_array_equal(st[0], oracle.state_next(inp.x[0], inp.s0[0], w.M))
    H = np.fft.fft(np.asarray(inp.h_ref, dtype=np.complex128), w.N)
    full = oracle.fir_ols_blocks(H, inp.x[0], inp.s0[0], w.M)
    check(y[0], full, inp.h_ref, inp.x, inp.s0, f"cfg3 (all {w.samples} outputs, block OLS)")


def test_cfg4_frequency_response_sampled():
    inp = W.make_inputs("cfg4")
    w = inp.workload
    say(f"cfg4: M={w.M} N={w.N} n={w.samples} (H given)")
    with fo.Plan(w.M, w.N) as p:
        p.set_freq_response(inp.H)
        y = run_calls(p, inp.x, w.calls)
    idx = sampled_indices(w, 44)
    ref = oracle.fir_direct(inp.h_ref, inp.x[0], inp.s0[0], idx=idx, threads=THREADS)
    check(y[0, idx], ref, inp.h_ref, inp.x, inp.s0, f"cfg4 ({idx.size} outputs)")
    full = oracle.fir_ols_blocks(inp.H, inp.x[0], inp.s0[0], w.M)
    check(y[0], full, inp.h_ref, inp.x, inp.s0, f"cfg4 (all {w.samples} outputs, block OLS)")


def _large_cases():
    rng = np.random.default_rng(77)
    cases = []
    for N in (32768, 65536):
        for M in (1, 2, 1025, N // 3, N):
            L = N - M + 1
            for n in sorted({1, max(M - 2, 1), L + 3, 3 * L + int(rng.integers(0, L))}):
                n = min(n, 300000, 2000 * L)
                cases.append((N, M, n, int(rng.choice([1, 2])), int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("N,M,n,nchan,seed", _large_cases())
def test_large_sizes(N, M, n, nchan, seed):
    # N = 65536 goes through the frequency-response entry here; its taps entry
    # is covered by test_large_taps_and_freq_response_agree_and_stream
    say(f"large: N={N} M={M} n={n} nchan={nchan} seed={seed}")
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal(M) + 1j * rng.standard_normal(M)).astype(np.complex64)
    x = W.complex_normal(rng, (nchan, n))
    s0 = W.complex_normal(rng, (nchan, M - 1))
    with fo.Plan(M, N, nchan) as p:
        if N == 65536:
            p.set_freq_response(W.freq_response_input(h, N))
        else:
            p.set_taps(h)
        y = run_calls(p, x, [n], s0=s0)
        st = p.get_state().cpu().numpy()
    idx = np.unique(np.concatenate([np.arange(min(n, 3000)), np.arange(max(0, n - 3000), n),
                                    W.sample_indices(seed, n, 4000)]))
    ref = oracle.fir_direct_multi(h, x, s0, idx=idx, threads=THREADS)
    check(y[:, idx], ref, h, x, s0, f"N={N} M={M} n={n}")
    for c in range(nchan):
        np.testing.assert_array_equal(st[c], oracle.state_next(x[c], s0[c], M))


@pytest.mark.parametrize("N,M", [(32768, 8193), (65536, 16385)])
def test_large_taps_and_freq_response_agree_and_stream(N, M):
    say(f"large taps vs H, chunked calls: N={N} M={M}")
    rng = np.random.default_rng(N + M)
    h = W.complex_taps(rng, M).astype(np.complex64)
    L = N - M + 1
    calls = [L // 2, 1, 2 * L + 5, M - 2, 3 * L]
    x = W.complex_normal(rng, (1, sum(calls)))
    with fo.Plan(M, N) as pa, fo.Plan(M, N) as pb:
        pa.set_taps(h)
        pb.set_freq_response(W.freq_response_input(h, N))
        ya = run_calls(pa, x, calls)
        yb = run_calls(pb, x, [x.shape[1]])
    idx = np.unique(np.concatenate([np.arange(0, x.shape[1], 7), [x.shape[1] - 1]]))
    ref = oracle.fir_direct(h, x[0], None, idx=idx, threads=THREADS)
    check(ya[0, idx], ref, h, x, None, "set_taps, chunked calls")
    check(yb[0, idx], ref, h, x, None, "set_freq_response")


@pytest.mark.parametrize("N,M,d", [(32768, 8193, 8192), (65536, 16385, 12345)])
def test_large_delay_response(N, M, d):
    say(f"large delay: N={N} M={M} d={d}")
    rng = np.random.default_rng(d)
    x = W.complex_normal(rng, (1, 3 * N))
    s0 = W.complex_normal(rng, (1, M - 1))
    H = np.exp(-2j * np.pi * np.arange(N) * d / N).astype(np.complex64)
    with fo.Plan(M, N) as p:
        p.set_freq_response(H)
        y = run_calls(p, x, [x.shape[1]], s0=s0)
    xt = np.concatenate([s0[0], x[0]])
    want = xt[M - 1 - d: M - 1 - d + x.shape[1]]
    check(y, want.astype(np.complex128), np.ones(1), x, s0, "delay")


@pytest.mark.parametrize("N,M", [(32768, 8193), (65536, 16385)])
def test_large_repeat_is_bitwise_identical(N, M):
    say(f"large determinism: N={N} M={M}")
    rng = np.random.default_rng(3)
    h = rng.standard_normal(M).astype(np.float32)
    x = W.complex_normal(rng, (1, 400000))
    outs = []
    for _ in range(2):
        with fo.Plan(M, N) as p:
            if N == 65536:
                p.set_freq_response(W.freq_response_input(h, N))
            else:
                p.set_taps(h)
            outs.append(run_calls(p, x, [123457, 276543]))
    np.testing.assert_array_equal(outs[0], outs[1])


@pytest.mark.parametrize("N,M", [(32768, 4097), (65536, 20000)])
def test_large_multichannel_padded_stride_streaming(N, M):
    # three channels 77 elements apart beyond their length, fed as several
    # calls (each call reads and writes a sub-range of every row)
    import torch
    say(f"large multichannel: N={N} M={M}")
    rng = np.random.default_rng(N ^ M)
    nchan, L = 3, N - M + 1
    calls = [L + 11, 2, M - 5, 2 * L]
    n = sum(calls)
    stride = n + 77
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (nchan, n))
    s0 = W.complex_normal(rng, (nchan, M - 1))
    xp = np.zeros((nchan, stride), np.complex64)
    xp[:, :n] = x
    xd = to_dev(xp)
    yd = torch.full_like(xd, complex(7.0, -7.0))
    with fo.Plan(M, N, nchan) as p:
        if N == 65536:
            p.set_freq_response(W.freq_response_input(h, N))
        else:
            p.set_taps(h)
        p.set_state(to_dev(s0))
        pos = 0
        for c in calls:
            fo.fir_ols_execute(p.handle, xd.data_ptr() + 8 * pos, yd.data_ptr() + 8 * pos, c,
                               stride, None)
            pos += c
        torch.cuda.synchronize()
        st = p.get_state().cpu().numpy()
    y = yd.cpu().numpy()
    # the padding between rows is untouched
    assert np.all(y[:, n:] == np.complex64(complex(7.0, -7.0)))
    idx = np.unique(np.concatenate([np.arange(0, n, 13), [n - 1]]))
    ref = oracle.fir_direct_multi(h, x, s0, idx=idx, threads=THREADS)
    check(y[:, idx], ref, h, x, s0, f"N={N} {nchan} channels, stride {stride}")
    for c in range(nchan):
        np.testing.assert_array_equal(st[c], oracle.state_next(x[c], s0[c], M))


@pytest.mark.parametrize("var,value", [("FIROLS_PAIR_QUEUES", "16"), ("FIROLS_PAIR_QUEUES", "1"),
                                       ("FIROLS_PAIR_LEAD", "1"), ("FIROLS_PAIR_LEAD", "64")])
def test_paired_kernel_schedules_are_bitwise_equal(var, value, monkeypatch):
    """The N = 65536 paired kernel under other schedules gives the same
    outputs and state, bit for bit, as the default, and meets the oracle
    bound on sampled outputs.  The schedules: its work in more queues than
    the GPU has XCDs (the last workgroup runs the unserved ones alone), in
    one queue, or with producers handed out 1 or 64 blocks ahead of their
    consumers."""
    say(f"paired kernel, {var}={value}")
    M, N = 16385, 65536
    rng = np.random.default_rng(int(value))
    h = W.complex_taps(rng, M).astype(np.complex64)
    L = N - M + 1
    n = 37 * L + 1000
    x = W.complex_normal(rng, (2, n))
    s0 = W.complex_normal(rng, (2, M - 1))
    H = W.freq_response_input(h, N)
    with fo.Plan(M, N, 2) as pa:
        pa.set_freq_response(H)
        ya = run_calls(pa, x, [n], s0=s0)
        sa = pa.get_state().cpu().numpy()
    monkeypatch.setenv(var, value)
    with fo.Plan(M, N, 2) as pb:
        pb.set_freq_response(H)
        yb = run_calls(pb, x, [n], s0=s0)
        sb = pb.get_state().cpu().numpy()
    monkeypatch.delenv(var)
    np.testing.assert_array_equal(yb, ya)
    np.testing.assert_array_equal(sb, sa)
    idx = np.unique(np.concatenate([np.arange(3000), W.sample_indices(5, n, 3000),
                                    np.arange(n - 2000, n)]))
    ref = oracle.fir_direct_multi(h, x, s0, idx=idx, threads=THREADS)
    check(yb[:, idx], ref, h, x, s0, f"{var}={value}")


def test_paired_wait_timeout_reports_error(monkeypatch):
    """A consumer whose bounded wait for the producer's parked half-spectrum
    runs out.  The timeout is forced from the host: with
    FIROLS_PAIR_HOLD_READY=1 at plan creation the producers raise no flag
    and the bound is 10 us, so every kernel still ends normally.
    fir_ols_check reports FIR_OLS_ERR_TIMEOUT once and clears it.  The full
    blocks' outputs are NaN, not a combine with stale data.  The partial
    last block (the one-workgroup kernel, which waits for nothing) and the
    state are still right.  A plan made without the switch is unaffected."""
    M, N = 16385, 65536
    L = N - M + 1
    n = 3 * L + 1000
    rng = np.random.default_rng(41)
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (1, n))
    s0 = W.complex_normal(rng, (1, M - 1))
    H = W.freq_response_input(h, N)
    say("paired kernel, FIROLS_PAIR_HOLD_READY=1 (every consumer's wait runs out)")
    monkeypatch.setenv("FIROLS_PAIR_HOLD_READY", "1")
    with fo.Plan(M, N, 1) as p:
        monkeypatch.delenv("FIROLS_PAIR_HOLD_READY")
        p.set_freq_response(H)
        y = run_calls(p, x, [n], s0=s0)
        with pytest.raises(fo.FirOlsError) as err:
            p.check()
        assert err.value.status == -9
        p.check()   # the word was cleared
        st = p.get_state().cpu().numpy()
    assert np.isnan(y[0, :3 * L].real).all() and np.isnan(y[0, :3 * L].imag).all()
    tail = np.arange(3 * L, n)
    ref = oracle.fir_direct_multi(h, x, s0, idx=tail, threads=THREADS)
    check(y[:, tail], ref, h, x, s0, "partial last block after the timeouts")
    np.testing.assert_array_equal(st[0], oracle.state_next(x[0], s0[0], M))

    with fo.Plan(M, N, 1) as q:
        q.set_freq_response(H)
        y2 = run_calls(q, x, [n], s0=s0)
        q.check()
    idx = np.unique(np.concatenate([np.arange(2000), W.sample_indices(9, n, 3000),
                                    np.arange(n - 2000, n)]))
    ref = oracle.fir_direct_multi(h, x, s0, idx=idx, threads=THREADS)
    check(y2[:, idx], ref, h, x, s0, "plan without the switch")


@pytest.mark.parametrize("M,nchan,nblk", [(3000, 3, 420), (16384, 1, 1300)])
def test_n16384_many_blocks_per_workgroup(M, nchan, nblk):
    """N = 16384 with more blocks than resident workgroups (two per CU), so
    each workgroup runs several blocks and requests the next block's input
    while it finishes the current one: every output against the oracle's
    float64 block overlap-save (H = DFT of the taps), sampled outputs
    against the direct form, the next state bit for bit, and a second run
    bit for bit equal to the first."""
    N = 16384
    L = N - M + 1
    n = nblk * L - 123
    say(f"N=16384 many blocks: M={M} nchan={nchan} blocks/ch={nblk} n={n}")
    rng = np.random.default_rng(M + nblk)
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (nchan, n))
    s0 = W.complex_normal(rng, (nchan, M - 1))
    with fo.Plan(M, N, nchan) as p:
        p.set_taps(h)
        y = run_calls(p, x, [n], s0=s0)
        st = p.get_state().cpu().numpy()
        y2 = run_calls(p, x, [n], s0=s0)
    np.testing.assert_array_equal(y2, y)
    H = np.fft.fft(np.asarray(h, dtype=np.complex128), N)
    for c in range(nchan):
        full = oracle.fir_ols_blocks(H, x[c], s0[c], M)
        check(y[c], full, h, x, s0, f"N=16384 M={M} channel {c} (all {n} outputs, block OLS)")
        np.testing.assert_array_equal(st[c], oracle.state_next(x[c], s0[c], M))
    idx = np.unique(np.concatenate([np.arange(min(n, 2000)), W.sample_indices(M, n, 3000),
                                    np.arange(max(0, n - 2000), n)]))
    ref = oracle.fir_direct_multi(h, x, s0, idx=idx, threads=THREADS)
    check(y[:, idx], ref, h, x, s0, f"N=16384 M={M} (direct form, {idx.size} outputs)")


@pytest.mark.parametrize("M,nchan,nfull", [(65536, 1, 70000), (65000, 2, 33000)])
def test_paired_kernel_more_units_than_one_launch(M, nchan, nfull):
    """More full blocks than one paired launch takes (65536 channel-blocks):
    the call runs as several launches, the later ones starting at a unit
    offset with their own cleared counters and flags.  M = N gives a block
    length of 1, so 70000 samples are 70000 full blocks (every output
    checked, and only the last position of each block is kept); M = 65000
    over two channels puts the launch boundary inside the second channel
    (blocks around it checked in full) and leaves a partial last block."""
    N = 65536
    L = N - M + 1
    n = nfull * L + L // 2
    say(f"paired launches: M={M} nchan={nchan} full blocks={nfull} n={n}")
    rng = np.random.default_rng(M + nchan)
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (nchan, n))
    s0 = W.complex_normal(rng, (nchan, M - 1))
    with fo.Plan(M, N, nchan) as p:
        p.set_taps(h)
        y = run_calls(p, x, [n], s0=s0)
        st = p.get_state().cpu().numpy()
        p.check()
    if n <= 100_000:
        idx = np.arange(n)
    else:
        c_b, i_b = divmod(65536, nfull)               # first unit of the second launch
        assert c_b < nchan
        near = [np.arange(b * L, (b + 1) * L) for b in (i_b - 1, i_b, i_b + 1)]
        idx = np.unique(np.concatenate(near + [np.arange(2000), np.arange(n - 2000, n),
                                               W.sample_indices(M, n, 3000)]))
    ref = oracle.fir_direct_multi(h, x, s0, idx=idx, threads=THREADS)
    check(y[:, idx], ref, h, x, s0, f"M={M} nchan={nchan} nfull={nfull}")
    for c in range(nchan):
        np.testing.assert_array_equal(st[c], oracle.state_next(x[c], s0[c], M))


def test_partial_last_blocks_outnumber_the_slots():
    """N = 65536 with 300 channels of one full and one partial block: the
    300 partial blocks go to the one-workgroup kernel, which holds one
    scratch slot per workgroup (256 on the plan's scratch, 128 on the static
    array), so workgroups take several blocks in turn and reuse their slot.
    The two entry points give the same bits, and sampled outputs (all of
    the partial block for a few channels) match the oracle."""
    import torch
    N, M, nchan = 65536, 16385, 300
    L = N - M + 1
    n = L + 777
    say(f"partial blocks vs slots: N={N} M={M} nchan={nchan} n={n}")
    rng = np.random.default_rng(300)
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (nchan, n))
    s0 = W.complex_normal(rng, (nchan, M - 1))
    xd = to_dev(x)
    outs = []
    for entry in (fo.fir_ols_execute, fo.fir_ols_execute_static):
        yd = torch.zeros_like(xd)
        with fo.Plan(M, N, nchan) as p:
            p.set_taps(h)
            p.set_state(to_dev(s0))
            entry(p.handle, xd.data_ptr(), yd.data_ptr(), n, n, None)
            st = p.get_state().cpu().numpy()
            p.check()
        torch.cuda.synchronize()
        outs.append((yd.cpu().numpy(), st))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
    y, st = outs[0]
    idx = np.unique(np.concatenate([np.arange(300), np.arange(L - 100, n),
                                    W.sample_indices(301, n, 300)]))
    pick = [0, 1, 255, 256, 257, 299]              # around the slot counts
    ref = oracle.fir_direct_multi(h, x[pick], s0[pick], idx=idx, threads=THREADS)
    check(y[pick][:, idx], ref, h, x[pick], s0[pick], "partial blocks vs slots")
    for c in range(nchan):
        np.testing.assert_array_equal(st[c], oracle.state_next(x[c], s0[c], M))


@pytest.mark.parametrize("N,M", [(4096, 1025), (32768, 8193), (65536, 16385), (262144, 65537)])
def test_call_beyond_two_to_the_31_samples(N, M):
    """One channel of 2^31 + 12345 samples (17 GB in and 17 GB out, drawn
    on the device): sample positions, block offsets and output addresses
    pass 2^31, so every index the kernels form from them must be 64-bit.
    Sampled outputs (the first ones, which read the state, the blocks and
    samples around position 2^31, the partial last block, random ones) are
    each checked against the oracle run on their own input window, and the
    carried state against the last M - 1 samples."""
    import torch
    n = (1 << 31) + 12345
    L = N - M + 1
    say(f"beyond 2^31: N={N} M={M} n={n}")
    rng = np.random.default_rng(N + 31)
    h = W.complex_taps(rng, M).astype(np.complex64)
    s0 = W.complex_normal(rng, (1, M - 1))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(N)
    x = torch.randn(n, dtype=torch.complex64, device="cuda", generator=gen)
    y = torch.empty_like(x)
    with fo.Plan(M, N, 1) as p:
        p.set_taps(h)
        p.set_state(to_dev(s0))
        fo.fir_ols_execute(p.handle, x.data_ptr(), y.data_ptr(), n, n, None)
        st = p.get_state().cpu().numpy()
        p.check()
    torch.cuda.synchronize()
    b31 = (1 << 31) // L
    t = np.unique(np.concatenate([
        np.arange(0, 48), np.arange(M - 8, M + 8),
        np.arange(b31 * L - 24, b31 * L + 24), np.arange((1 << 31) - 24, (1 << 31) + 24),
        np.arange(n - L // 2 - 8, n - L // 2 + 8), np.arange(n - 48, n),
        W.sample_indices(N, n, 160)]))
    t = t[(t >= 0) & (t < n)]
    # the stream xt = {S0, x}: output t reads xt[t .. t + M - 1]
    far = t[t >= M - 1]
    win = x[torch.from_numpy(far - (M - 1)).to("cuda")[:, None]
            + torch.arange(M, device="cuda")[None, :]].cpu().numpy()
    got = y[torch.from_numpy(t).to("cuda")].cpu().numpy()
    ref = np.empty(t.size, np.complex128)
    used = []
    xs_head = x[:M].cpu().numpy()
    for k, tk in enumerate(t):
        if tk >= M - 1:
            w = win[np.searchsorted(far, tk)]
        else:
            w = np.concatenate([s0[0, tk:], xs_head[:tk + 1]])
        used.append(w)
        ref[k] = oracle.fir_direct(h, w[M - 1:], w[:M - 1])[0]
    used = np.concatenate(used)[None, :]
    check(got, ref, h, used, None, f"N={N} M={M} beyond 2^31")
    np.testing.assert_array_equal(st[0], x[n - (M - 1):].cpu().numpy())
    del x, y
    torch.cuda.empty_cache()


def test_plans_on_concurrent_streams_equal_their_sequential_runs():
    """Three plans (two at N = 65536, one at N = 32768) each on its own
    stream, their calls enqueued interleaved with no synchronization in
    between, so the kernels can run at the same time and share the CUs:
    each plan's outputs and state are bitwise those of the same calls run
    alone (each plan has its own scratch, queues and flags, and a paired
    consumer only waits on a producer that is already running)."""
    import torch
    specs = [(65536, 16385, 1, 200), (65536, 4097, 2, 150), (32768, 8193, 1, 300)]
    rng = np.random.default_rng(555)
    setups = []
    for N, M, nchan, nblk in specs:
        L = N - M + 1
        n = nblk * L + L // 2
        h = W.complex_taps(rng, M).astype(np.complex64)
        x = to_dev(W.complex_normal(rng, (nchan, n)))
        s0 = to_dev(W.complex_normal(rng, (nchan, M - 1)))
        calls = [n // 3, n // 3, n - 2 * (n // 3)]
        setups.append((N, M, nchan, n, h, x, s0, calls))

    def run_all(concurrent):
        plans, outs, streams = [], [], []
        for N, M, nchan, n, h, x, s0, calls in setups:
            p = fo.Plan(M, N, nchan)
            p.set_taps(h)
            p.set_state(s0)
            plans.append(p)
            outs.append(torch.zeros_like(x))
            streams.append(torch.cuda.Stream())
        torch.cuda.synchronize()
        order = ([(k, j) for j in range(3) for k in range(len(setups))] if concurrent
                 else [(k, j) for k in range(len(setups)) for j in range(3)])
        pos = [0] * len(setups)
        for k, j in order:
            N, M, nchan, n, h, x, s0, calls = setups[k]
            c = calls[j]
            fo.fir_ols_execute(plans[k].handle, x.data_ptr() + 8 * pos[k],
                               outs[k].data_ptr() + 8 * pos[k], c, n, streams[k].cuda_stream)
            pos[k] += c
            if not concurrent:
                streams[k].synchronize()
        res = []
        for k, p in enumerate(plans):
            st = p.get_state(streams[k])
            streams[k].synchronize()
            p.check()
            res.append((outs[k].cpu().numpy(), st.cpu().numpy()))
            p.close()
        return res

    alone = run_all(False)
    together = run_all(True)
    for (ya, sa), (yt, st), spec in zip(alone, together, specs):
        say(f"  concurrent plan {spec}: outputs and state compared")
        np.testing.assert_array_equal(yt, ya)
        np.testing.assert_array_equal(st, sa)
