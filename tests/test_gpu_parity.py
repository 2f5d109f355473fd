"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Method page ("一种基于GPU的高阶数字FIR滤波器频域并行处理实现方法", claim 1):
the kept points of every block are the linear convolution of the taps with
the stream {S0, X}; the oracle is that sum.  Gate on every case:
max|y - y_ref| <= 1e-5 * max|xt| * sum|h| (complex64 against float64),
with a relative-RMS alarm at 1e-5.
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


def oracle_multi(h, x2d, s02d, idx=None):
    return oracle.fir_direct_multi(h, x2d, s02d, idx=idx, threads=THREADS)


def test_cfg1_full():
    inp = W.make_inputs("cfg1")
    w = inp.workload
    say(f"cfg1: M={w.M} N={w.N} n={w.samples}")
    with fo.Plan(w.M, w.N) as p:
        p.set_taps(inp.taps)
        y = run_calls(p, inp.x, w.calls)
    ref = oracle_multi(inp.h_ref, inp.x, inp.s0)
    check(y, ref, inp.h_ref, inp.x, inp.s0, "cfg1")


def test_cfg2_four_calls_with_state_full():
    inp = W.make_inputs("cfg2")
    w = inp.workload
    say(f"cfg2: M={w.M} N={w.N} calls={w.calls}")
    with fo.Plan(w.M, w.N) as p:
        p.set_taps(inp.taps)
        y = run_calls(p, inp.x, w.calls)
        st = p.get_state().cpu().numpy()
    ref = oracle_multi(inp.h_ref, inp.x, inp.s0)
    check(y, ref, inp.h_ref, inp.x, inp.s0, "cfg2")
    np.testing.assert_array_equal(st[0], oracle.state_next(inp.x[0], inp.s0[0], w.M))


def test_cfg5_batched_channels_full():
    """Every output of all 1024 channels and every channel's next state
    (claim 1, step 3: each stream carries its own S0)."""
    inp = W.make_inputs("cfg5")
    w = inp.workload
    say(f"cfg5: M={w.M} N={w.N} nchan={w.nchan} n={w.samples}")
    with fo.Plan(w.M, w.N, w.nchan) as p:
        p.set_taps(inp.taps)
        y = run_calls(p, inp.x, w.calls, s0=inp.s0)
        st = p.get_state().cpu().numpy()
    ref = oracle_multi(inp.h_ref, inp.x, inp.s0)
    check(y, ref, inp.h_ref, inp.x, inp.s0, "cfg5 all channels, all outputs")
    for c in range(w.nchan):
        np.testing.assert_array_equal(st[c], oracle.state_next(inp.x[c], inp.s0[c], w.M))


def _sweep_cases():
    rng = np.random.default_rng(2026)
    cases = []
    for logn in range(3, 15):
        N = 1 << logn
        for M in sorted({1, 2, N // 3 + 1, N - 1, N}):
            if M < 1 or M > N:
                continue
            L = N - M + 1
            n = int(rng.choice([1, max(M - 2, 1), L - 1 if L > 1 else 1, L, L + 1,
                                3 * L + int(rng.integers(0, L)), 5 * L]))
            n = max(1, min(n, 200000))
            nchan = int(rng.choice([1, 1, 3]))
            complex_taps = bool(rng.integers(0, 2))
            cases.append((N, M, n, nchan, complex_taps, int(rng.integers(0, 1 << 30))))
    return cases


@pytest.mark.parametrize("N,M,n,nchan,complex_taps,seed", _sweep_cases())
def test_random_sizes(N, M, n, nchan, complex_taps, seed):
    say(f"sweep: N={N} M={M} n={n} nchan={nchan} complex={complex_taps} seed={seed}")
    rng = np.random.default_rng(seed)
    h = rng.standard_normal(M).astype(np.float32)
    if complex_taps:
        h = (h + 1j * rng.standard_normal(M)).astype(np.complex64)
    x = W.complex_normal(rng, (nchan, n))
    s0 = W.complex_normal(rng, (nchan, M - 1))
    with fo.Plan(M, N, nchan) as p:
        p.set_taps(h)
        y = run_calls(p, x, [n], s0=s0)
    ref = oracle_multi(h, x, s0)
    check(y, ref, h, x, s0, f"N={N} M={M}")


@pytest.mark.parametrize("N,M", [(256, 65), (1024, 257), (4096, 1025), (64, 64), (16384, 3000)])
def test_streaming_chunks_equal_one_shot(N, M):
    say(f"stream chunks: N={N} M={M}")
    rng = np.random.default_rng(N + M)
    h = rng.standard_normal(M).astype(np.float32)
    L = N - M + 1
    chunks = [1, max(M - 2, 1), L, 3, L + 7, 2 * L - 1, 1, 5 * L]
    n = sum(chunks)
    x = W.complex_normal(rng, (2, n))
    s0 = W.complex_normal(rng, (2, M - 1))
    with fo.Plan(M, N, 2) as p:
        p.set_taps(h)
        y = run_calls(p, x, chunks, s0=s0)
        st = p.get_state().cpu().numpy()
    ref = oracle_multi(h, x, s0)
    check(y, ref, h, x, s0, "chunked")
    for c in range(2):
        np.testing.assert_array_equal(st[c], oracle.state_next(x[c], s0[c], M))


def test_checkpoint_resume_in_new_plan_is_bitwise():
    say("checkpoint/resume")
    import torch
    M, N = 257, 1024
    rng = np.random.default_rng(5)
    h = W.hamming_sinc(M)
    x = W.complex_normal(rng, (3, 5000))
    s0 = W.complex_normal(rng, (3, M - 1))
    with fo.Plan(M, N, 3) as p:
        p.set_taps(h)
        y_all = run_calls(p, x, [2000, 3000], s0=s0)
    with fo.Plan(M, N, 3) as p1:
        p1.set_taps(h)
        y1 = run_calls(p1, x[:, :2000], [2000], s0=s0)
        saved = p1.get_state()
    with fo.Plan(M, N, 3) as p2:
        p2.set_taps(h)
        p2.set_state(saved)
        y2 = run_calls(p2, x[:, 2000:], [3000])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y_all)


@pytest.mark.parametrize("N,M", [(64, 17), (4096, 1025), (16384, 100)])
def test_unit_response_is_identity(N, M):
    say(f"H=1: N={N} M={M}")
    rng = np.random.default_rng(N)
    x = W.complex_normal(rng, (1, 3 * N))
    s0 = W.complex_normal(rng, (1, M - 1))
    with fo.Plan(M, N) as p:
        p.set_freq_response(np.ones(N, np.complex64))
        y = run_calls(p, x, [x.shape[1]], s0=s0)
    check(y, x.astype(np.complex128), np.ones(1), x, s0, "identity")


@pytest.mark.parametrize("N,M,d", [(256, 65, 64), (256, 65, 1), (4096, 1025, 1024), (4096, 1025, 333)])
def test_delay_response(N, M, d):
    say(f"delay: N={N} M={M} d={d}")
    rng = np.random.default_rng(d)
    x = W.complex_normal(rng, (1, 4 * N))
    s0 = W.complex_normal(rng, (1, M - 1))
    H = np.exp(-2j * np.pi * np.arange(N) * d / N).astype(np.complex64)
    with fo.Plan(M, N) as p:
        p.set_freq_response(H)
        y = run_calls(p, x, [x.shape[1]], s0=s0)
    xt = np.concatenate([s0[0], x[0]])
    want = xt[M - 1 - d: M - 1 - d + x.shape[1]]
    check(y, want.astype(np.complex128), np.ones(1), x, s0, "delay")


@pytest.mark.parametrize("N,M", [(1024, 257), (8192, 3001)])
def test_taps_and_freq_response_entries_agree(N, M):
    say(f"taps vs H: N={N} M={M}")
    rng = np.random.default_rng(M)
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (1, 3 * N + 11))
    with fo.Plan(M, N) as pa, fo.Plan(M, N) as pb:
        pa.set_taps(h)
        pb.set_freq_response(W.freq_response_input(h, N))
        ya = run_calls(pa, x, [x.shape[1]])
        yb = run_calls(pb, x, [x.shape[1]])
    ref = oracle_multi(h, x, None)
    check(ya, ref, h, x, None, "set_taps")
    check(yb, ref, h, x, None, "set_freq_response")


@pytest.mark.parametrize("N,M", [(64, 9), (512, 100), (16, 16)])
def test_arbitrary_response_matches_block_oracle(N, M):
    say(f"arbitrary H: N={N} M={M}")
    rng = np.random.default_rng(N * M)
    H = W.complex_normal(rng, N)
    x = W.complex_normal(rng, (1, 7 * N + 3))
    s0 = W.complex_normal(rng, (1, M - 1))
    with fo.Plan(M, N) as p:
        p.set_freq_response(H)
        y = run_calls(p, x, [x.shape[1]], s0=s0)
    ref = oracle.fir_ols_blocks(H, x[0], s0[0], M)
    g = np.fft.ifft(H.astype(np.complex128))
    check(y, ref, g, x, s0, "arbitrary H")


def test_repeat_runs_are_bitwise_identical():
    say("determinism")
    inp = W.make_inputs("cfg2", samples=400000)
    w = inp.workload
    outs = []
    for _ in range(2):
        with fo.Plan(w.M, w.N) as p:
            p.set_taps(inp.taps)
            outs.append(run_calls(p, inp.x, [100000, 300000]))
    np.testing.assert_array_equal(outs[0], outs[1])


def test_error_paths_leave_state_unchanged():
    say("error paths")
    import torch
    M, N = 33, 128
    rng = np.random.default_rng(9)
    x = to_dev(W.complex_normal(rng, (1, 1000)))
    y = torch.empty_like(x)
    s0 = to_dev(W.complex_normal(rng, (1, M - 1)))
    with fo.Plan(M, N) as p:
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute(p.handle, x, y, 1000, 1000)
        assert e.value.status == -3                      # no filter yet
        p.set_taps(np.ones(M, np.float32))
        p.set_state(s0)
        before = p.get_state().cpu().numpy()
        for args, status in [
            ((x, x, 1000, 1000), -4),                     # in place
            ((x, x.data_ptr() + 8 * 500, 1000, 1000), -4),  # overlapping ranges
            ((x.data_ptr() + 4, y, 999, 999), -5),        # misaligned
            ((x, y, 1000, 999), -1),                      # stride < n
            ((x, y, -1, 1000), -1),                       # negative count
            ((None, y, 10, 10), -1),                      # null pointer
        ]:
            with pytest.raises(fo.FirOlsError) as e:
                fo.fir_ols_execute(p.handle, *args)
            assert e.value.status == status, args
        fo.fir_ols_execute(p.handle, x, y, 0, 0)          # zero samples: no-op
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_set_taps(p.handle, np.ones(M + 1, np.float32))
        assert e.value.status == -1
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_set_freq_response(p.handle, np.ones(N // 2, np.complex64))
        assert e.value.status == -1
        after = p.get_state().cpu().numpy()
    np.testing.assert_array_equal(before, after)


def test_set_state_none_zeroes_and_m1_has_no_state():
    say("state reset / M=1")
    rng = np.random.default_rng(10)
    with fo.Plan(9, 64, 2) as p:
        p.set_taps(np.ones(9, np.float32))
        p.set_state(to_dev(W.complex_normal(rng, (2, 8))))
        p.set_state(None)
        assert not p.get_state().cpu().numpy().any()
    x = W.complex_normal(rng, (1, 100))
    with fo.Plan(1, 16) as p:
        p.set_taps(np.array([2.0], np.float32))
        y = run_calls(p, x, [40, 60])
    check(y, 2.0 * x.astype(np.complex128), np.array([2.0]), x, None, "M=1")


def _many_block_cases():
    # (N, threads per block TB, blocks per channel, channels): enough blocks
    # that every resident workgroup takes several, with L = N - M + 1 a
    # multiple s*TB of the threads per block, so that the overlap of a block
    # ends on each possible register row boundary
    cases = []
    for N, TB, nb, nchan in ((1024, 64, 131, 47), (2048, 128, 97, 31), (4096, 256, 211, 9)):
        P = N // TB
        for s in sorted({1, 2, P // 4, P // 2 + 1, 3 * P // 4, P - 1}):
            cases.append((N, N - s * TB + 1, nb, nchan))
    return cases


@pytest.mark.parametrize("N,M,nb,nchan", _many_block_cases())
def test_many_blocks_block_length_on_row_boundaries(N, M, nb, nchan):
    """Many blocks per workgroup, each block's overlap (claim 1, step 3:
    D_(i-1) in front of B_i) ending on every register row boundary: every
    output and state against the oracle, over ragged channel lengths and
    two calls."""
    L = N - M + 1
    n = nb * L - 17
    say(f"row boundaries: N={N} M={M} L={L} blocks/ch={nb} nchan={nchan}")
    rng = np.random.default_rng(N + M)
    h = rng.standard_normal(M).astype(np.float32) / np.sqrt(M)
    x = W.complex_normal(rng, (nchan, n))
    s0 = W.complex_normal(rng, (nchan, M - 1))
    calls = [n // 3 * 2 + 5, n - (n // 3 * 2 + 5)]
    with fo.Plan(M, N, nchan) as p:
        p.set_taps(h)
        y = run_calls(p, x, calls, s0=s0)
        st = p.get_state().cpu().numpy()
    ref = oracle_multi(h, x, s0)
    check(y, ref, h, x, s0, f"rows N={N} M={M}")
    for c in range(nchan):
        np.testing.assert_array_equal(st[c], oracle.state_next(x[c], s0[c], M))
