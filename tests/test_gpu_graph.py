"""fir_ols_execute under HIP graph capture.

execute allocates, synchronizes and clears nothing, so a caller can
capture a run of calls into a graph.  Each replay must equal the same
calls run eagerly (bit for bit: same kernels, same inputs), with the state
carried from replay to replay, and with unrelated eager work and
synchronizations between the replays.
"""
import numpy as np
import pytest

import workloads as W
import order_fir_filtering_amd as fo
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,M,nchan", [(1024, 257, 3), (4096, 1025, 1), (16384, 3000, 2),
                                       (32768, 8193, 1), (65536, 16385, 1), (131072, 40000, 2)])
def test_graph_replays_equal_eager_calls(N, M, nchan):
    import torch
    say(f"graph: N={N} M={M} nchan={nchan}")
    rng = np.random.default_rng(N + M + nchan)
    h = W.complex_taps(rng, M).astype(np.complex64)
    L = N - M + 1
    calls = [2 * L + 5, L - 3]     # an even number of calls: the state parity returns
    n = sum(calls)
    x = to_dev(W.complex_normal(rng, (nchan, n)))
    stream = torch.cuda.Stream()
    reps = 3

    def set_filter(p):
        if N == 65536:
            p.set_freq_response(W.freq_response_input(h, N))
        else:
            p.set_taps(h)

    def run(p, y):
        pos = 0
        for c in calls:
            fo.fir_ols_execute(p.handle, x.data_ptr() + 8 * pos, y.data_ptr() + 8 * pos, c, n,
                               stream.cuda_stream)
            pos += c

    want = []
    with fo.Plan(M, N, nchan) as pe:
        set_filter(pe)
        for _ in range(reps):
            y = torch.zeros_like(x)
            run(pe, y)
            stream.synchronize()
            want.append(y.cpu().numpy())
    assert not np.array_equal(want[0], want[1])    # the carried state matters

    with fo.Plan(M, N, nchan) as pg:
        set_filter(pg)
        yg = torch.zeros_like(x)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run(pg, yg)
        for r in range(reps):
            g.replay()
            torch.cuda.synchronize()
            got = yg.cpu().numpy()
            np.testing.assert_array_equal(got, want[r])
            # unrelated eager work between replays
            yg.copy_(x * 2)
            torch.cuda.synchronize()
        del g


@pytest.mark.parametrize("entry", ["static", "real"])
@pytest.mark.parametrize("N,M", [(4096, 1025), (65536, 16385), (131072, 40000)])
def test_graph_replays_of_static_and_real_entry_points(entry, N, M):
    """The same replay check for fir_ols_execute_static (scratch in the
    library's fixed array, the entry meant for capture) and for
    fir_ols_execute_real (two float rows per channel, real taps)."""
    import torch
    say(f"graph {entry}: N={N} M={M}")
    rng = np.random.default_rng(N + M + (7 if entry == "real" else 0))
    nchan = 2
    L = N - M + 1
    calls = [2 * L + 5, L - 3]
    n = sum(calls)
    if entry == "real":
        h = (rng.standard_normal(M) / np.sqrt(M)).astype(np.float32)
        x = to_dev(rng.standard_normal((2 * nchan, n)).astype(np.float32))
        fn, item = fo.fir_ols_execute_real, 4
    else:
        h = W.complex_taps(rng, M).astype(np.complex64)
        x = to_dev(W.complex_normal(rng, (nchan, n)))
        fn, item = fo.fir_ols_execute_static, 8
    stream = torch.cuda.Stream()
    reps = 3

    def run(p, y):
        pos = 0
        for c in calls:
            fn(p.handle, x.data_ptr() + item * pos, y.data_ptr() + item * pos, c, n,
               stream.cuda_stream)
            pos += c

    want = []
    with fo.Plan(M, N, nchan) as pe:
        pe.set_taps(h)
        for _ in range(reps):
            y = torch.zeros_like(x)
            run(pe, y)
            stream.synchronize()
            want.append(y.cpu().numpy())
    assert not np.array_equal(want[0], want[1])

    with fo.Plan(M, N, nchan) as pg:
        pg.set_taps(h)
        yg = torch.zeros_like(x)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run(pg, yg)
        for r in range(reps):
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(yg.cpu().numpy(), want[r])
            yg.copy_(x * 2)
            torch.cuda.synchronize()
        del g
