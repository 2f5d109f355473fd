"""fir_ols_execute_static (the call that allocates nothing) against
fir_ols_execute: the same plan shape, the same inputs, two calls in a row
(the second smaller), bit-for-bit equal outputs and states, and the first
call's outputs against the float64 oracle on sampled indices."""
import os

import numpy as np
import pytest

import oracle
import order_fir_filtering_amd as fo
import workloads as W
from gpu_util import check, say, to_dev

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


def _run(plan, fn, x2d, calls, s0):
    import torch
    xd = to_dev(x2d)
    yd = torch.zeros_like(xd)
    plan.set_state(to_dev(s0))
    n = x2d.shape[1]
    pos = 0
    for c in calls:
        fn(plan.handle, xd.data_ptr() + 8 * pos, yd.data_ptr() + 8 * pos, c, n, None)
        pos += c
    torch.cuda.synchronize()
    return yd.cpu().numpy(), plan.get_state().cpu().numpy()


# (N, M, nchan, first call, second call): the split path (N = 65536: at most
# 128 workgroups on the array), the multi-pass path (N = 2^17 and 2^20, the
# latter spanning several batches of the array), and a fused-path plan
# (no scratch)
CASES = [
    (65536, 16385, 1, 300 * 49152 + 1234, 49152 * 3 + 7),
    (65536, 20000, 2, 200000, 65536),
    (131072, 40000, 2, 700000, 150000),
    (1048576, 262145, 1, 20 * 786432 + 5, 786432 * 9 + 1),
    (4096, 1025, 3, 100000, 30000),
]


@pytest.mark.parametrize("N,M,nchan,n1,n2", CASES)
def test_static_scratch_matches_execute(N, M, nchan, n1, n2):
    say(f"execute_static: N={N} M={M} nchan={nchan} calls={n1},{n2}")
    rng = np.random.default_rng(N + M + nchan)
    h = W.complex_taps(rng, M).astype(np.complex64)
    x = W.complex_normal(rng, (nchan, n1 + n2))
    s0 = W.complex_normal(rng, (nchan, M - 1))
    H = W.freq_response_input(h, N)
    with fo.Plan(M, N, nchan) as pa, fo.Plan(M, N, nchan) as pb:
        pa.set_freq_response(H)
        pb.set_freq_response(H)
        ya, sa = _run(pa, fo.fir_ols_execute, x, [n1, n2], s0)
        yb, sb = _run(pb, fo.fir_ols_execute_static, x, [n1, n2], s0)
    np.testing.assert_array_equal(yb, ya)
    np.testing.assert_array_equal(sb, sa)
    for c in range(nchan):
        np.testing.assert_array_equal(sb[c], oracle.state_next(x[c], s0[c], M))
    idx = np.unique(np.concatenate([np.arange(min(n1, 2000)), np.arange(n1 - 2000, n1 + 2000),
                                    np.arange(n1 + n2 - 2000, n1 + n2),
                                    W.sample_indices(N + 1, n1 + n2, 3000)]))
    ref = oracle.fir_direct_multi(h, x, s0, idx=idx, threads=THREADS)
    check(yb[:, idx], ref, h, x, s0, f"static N={N} M={M}")


def test_static_scratch_size_and_errors():
    import torch
    say("execute_static: size and argument checks")
    assert fo.fir_ols_static_scratch_bytes() == 64 << 20
    x = torch.zeros(100, dtype=torch.complex64, device="cuda:0")
    with fo.Plan(16385, 65536) as p:
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_static(p.handle, x, x, 100, 100)
        assert e.value.status == -3                       # no filter yet
        p.set_freq_response(np.ones(65536, np.complex64))
        with pytest.raises(fo.FirOlsError) as e:
            fo.fir_ols_execute_static(p.handle, x, x, 100, 100)
        assert e.value.status == -4                       # in place
        fo.fir_ols_execute_static(p.handle, x, x, 0, 0)   # zero samples: no-op
