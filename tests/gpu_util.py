"""Helpers shared by the GPU tests (imported only by tests marked gpu)."""
import sys

import numpy as np

import oracle
import order_fir_filtering_amd as fo

REL_RMS_ALARM = 1e-5


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def run_calls(plan: "fo.Plan", x2d: np.ndarray, calls, s0=None):
    """Feed x2d [nchan, n] as consecutive calls; returns y [nchan, n] (numpy)."""
    import torch
    xd = to_dev(x2d)
    yd = torch.zeros_like(xd)
    if s0 is not None:
        plan.set_state(to_dev(s0))
    n = x2d.shape[1]
    pos = 0
    item = xd.element_size()
    for c in calls:
        fo.fir_ols_execute(plan.handle, xd.data_ptr() + pos * item, yd.data_ptr() + pos * item,
                           c, n, None)
        pos += c
    assert pos == n
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def check(y, ref, h, x_used, s0_used, what=""):
    """Parity gate: max|y - ref| <= 1e-5 max|xt| sum|h|, plus a rel-RMS alarm."""
    y = np.asarray(y).ravel()
    ref = np.asarray(ref).ravel()
    assert y.shape == ref.shape
    bound = oracle.parity_bound(h, x_used, s0_used)
    if y.size == 0:
        return 0.0
    err = float(np.abs(y.astype(np.complex128) - ref).max())
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(y - ref) / nref) if nref > 0 else err
    say(f"  {what}: max err {err:.3e} bound {bound:.3e} rel-rms {rel:.2e}")
    assert err <= bound, f"{what}: max error {err} above bound {bound}"
    if nref > 0:
        assert rel < REL_RMS_ALARM, f"{what}: relative RMS error {rel}"
    return err
