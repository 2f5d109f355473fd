"""Measure the filtering rate of every supported block size N on this GPU.

For each N = 2^8 .. 2^20 the script times one long single-channel call with
M = N/4 + 1 (so L = 3N/4) and many blocks, and records blocks per second.
A block's cost depends on N, not on M (the transform is the same; only the
number of kept outputs changes), so the output rate of a plan (M, N) is
about (N - M + 1) x blocks_per_second(N): the planner choice of N for a
given M (the method page leaves N free, claim 1 step 1) maximizes that.

    python -m order_fir_filtering_amd.tune_n [--out FILE] [--logn LO HI]

prints one JSON object {N: blocks_per_second} (and writes it to FILE).
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np


def sweep(max_samples: int = 1 << 27, lo: int = 8, hi: int = 20) -> dict:
    import torch

    import order_fir_filtering_amd as fo
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(11)
    res = {}
    for logn in range(lo, hi + 1):
        N = 1 << logn
        M = N // 4 + 1
        L = N - M + 1
        # enough blocks to fill the GPU: one block per workgroup up to
        # N = 65536, while a larger block spreads over many workgroups
        nblk = max(1024 if logn <= 16 else 64, min(max_samples // L, 1 << 20))
        n = nblk * L
        x = torch.randn(n, dtype=torch.complex64, device=dev)
        y = torch.empty_like(x)
        h = (rng.standard_normal(M) / np.sqrt(M)).astype(np.float32)
        with fo.Plan(M, N, 1) as p:
            p.set_taps(h)
            for _ in range(3):
                p.execute(x, y)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record()
            for _ in range(reps):
                p.execute(x, y)
            e1.record()
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) / reps * 1e-3
        res[N] = nblk / sec
        print(f"N={N:6d} M={M:6d} blocks={nblk:8d}: {nblk / sec:.4g} blocks/s, "
              f"{n / sec / 1e6:.1f} Msamples/s", file=sys.stderr, flush=True)
        del x, y
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default="")
    ap.add_argument("--logn", type=int, nargs=2, default=(8, 20), metavar=("LO", "HI"),
                    help="sweep N = 2^LO .. 2^HI only")
    a = ap.parse_args()
    res = sweep(lo=a.logn[0], hi=a.logn[1])
    text = json.dumps({str(k): round(v, 1) for k, v in res.items()})
    print(text)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
