"""Seeded synthetic workloads for overlap-save FIR filtering.

This module only draws numbers: filter taps, complex input streams and
initial states, for the five workload shapes below and for the small
random cases the tests use.  It contains none of the filtering arithmetic,
so both the float64 oracle and the GPU library can take their inputs from
here without sharing any code with each other.

Conventions
-----------
* Complex N(0,1) streams: the real parts are the first ``count`` draws of a
  float32 standard normal, the imaginary parts the next ``count`` draws.
* Windowed-sinc taps follow the window method of the polyphase-channelizer
  page ("GPU polyphase filter bank channelizer", section 2.2): a Hamming
  window and a cutoff given relative to Nyquist (fs = 2), scaled to unit
  DC gain.  Designed in float64, rounded to float32; the float32 taps are
  the filter both sides use.
* The frequency-response workload gives H as the N-point DFT of a random
  complex M-tap h, computed in float64 with numpy and rounded to
  complex64.  That DFT only builds the input; the library receives H.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

BASE_SEED = 20261202


@dataclasses.dataclass(frozen=True)
class Workload:
    """One filtering workload: filter length M, FFT size N, channels, calls."""

    key: str
    M: int
    N: int
    nchan: int
    samples: int                 # samples per channel over all calls
    calls: tuple                 # per-call sample counts (sum == samples)
    taps: str                    # "hamming_sinc" | "uniform" | "complex_H"
    state: str                   # "zero" | "random"
    description: str

    @property
    def L(self) -> int:
        return self.N - self.M + 1

    @property
    def seed(self) -> int:
        return BASE_SEED + int(self.key[-1])


WORKLOADS = {
    "cfg1": Workload(
        "cfg1", 65, 256, 1, 64 * 192, (64 * 192,), "hamming_sinc", "zero",
        "M=65 Hamming windowed-sinc (cutoff 0.25 of Nyquist), N=256, L=192, "
        "64 blocks, one call, zero state"),
    "cfg2": Workload(
        "cfg2", 1025, 4096, 1, 1024 * 3072, (256 * 3072,) * 4, "hamming_sinc",
        "zero",
        "M=1025 windowed-sinc, N=4096, L=3072, 1024 blocks fed as 4 calls "
        "of 786432 samples carrying the state between calls"),
    "cfg3": Workload(
        "cfg3", 8193, 32768, 1, 2048 * 24576, (2048 * 24576,), "uniform",
        "zero",
        "M=8193 taps uniform[-1,1]/M, N=32768, L=24576, 2048 blocks, one call"),
    "cfg4": Workload(
        "cfg4", 16385, 65536, 1, 5120 * 49152, (5120 * 49152,), "complex_H",
        "zero",
        "H given directly: 65536-point DFT of a random complex 16385-tap h, "
        "L=49152, 5120 blocks, one call"),
    "cfg5": Workload(
        "cfg5", 257, 1024, 1024, 65536, (65536,), "hamming_sinc", "random",
        "1024 channels x 65536 samples, each with its own random state, "
        "shared M=257 windowed-sinc filter, N=1024, L=768, one call"),
}


def rngs(seed: int, n: int = 3) -> List[np.random.Generator]:
    """Independent generators spawned from one seed (taps, input, state)."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def complex_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """complex64 array whose re/im parts are i.i.d. float32 N(0,1)."""
    shape = (shape,) if np.isscalar(shape) else tuple(shape)
    count = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(count, dtype=np.complex64)
    pair = out.view(np.float32).reshape(count, 2)
    pair[:, 0] = rng.standard_normal(count, dtype=np.float32)
    pair[:, 1] = rng.standard_normal(count, dtype=np.float32)
    return out.reshape(shape)


def hamming_sinc(M: int, cutoff: float = 0.25) -> np.ndarray:
    """Hamming-windowed sinc low-pass, cutoff relative to Nyquist, sum = 1.

    Designed in float64 and returned rounded to float32.
    """
    if M == 1:
        return np.ones(1, dtype=np.float32)
    n = np.arange(M, dtype=np.float64)
    alpha = 0.5 * (M - 1)
    proto = cutoff * np.sinc(cutoff * (n - alpha))
    window = 0.54 - 0.46 * np.cos(2.0 * np.pi * n / (M - 1))
    h = proto * window
    h /= h.sum()
    return h.astype(np.float32)


def uniform_taps(rng: np.random.Generator, M: int) -> np.ndarray:
    """float32 taps i.i.d. uniform[-1, 1] scaled by 1/M."""
    return (rng.uniform(-1.0, 1.0, M) / M).astype(np.float32)


def complex_taps(rng: np.random.Generator, M: int) -> np.ndarray:
    """complex128 taps (N(0,1) + j N(0,1)) / sqrt(M), kept in float64."""
    re = rng.standard_normal(M)
    im = rng.standard_normal(M)
    return (re + 1j * im) / np.sqrt(M)


def freq_response_input(h: np.ndarray, N: int) -> np.ndarray:
    """complex64 H = N-point DFT (float64, numpy) of the zero-padded taps.

    Builds the input of the frequency-response entry point; bin 0 first,
    forward kernel exp(-2 pi j q m / N).
    """
    return np.fft.fft(np.asarray(h, dtype=np.complex128), N).astype(np.complex64)


@dataclasses.dataclass
class Inputs:
    workload: Workload
    taps: Optional[np.ndarray]        # float32 real taps, or None
    h_ref: np.ndarray                 # taps the oracle uses (float32 or complex128)
    H: Optional[np.ndarray]           # complex64 frequency response, or None
    x: np.ndarray                     # complex64 [nchan, samples]
    s0: np.ndarray                    # complex64 [nchan, M-1]


def make_inputs(key: str, samples: Optional[int] = None) -> Inputs:
    """Inputs of a named workload; ``samples`` truncates the stream length."""
    w = WORKLOADS[key]
    g_taps, g_x, g_s0 = rngs(w.seed)
    H = None
    taps = None
    if w.taps == "hamming_sinc":
        taps = hamming_sinc(w.M)
        h_ref = taps
    elif w.taps == "uniform":
        taps = uniform_taps(g_taps, w.M)
        h_ref = taps
    elif w.taps == "complex_H":
        h_ref = complex_taps(g_taps, w.M)
        H = freq_response_input(h_ref, w.N)
    else:
        raise ValueError(w.taps)
    n = w.samples if samples is None else int(samples)
    x = complex_normal(g_x, (w.nchan, n))
    if w.state == "random":
        s0 = complex_normal(g_s0, (w.nchan, w.M - 1))
    else:
        s0 = np.zeros((w.nchan, w.M - 1), dtype=np.complex64)
    return Inputs(w, taps, h_ref, H, x, s0)


def sample_indices(seed: int, total: int, count: int) -> np.ndarray:
    """Sorted distinct random output indices in [0, total)."""
    rng = np.random.default_rng(seed)
    count = min(count, total)
    return np.sort(rng.choice(total, size=count, replace=False)).astype(np.int64)


# Channelizer workloads (the polyphase-channelizer page, "GPU polyphase
# filter bank channelizer": section 2.2's 50 % overlap, D = K / 2, for its
# 1024- and 128-channel configurations).  The prototype is the page's
# window-method low-pass, cutoff 1/D of Nyquist with a Hamming window, here
# 8 taps per branch; the input is complex N(0,1), 2^26 samples (the page's
# 40 ms at 6.5536 MHz is 2^18 samples; 256 times that fills the GPU).
PFB_WORKLOADS = {
    "pfb1024": dict(K=1024, D=512, Nh=8192, samples=1 << 26,
                    description="K=1024 channels, D=512 (50% overlap), Nh=8192 Hamming "
                                "windowed-sinc taps (cutoff 1/D of Nyquist), 2^26 samples"),
    "pfb128": dict(K=128, D=64, Nh=1024, samples=1 << 26,
                   description="K=128 channels, D=64 (50% overlap), Nh=1024 Hamming "
                               "windowed-sinc taps (cutoff 1/D of Nyquist), 2^26 samples"),
}


def make_pfb_inputs(key: str, samples: Optional[int] = None):
    """(taps float32 [Nh], x complex64 [samples]) of a channelizer workload."""
    w = PFB_WORKLOADS[key]
    h = hamming_sinc(w["Nh"], 1.0 / w["D"])
    _, g_x, _ = rngs(BASE_SEED + 1000 + w["K"])
    n = w["samples"] if samples is None else int(samples)
    return h, complex_normal(g_x, n)
