"""Build libfirols.so (HIP, gfx950) in-tree with hipcc.

Every source compiles to its own object (in parallel, under _build/), and
one hipcc link makes the shared library; build() always recompiles."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfirols.so")
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = ["plan.cpp", "host_stream.cpp", "ols_fused.hip", "ols_mid.hip", "ols_big.hip", "ols_split.hip",
           "ols_pair.hip", "ols_multi.hip", "pfb_plan.cpp", "pfb.hip", "static_scratch.hip"]
ARCH = "gfx950"

COMPILE_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _filter(text: str) -> str:
    return "\n".join(l for l in text.splitlines()
                     if "is not a recognized feature for this target" not in l)


def _compile(hipcc: str, src: str) -> tuple[str, int, str]:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = ([hipcc] + COMPILE_FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                      "-c", os.path.join(CSRC, src), "-o", obj])
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return obj, res.returncode, _filter(res.stdout)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source and link libfirols.so; returns the library path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s), SOURCES))
    failed = [(o, out) for o, rc, out in results if rc != 0]
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(out for _, out in failed))
    if verbose:
        for _, _, out in results:
            if out.strip():
                print(out, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + [o for o, _, _ in results] + [
        "-o", tmp]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc link failed:\n" + _filter(res.stdout))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
