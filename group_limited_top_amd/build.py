"""Build libmoe.so (HIP, gfx950 only) in the package directory.

    python -m group_limited_top_amd.build

Flags: -ffp-contract=off keeps the router's specified fp32/fp64 arithmetic
(sigma32, selection, weight normalisation) free of fused multiply-adds the
source did not write; -packed-fp32-ops is disabled for every HIP source.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SO = os.path.join(PKG, "libmoe.so")
PROBE_SO = os.path.join(PKG, "libmoe_probe.so")  # measurement kernels (bench.py only)
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


def command(out: str = SO, srcs: list[str] | None = None) -> list[str]:
    if srcs is None:
        srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC, *srcs, "-o", out,
    ]


def _compile(out: str, srcs: list[str] | None, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = command(tmp, srcs)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{os.path.basename(out)} build failed:\n{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Builds libmoe.so and the measurement library libmoe_probe.so."""
    _compile(PROBE_SO, [os.path.join(PKG, "probe", "probe.hip")], verbose)
    return _compile(SO, None, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
