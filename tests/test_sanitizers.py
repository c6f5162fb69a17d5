"""Host AddressSanitizer + UndefinedBehaviorSanitizer builds (CPU only).

* The oracle (oracle/oracle.c) with a driver that calls every function it
  declares on small inputs of every dtype (tests/sanitize/oracle_driver.c),
  built with gcc.
* libmoe's host code (the C ABI's validation, workspace sizing and error
  paths, tests/sanitize/abi_driver.cpp) built with hipcc, the sanitizers on
  the host code only; no call in the driver reaches a kernel launch, so no
  device is needed.
A sanitizer finding aborts the driver (no recovery), failing the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fno-fast-math", "-pthread",
          "-I", os.path.join(ROOT, "oracle"), "-o", exe, os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    r = _run([exe], env=ENV)
    assert "oracle sanitizer driver ok" in r.stdout


def test_abi_validation_under_sanitizers(tmp_path):
    from group_limited_top_amd import build
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    csrc = os.path.join(ROOT, "group_limited_top_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    exe = str(tmp_path / "abi_driver")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    _run([hipcc, f"--offload-arch={build.ARCH}", "-O1", "-g", "-fno-omit-frame-pointer", *san,
          "-std=c++17", "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", csrc, *srcs,
          "-x", "hip", os.path.join(SAN, "abi_driver.cpp"), "-o", exe])
    r = _run([exe], env=ENV)
    assert "abi sanitizer driver ok" in r.stdout
