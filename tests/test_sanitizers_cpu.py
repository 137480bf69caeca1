"""Host AddressSanitizer and UndefinedBehaviorSanitizer runs (no GPU needed):

* the oracle (plain C) driven through every entry point on small and edge-case inputs,
  serially and with OpenMP threads, each buffer allocated at exactly its contract size;
* the library's host code (the C ABI's argument checks, plans and workspace sizes),
  built with the sanitizers on the host side only (device code is built as usual and
  never launched), driven with rejected and accepted arguments.

The drivers are tests/sanitize/*.c; each exits non-zero on a failed expectation, and
the sanitizers abort on the first report."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("openmp", [False, True])
def test_oracle_under_sanitizers(tmp_path, openmp):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", *(["-fopenmp"] if openmp else []), *SAN,
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "i8gs_oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env={**os.environ, "OMP_NUM_THREADS": "4"})
    assert "ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not available")
@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host-only check: accepted calls would reach a GPU here")
def test_abi_host_code_under_sanitizers(tmp_path):
    objs = []
    procs = []
    for src in sorted(glob.glob(os.path.join(ROOT, "int8_group_scaled_amd", "csrc", "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        # sanitizers on the host side only: each -fsanitize= right after -Xarch_host
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-g", "-fPIC", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "int8_group_scaled_amd", "csrc"),
               "-c", src, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for cmd, p in procs:
        out, err = p.communicate(timeout=900)
        assert p.returncode == 0, f"{cmd[-3]}:\n{err[-3000:]}"
    drv = str(tmp_path / "driver.o")
    _run([CLANG, "-std=c11", "-O1", "-g", *SAN, "-I" + os.path.join(ROOT, "include"), "-c",
          os.path.join(HERE, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run([CLANG + "++", *SAN, *objs, drv, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # the HIP runtime's own allocations at exit are not this library's: leak checks off
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert "ok" in r.stdout
