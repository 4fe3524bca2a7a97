"""AddressSanitizer build of the host code (no GPU): the format converters
(formats_host.cpp) and the C ABI's argument validation (the host part of
api.hip, exercised through dry-run mode), linked with tests/asan/
host_driver.cpp, whose launcher stubs abort if a dry run ever reaches one.
The driver runs every converter over every BF16 pattern times a range of
powers of two and calls every device entry point with valid and invalid
arguments; a sanitizer report or a failed expectation fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mx_scaled_fp8_amd", "csrc")
INC = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/bin/amdclang++"          # the compiler hipcc drives: one sanitizer runtime for all objects

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="needs the ROCm compilers")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_host_code_under_address_sanitizer(tmp_path):
    san = ["-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-O1", "-fPIC"]
    # api.hip with the sanitizer on its host compile only (its device part,
    # the scratch array of mx_linear_noalloc, is built as usual)
    api = str(tmp_path / "api.o")
    _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", f"-I{INC}", f"-I{CSRC}",
          *[a for f in san for a in ("-Xarch_host", f)], "-c", os.path.join(CSRC, "api.hip"), "-o", api])
    fmt = str(tmp_path / "formats.o")
    _run([CLANG, "-std=c++17", *san, f"-I{INC}", "-c", os.path.join(CSRC, "formats_host.cpp"), "-o", fmt])
    drv = str(tmp_path / "driver.o")
    _run([CLANG, "-std=c++17", *san, f"-I{INC}", "-c", os.path.join(ROOT, "tests", "asan", "host_driver.cpp"),
          "-o", drv])
    exe = str(tmp_path / "host_driver")
    _run([CLANG, "-fsanitize=address", api, fmt, drv, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout + r.stderr
    assert "AddressSanitizer" not in r.stderr, r.stderr
