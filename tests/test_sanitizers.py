"""Host AddressSanitizer / UndefinedBehaviorSanitizer builds, run on the CPU.

* The fp64 oracle (oracle/rsu_oracle.c) is built with gcc and both sanitizers and driven
  through every one of its functions on small heads by tests/sanitize/oracle_driver.c.
* The C ABI (csrc/*.hip) is built with the sanitizers on its host code only (the device
  code is compiled as usual and never runs) and tests/sanitize/abi_driver.c calls every
  entry point with arguments that fail validation, or with an empty batch, so only the
  argument checks and the error reporting run, with no GPU.

Any out-of-bounds access, use after free or undefined operation aborts the driver with a
report, which the test prints.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

UBSAN_ENV = {"UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, env=None, timeout=300):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout,
                         env={**os.environ, **(env or {})})
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout[-4000:] + res.stderr[-4000:]
    return res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fopenmp", "-std=c11", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "rsu_oracle.c"),
          "-o", exe, "-lm"])
    out = _run([exe], env={**UBSAN_ENV, "ASAN_OPTIONS": "detect_leaks=1", "OMP_NUM_THREADS": "2"})
    assert "oracle driver ok" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_validation_under_host_asan_ubsan(tmp_path):
    lib = str(tmp_path / "librsu_san.so")
    srcs = sorted(os.path.join(ROOT, "recurrent_state_update_head_amd", "csrc", f)
                  for f in os.listdir(os.path.join(ROOT, "recurrent_state_update_head_amd", "csrc"))
                  if f.endswith(".hip"))
    # each sanitizer flag is scoped to the host pass with its own -Xarch_host
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", *host_san,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-I", os.path.join(ROOT, "include"),
          "-o", lib, *srcs], timeout=600)
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "-x", "c", "-O1", "-g", *host_san, "-I", os.path.join(ROOT, "include"),
          os.path.join(SAN, "abi_driver.c"), "-o", exe, "-L", str(tmp_path), "-lrsu_san",
          "-Wl,-rpath," + str(tmp_path)])
    # the HIP runtime keeps its allocations until exit: leak checking stays off here
    out = _run([exe], env={**UBSAN_ENV, "ASAN_OPTIONS": "detect_leaks=0"})
    assert "abi driver ok" in out
