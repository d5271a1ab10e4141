"""Build librsu.so (the gfx950 kernels and the C ABI of include/rsu.h) in-tree with hipcc,
and librsu_check.so, the same library with the log kernels' metadata write counters
(RSU_CHECK_METADATA), which only the single-writer test loads."""
from __future__ import annotations

import glob
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librsu.so")
CHECK_LIB = os.path.join(PKG, "librsu_check.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the LeapQuant boundaries need no AGPR block
    # beside the refit's registers, which keeps three of their workgroups on a CU
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"),
]
# the one source whose kernels carry the checking build's counters
CHECKED = "deltalog.hip"


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res.stdout + res.stderr


def build(verbose: bool = False) -> str:
    """Compile every HIP source (always recompiles) and link librsu.so and librsu_check.so."""
    with tempfile.TemporaryDirectory(prefix="rsu_build_") as tmp:
        jobs = [(src, os.path.join(tmp, os.path.basename(src) + ".o"), []) for src in sources()]
        jobs.append((os.path.join(CSRC, CHECKED), os.path.join(tmp, "checked.o"), ["-DRSU_CHECK_METADATA"]))
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
        with ThreadPoolExecutor(workers) as pool:
            logs = list(pool.map(lambda j: _run([HIPCC, *FLAGS, *j[2], "-c", "-o", j[1], j[0]]), jobs))
        plain = [o for s, o, extra in jobs if not extra]
        checked = [o for s, o, extra in jobs if extra or os.path.basename(s) != CHECKED]
        for lib, objs in ((LIB, plain), (CHECK_LIB, checked)):
            logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp", *objs]))
            os.replace(lib + ".tmp", lib)
    if verbose:
        print("".join(logs))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
