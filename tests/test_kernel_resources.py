"""Every kernel of the library keeps its data in registers and LDS: no private (scratch)
segment. A register array indexed by lane-dependent values, or a select between its elements
that the compiler folds into such an index, lands in scratch memory, which costs HBM traffic
and latency in every launch while the results stay correct (no parity test notices it).

The check compiles the device code of every HIP source with the library's own flags and reads
the compiler's resource remarks; it needs hipcc but no GPU."""
import concurrent.futures
import glob
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("_rsu_build_flags",
                                                  os.path.join(ROOT, "recurrent_state_update_head_amd", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _scratch_by_kernel(src, hipcc, flags):
    cmd = [hipcc, *[f for f in flags if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-c", src,
           "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True)
    assert out.returncode == 0, out.stderr[-2000:]
    found, name = {}, None
    for line in out.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            found[name] = int(m.group(1))
    return found


def test_no_kernel_uses_scratch():
    b = _build_module()
    if not os.path.exists(b.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    hipcc = b.HIPCC if os.path.exists(b.HIPCC) else shutil.which("hipcc")
    srcs = sorted(glob.glob(os.path.join(b.CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda s: _scratch_by_kernel(s, hipcc, b.FLAGS), srcs))
    kernels = {k: v for r in results for k, v in r.items()}
    assert len(kernels) > 20, f"expected the library's kernels, found {len(kernels)}"
    bad = {k: v for k, v in kernels.items() if v}
    assert not bad, f"kernels with a private segment (bytes per lane): {bad}"
