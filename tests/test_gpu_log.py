"""GPU parity of the dense base + log path (append / merge) against the fp64 oracle's
base + log steps, which equal eager decoding (a pinned oracle property), and
against the GPU's own eager dense step.

Tolerance: 1e-5 relative error (norm-wise and element-wise) for outputs, merged bases and logged
value factors; logged keys are copied bit-exactly; log-decays within 1e-5."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity import (DEV, TOL_F32, dev_inputs, log_step, new_log_buffers, rel_err, rsu, run_log,
                    run_log_slots, say)

pytestmark = pytest.mark.gpu


def _check(err, name):
    say(f"[log] {name}: {err}")
    assert err["y"] < TOL_F32 and err["Sbase"] < TOL_F32 and err["Ulog"] < TOL_F32
    assert err["Klog"] == 0.0
    assert err["lbar"] < 1e-5 and err["Lam"] < 1e-5


@pytest.mark.parametrize("variant,M,B,H,qkv", [("gdn", 8, 3, 7, "bf16"), ("gdn", 1, 2, 3, "bf16"),
                                               ("gdn", 2, 2, 2, "f32"), ("kda", 4, 2, 5, "bf16"),
                                               ("kda", 8, 1, 3, "f32"), ("gdn", 17, 1, 2, "bf16"),
                                               ("gdn", 8, 10, 10, "bf16"), ("gdn", 32, 2, 3, "bf16"),
                                               ("kda", 64, 1, 2, "bf16"), ("gdn", 64, 1, 3, "f32")])
def test_log_small_all_heads(variant, M, B, H, qkv):
    w = wl.custom(wl.WORKLOADS[5], B=B, H=H, M=M, qkv=qkv, steps=2 * M + 3, variant=variant,
                  gate_lo=0.8 if variant == "kda" else 0.9, gate_hi=1.0 if variant == "kda" else 0.999)
    _check(run_log(w), f"{variant} M={M} B={B} H={H} {qkv}")


def test_log_b256_h48_full_size_sampled():
    """The base + log workload at full size (B=256, H=48, M=8, 128 steps), 64 sampled heads."""
    w = wl.WORKLOADS[5]
    say(f"[log] {w.name}: full size, 64 sampled heads, {w.steps} steps")
    _check(run_log(w, sample=64), w.name)


@pytest.mark.parametrize("M", [4, 8])
def test_kda_log_b128_h32_full_grid_sampled(M):
    """KDA gates on the base + log path over the full grid of the KDA workload (B=128,
    H=32, 4,096 heads, the XCD-grouped head order of every full block), three cycles and
    two steps into the fourth, 64 sampled heads."""
    w = wl.custom(wl.WORKLOADS[5], B=128, H=32, M=M, steps=3 * M + 2, variant="kda", gate_lo=0.8, gate_hi=1.0)
    say(f"[log] kda B=128 H=32 M={M}: full grid, 64 sampled heads, {w.steps} steps")
    _check(run_log(w, sample=64), f"kda log b128 h32 m{M}")


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_log_matches_gpu_eager(variant):
    """The deferred representation and the GPU's eager dense step give the same outputs."""
    m = rsu()
    w = wl.custom(wl.WORKLOADS[5], B=4, H=6, steps=20, variant=variant,
                  gate_lo=0.8 if variant == "kda" else 0.9, gate_hi=1.0 if variant == "kda" else 0.999)
    C = w.M - 1
    S0 = torch.from_numpy(wl.initial_state(w)).to(DEV).view(w.B, w.H, 128, 128)
    S_eager, S_base = S0.clone(), S0.clone()
    buf = new_log_buffers(w, C)
    y_e = torch.empty(w.B, w.H, 128, device=DEV)
    y_l = torch.empty_like(y_e)
    L = 0
    worst = 0.0
    for t in range(w.steps):
        _, d = dev_inputs(w, t)
        (m.kda_decode_step if variant == "kda" else m.gdn_decode_step)(
            S_eager, d["q"], d["k"], d["v"], d["gate"], d["beta"], y_e)
        L = log_step(w, C, L, S_base, buf, d, y_l)
        worst = max(worst, rel_err(y_l.cpu().numpy().reshape(-1, 128), y_e.cpu().numpy().reshape(-1, 128)))
        if L == 0:
            worst = max(worst, rel_err(S_base.cpu().numpy().reshape(-1, 128 * 128),
                                       S_eager.cpu().numpy().reshape(-1, 128 * 128)))
    say(f"[log] GPU log vs GPU eager ({variant}): {worst:.3e}")
    assert worst < TOL_F32


def _check_slots(err, name, C):
    say(f"[log slots] {name}: {err}")
    assert err["L"] == 0
    assert err["merges"] > 0 and (err["appends"] > 0 or C == 0)
    assert err["y"] < TOL_F32 and err["Sbase"] < TOL_F32 and err["Ulog"] < TOL_F32
    assert err["Klog"] == 0.0
    assert err["lbar"] < 1e-5 and err["Lam"] < 1e-5


@pytest.mark.parametrize("variant,M,B,H,qkv", [("gdn", 8, 2, 5, "bf16"), ("kda", 4, 2, 5, "bf16"),
                                               ("gdn", 1, 1, 3, "f32"), ("kda", 32, 1, 4, "f32"),
                                               ("gdn", 64, 1, 3, "bf16")])
def test_log_slots_mixed_phases(variant, M, B, H, qkv):
    """Per-slot live lengths: heads at staggered points of their cycle, so appends and
    merges of different heads share each launch; live lengths advance on the device."""
    w = wl.custom(wl.WORKLOADS[5], B=B, H=H, M=M, qkv=qkv, steps=2 * M + 3, variant=variant,
                  gate_lo=0.8 if variant == "kda" else 0.9, gate_hi=1.0 if variant == "kda" else 0.999)
    _check_slots(run_log_slots(w), f"{variant} M={M} B={B} H={H} {qkv}", M - 1)


def test_log_slots_b256_h48_sampled():
    """Per-slot live lengths at full size (B=256, H=48, M=8), 64 sampled heads."""
    w = wl.WORKLOADS[5]
    say(f"[log slots] {w.name}: full size, 64 sampled heads, 24 steps")
    _check_slots(run_log_slots(w, sample=64, steps=24), w.name + " slots", w.M - 1)
