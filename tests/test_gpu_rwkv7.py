"""GPU parity of the RWKV7 step (erase along kappa read with a * kappa, then write k v^T, in
one pass over the state) against the pinned fp64 oracle, which takes the two sub-steps of
LeapQuant App. A in order. Tolerance: 1e-5 norm-wise relative error for outputs and the
final state."""
import pytest

import workloads as wl
from parity import TOL_F32, TOL_Q8, run_dense, run_window, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("qkv,B,H,steps", [("bf16", 3, 7, 12), ("f32", 5, 3, 12), ("bf16", 10, 10, 6)])
def test_rwkv7_dense_small_all_heads(qkv, B, H, steps):
    w = wl.custom(wl.WORKLOADS[10], B=B, H=H, qkv=qkv, steps=steps)
    ey, eS = run_dense(w)
    say(f"[rwkv7] dense {qkv} B={B} H={H}: y {ey:.2e} S {eS:.2e}")
    assert ey < TOL_F32 and eS < TOL_F32


def test_rwkv7_dense_b128_h32_full_size_sampled():
    w = wl.WORKLOADS[10]
    say(f"[rwkv7] {w.name}: full size, 64 sampled heads, {w.steps} steps")
    ey, eS = run_dense(w, sample=64)
    say(f"[rwkv7] {w.name}: y {ey:.2e} S {eS:.2e}")
    assert ey < TOL_F32 and eS < TOL_F32


# ---------------------------------------------------------------- two records per token

def _check_window(st, name):
    say(f"[rwkv7] {name}: {st}")
    assert st["init_codes_equal"] and st["init_scales_equal"]
    assert st["y"] < TOL_Q8
    assert st["a"] < 1e-5
    assert st["z_maxdiff"] <= 1
    assert st["z_flips_outside_band"] == 0
    assert st["boundaries"] > 0


@pytest.mark.parametrize("W,B,H,qkv", [(16, 3, 7, "bf16"), (5, 2, 5, "f32"), (1, 2, 3, "bf16"),
                                       (16, 10, 10, "bf16")])
def test_rwkv7_q8_window_small_all_heads(W, B, H, qkv):
    """Teacher-forced per window against the oracle's same schedule (outputs within 1e-4,
    codes +-1 only at rounding ties, row scales within 1e-5)."""
    w = wl.custom(wl.WORKLOADS[11], B=B, H=H, W=W, qkv=qkv, steps=2 * W + min(W, 3))
    _check_window(run_window(w), f"q8 window W={W} B={B} H={H} {qkv}")


def test_rwkv7_q8_window_b128_h32_full_size_sampled():
    w = wl.WORKLOADS[11]
    say(f"[rwkv7] {w.name}: full size, 64 sampled heads, 48 steps")
    _check_window(run_window(w, sample=64, steps=48), w.name)
