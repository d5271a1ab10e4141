"""GPU parity of DeltaProduct (n delta-rule sub-steps per token, LeapQuant App. A Table 4)
against the fp64 oracle: the dense one-pass step, and the int8 window with one record per
sub-step, teacher-forced per window like the single-record window.

Bars: dense state and outputs within 1e-5 relative error (norm-wise and element-wise);
window outputs within 1e-4 of the oracle restarted from the GPU's window-start state,
requantized codes within 1 LSB and only inside the 1e-3-LSB tie band, row scales within
1e-5 relative."""
import pytest

import workloads as wl
from parity import TOL_F32, TOL_Q8, run_dense, run_window, say

pytestmark = pytest.mark.gpu


def _dense(n, qkv, B=2, H=5, steps=6):
    return wl.custom(wl.WORKLOADS[14], B=B, H=H, n=n, qkv=qkv, steps=steps)


@pytest.mark.parametrize("n,qkv", [(1, "bf16"), (2, "bf16"), (2, "f32"), (3, "bf16"), (4, "f32"), (4, "bf16")])
def test_dense_small_all_heads(n, qkv):
    ey, eS = run_dense(_dense(n, qkv))
    say(f"[dp dense] n={n} {qkv}: y {ey:.2e} S {eS:.2e}")
    assert ey < TOL_F32 and eS < TOL_F32


def test_dense_b256_h48_full_size_sampled():
    w = wl.WORKLOADS[14]
    say(f"[dp dense] {w.name}: full size, 96 sampled heads, {w.steps} steps")
    ey, eS = run_dense(w, sample=96)
    say(f"[dp dense] {w.name}: y {ey:.2e} S {eS:.2e}")
    assert ey < TOL_F32 and eS < TOL_F32


def _check(st, name):
    say(f"[dp q8] {name}: {st}")
    assert st["init_codes_equal"] and st["init_scales_equal"]
    assert st["y"] < TOL_Q8
    assert st["a"] < 1e-5
    assert st["z_maxdiff"] <= 1
    assert st["z_flips_outside_band"] == 0


@pytest.mark.parametrize("n,W,qkv,B,H", [(2, 16, "bf16", 3, 7), (2, 1, "bf16", 2, 3), (2, 3, "f32", 2, 3),
                                         (3, 5, "bf16", 2, 3), (4, 8, "f32", 2, 2), (1, 16, "bf16", 2, 3),
                                         (2, 16, "bf16", 10, 10)])
def test_window_small_all_heads(n, W, qkv, B, H):
    w = wl.custom(wl.WORKLOADS[15], B=B, H=H, n=n, W=W, qkv=qkv, steps=2 * W + 3)
    _check(run_window(w), f"n={n} W={W} {qkv} B={B} H={H}")


def test_window_b256_h48_full_size_sampled():
    """The DeltaProduct window at full size (B=256, H=48, n=2, W=16: 32 records per window),
    three windows and two steps into the fourth, 64 sampled heads."""
    w = wl.custom(wl.WORKLOADS[15], steps=3 * 16 + 2)
    say(f"[dp q8] {w.name}: full size, 64 sampled heads, {w.steps} steps")
    _check(run_window(w, sample=64), w.name)
