"""GPU parity of the RWKV7 step (erase along kappa read with a * kappa, then write k v^T, in
one pass over the state) against the pinned fp64 oracle, which takes the two sub-steps of
LeapQuant App. A in order. Tolerance: 1e-5 norm-wise relative error for outputs and the
final state."""
import pytest

import workloads as wl
from parity import TOL_F32, run_dense, say

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
