"""GPU parity of the RWKV6 path (dense step and base + log) against the fp64 oracle.

The update is the pages' common form without the delta read, S <- Diag(w) S + k v^T and
y = S^T q (DeltaLog Table 1, RWKV6 row; LeapQuant App. A eq. 1 with read vector 0). The
oracle's base + log steps equal its eager steps (a pinned property), so both GPU paths
are compared with the oracle of their own representation.

Tolerance: 1e-5 norm-wise relative error for outputs, final / merged states; logged keys
and logged values are copies of the inputs and must match bit for bit; log-decays within
1e-5."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity import DEV, TOL_F32, dev_inputs, log_step, new_log_buffers, rsu, run_dense, run_log, \
    run_log_slots, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("qkv,B,H,steps", [("bf16", 3, 7, 12), ("f32", 5, 3, 12), ("bf16", 10, 10, 6)])
def test_rwkv6_dense_small_all_heads(qkv, B, H, steps):
    w = wl.custom(wl.WORKLOADS[7], B=B, H=H, qkv=qkv, steps=steps)
    ey, eS = run_dense(w)
    say(f"[rwkv6] dense {qkv} B={B} H={H}: y {ey:.2e} S {eS:.2e}")
    assert ey < TOL_F32 and eS < TOL_F32


def test_rwkv6_dense_b128_h32_full_size_sampled():
    w = wl.WORKLOADS[7]
    say(f"[rwkv6] {w.name}: full size, 64 sampled heads, {w.steps} steps")
    ey, eS = run_dense(w, sample=64)
    say(f"[rwkv6] {w.name}: y {ey:.2e} S {eS:.2e}")
    assert ey < TOL_F32 and eS < TOL_F32


def _check_log(err, name):
    say(f"[rwkv6] {name}: {err}")
    assert err["y"] < TOL_F32 and err["Sbase"] < TOL_F32
    assert err["Ulog"] == 0.0 and err["Klog"] == 0.0
    assert err["lbar"] < 1e-5 and err["Lam"] < 1e-5


@pytest.mark.parametrize("M,B,H,qkv", [(4, 3, 7, "bf16"), (1, 2, 3, "bf16"), (8, 2, 5, "f32"),
                                       (17, 1, 3, "bf16"), (64, 1, 2, "bf16"), (4, 10, 10, "bf16")])
def test_rwkv6_log_small_all_heads(M, B, H, qkv):
    w = wl.custom(wl.WORKLOADS[8], B=B, H=H, M=M, qkv=qkv, steps=2 * M + 3)
    _check_log(run_log(w), f"log M={M} B={B} H={H} {qkv}")


def test_rwkv6_log_b128_h32_m4_full_size_sampled():
    w = wl.WORKLOADS[8]
    say(f"[rwkv6] {w.name}: full size, 64 sampled heads, {w.steps} steps")
    _check_log(run_log(w, sample=64), w.name)


@pytest.mark.parametrize("M,B,H", [(4, 2, 5), (8, 3, 4)])
def test_rwkv6_log_slots(M, B, H):
    w = wl.custom(wl.WORKLOADS[8], B=B, H=H, M=M, steps=2 * M + 3)
    err = run_log_slots(w)
    say(f"[rwkv6] slots M={M}: {err}")
    assert err["L"] == 0 and err["merges"] > 0 and err["appends"] > 0
    assert err["y"] < TOL_F32 and err["Sbase"] < TOL_F32
    assert err["Ulog"] == 0.0 and err["Klog"] == 0.0
    assert err["lbar"] < 1e-5 and err["Lam"] < 1e-5


def test_rwkv6_log_matches_gpu_eager():
    """The deferred representation and the GPU's eager RWKV6 step give the same outputs."""
    m = rsu()
    w = wl.custom(wl.WORKLOADS[8], B=4, H=6, steps=20)
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
        m.rwkv6_decode_step(S_eager, d["q"], d["k"], d["v"], d["gate"], y_e)
        L = log_step(w, C, L, S_base, buf, d, y_l)
        num = torch.linalg.vector_norm(y_l - y_e, dim=-1)
        den = torch.linalg.vector_norm(y_e, dim=-1).clamp_min(1e-30)
        worst = max(worst, float((num / den).max()))
    say(f"[rwkv6] GPU log vs GPU eager: {worst:.3e}")
    assert worst < TOL_F32
