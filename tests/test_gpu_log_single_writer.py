"""The base + log path's single-writer rule (DeltaLog, sec. 3.3 and the caption of Fig. 5:
one writer per head commits K_log[L], Lam_log[L], lbar and L), checked on the GPU with the
checking build of the library (librsu_check.so, built with RSU_CHECK_METADATA), whose log
kernels count every metadata element they write per head.

Per step and head, an append writes each of the 128 K_log and U_log elements of entry L
once and the Lam entry and lbar once per element (128 with per-key gates, 1 with a scalar
gate); a merge writes only lbar; a per-slot step also writes L once. The checking build
must also give the same results, bit for bit, as the ordinary one."""
import os

import numpy as np
import pytest
import torch

import workloads as wl
from parity import DEV, dev_inputs, log_step, new_log_buffers, rsu, say

pytestmark = pytest.mark.gpu

K, LAM, LBAR, LEN, U = range(5)


@pytest.fixture
def libs():
    m = rsu()
    from recurrent_state_update_head_amd._build import CHECK_LIB
    assert os.path.exists(CHECK_LIB), f"{CHECK_LIB} is not built (python -m recurrent_state_update_head_amd._build)"
    plain, checked = m.raw_library(), m._open(CHECK_LIB)
    with pytest.raises(m.RsuError, match="RSU_CHECK_METADATA"):
        m.debug_metadata_counts(1)  # the ordinary build keeps no counters
    return m, plain, checked


def _expected(L_before: np.ndarray, C: int, per_key: bool, slots: bool) -> np.ndarray:
    nl = 128 if per_key else 1
    e = np.zeros((len(L_before), 8), dtype=np.uint32)
    app = L_before < C
    e[app, K] = 128
    e[app, U] = 128
    e[app, LAM] = nl
    e[:, LBAR] = nl
    if slots:
        e[:, LEN] = 1
    return e


def _run(m, lib, w, slots: bool, check: bool):
    """C + 2 steps (a full cycle, a merge and one more append) on one library build;
    returns the final buffers and the number of steps whose counts were checked."""
    m.select_library(lib)
    B, H, C = w.B, w.H, w.M - 1
    Sbase = torch.from_numpy(wl.initial_state(w)).to(DEV).view(B, H, 128, 128)
    buf = new_log_buffers(w, C)
    y = torch.empty(B, H, 128, device=DEV)
    L_all = (np.arange(w.heads, dtype=np.int32) * 5) % (C + 1)
    Ld = torch.from_numpy(L_all.copy()).to(DEV).view(B, H)
    L = 0
    checked = 0
    if check:
        m.debug_metadata_counts(w.heads)  # clear what earlier calls counted
    for t in range(C + 2):
        _, d = dev_inputs(w, t)
        if slots:
            L_before = Ld.flatten().cpu().numpy()
            if w.variant == "rwkv6":
                m.rwkv6_log_step_slots(C, Ld, Sbase, buf["lbar"], buf["Klog"], buf["Ulog"], buf["Lam"],
                                       d["q"], d["k"], d["v"], d["gate"], y)
            else:
                (m.kda_log_step_slots if w.per_key_gate else m.gdn_log_step_slots)(
                    C, Ld, Sbase, buf["lbar"], buf["Klog"], buf["Ulog"], buf["Lam"],
                    d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
        else:
            L_before = np.full(w.heads, L, dtype=np.int32)
            L = log_step(w, C, L, Sbase, buf, d, y)
        if check:
            got = m.debug_metadata_counts(w.heads)
            want = _expected(L_before, C, w.per_key_gate, slots)
            bad = np.flatnonzero((got != want).any(axis=1))
            assert len(bad) == 0, (f"step {t}: {len(bad)} heads break the single-writer rule; head "
                                   f"{bad[0]} (L={L_before[bad[0]]}) wrote {got[bad[0], :5]}, "
                                   f"expected {want[bad[0], :5]}")
            checked += 1
    torch.cuda.synchronize()
    return {"Sbase": Sbase, "y": y, "L": Ld, **buf}, checked


@pytest.mark.parametrize("variant,qkv", [("gdn", "bf16"), ("kda", "bf16"), ("rwkv6", "bf16"), ("gdn", "f32")])
@pytest.mark.parametrize("slots", [False, True])
def test_log_metadata_written_once_per_head(libs, variant, qkv, slots):
    m, plain, checked_lib = libs
    if variant == "rwkv6":
        w = wl.custom(wl.WORKLOADS[8], B=64, H=48, M=8, qkv=qkv)
    else:
        w = wl.custom(wl.WORKLOADS[5], B=64, H=48, M=8, qkv=qkv, variant=variant,
                      gate_lo=0.8 if variant == "kda" else 0.9, gate_hi=1.0 if variant == "kda" else 0.999)
    say(f"[single writer] {variant} {qkv} slots={slots}: B=64 H=48 C=7, 9 steps")
    try:
        ref, _ = _run(m, plain, w, slots, check=False)
        got, n = _run(m, checked_lib, w, slots, check=True)
    finally:
        m.select_library(plain)
    assert n == w.M + 1
    for name in ref:
        assert torch.equal(ref[name], got[name]), f"{name} differs between the checking and ordinary builds"
