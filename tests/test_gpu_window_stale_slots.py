"""Stale record slots never reach a result, on every window path.

Inside a window the state is the window-start representation plus the records appended so far
(LeapQuant, sec. 3.2, eq. 9; the token format's readout, eq. 10): a slot at or past the current
position holds whatever an earlier window, or the allocator, left there. The step kernels load
record slots without a branch (a branch around a load makes the compiler wait for every earlier
load): a lane past the last record reads slot 0, and a slot group with no record at all reads the
lane's own inputs; such values must never be used, or meet only a zero coefficient.

Each path runs two windows twice from the same start, once with zeroed record buffers and once
with every record slot set to NaN; the outputs y of every step and the representation at the end
must agree bit for bit (the kernels are deterministic, so any use of a stale slot shows as a NaN or
as a difference)."""
import pytest
import torch

import workloads as wl
from parity import DEV, dev_inputs, new_lq_buffers, new_window_buffers, rsu, say, window_step

pytestmark = pytest.mark.gpu

RECORDS = ("Kbuf", "Ubuf", "Gbuf")


def _q8_run(w, fill):
    m = rsu()
    buf = new_window_buffers(w)
    for name in RECORDS:
        buf[name].fill_(fill)
    S0 = torch.from_numpy(wl.initial_state(w)).to(DEV).view(w.B, w.H, 128, 128)
    m.q8_quantize(S0, buf["Z"], buf["A"])
    y = torch.empty(w.B, w.H, 128, device=DEV)
    ys = []
    for t in range(2 * w.W):
        _, d = dev_inputs(w, t)
        window_step(w, t % w.W, buf, d, y)
        ys.append(y.clone())
    torch.cuda.synchronize()
    return torch.stack(ys), {"Z": buf["Z"], "A": buf["A"]}


def _lq_fns(m, w):
    pre = "kda" if w.per_key_gate else "gdn"
    bits = {8: "lq", 6: "lq6", 4: "lq4"}[w.bits]
    return getattr(m, f"{pre}_{bits}_quantize"), getattr(m, f"{pre}_{bits}_window")


def _lq_run(w, fill):
    m = rsu()
    quantize, window = _lq_fns(m, w)
    buf = new_lq_buffers(w)
    for name in RECORDS:
        buf[name].fill_(fill)
    S0 = torch.from_numpy(wl.initial_state(w)).to(DEV).view(w.B, w.H, 128, 128)
    quantize(S0, 8, buf["Z"], buf["B"], buf["C"], buf["Kc"], buf["Uc"])
    y = torch.empty(w.B, w.H, 128, device=DEV)
    ys = []
    for t in range(2 * w.W):
        _, d = dev_inputs(w, t)
        window(w.W, t % w.W, 1, buf["Z"], buf["B"], buf["C"], buf["Kc"], buf["Uc"], buf["Kbuf"], buf["Ubuf"],
               buf["Gbuf"], d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
        ys.append(y.clone())
    torch.cuda.synchronize()
    return torch.stack(ys), {k: buf[k] for k in ("Z", "B", "C", "Kc", "Uc")}


# (label, workload index, overrides, runner); 2 x 48 heads: more than one block of the
# head order that groups heads by XCD
CASES = [
    ("gdn q8", 4, {}, _q8_run),
    ("kda q8", 4, {"variant": "kda", "gate_lo": 0.8, "gate_hi": 1.0}, _q8_run),
    ("rwkv7 q8", 11, {}, _q8_run),
    ("deltaproduct q8", 15, {}, _q8_run),
    ("gdn lq", 6, {}, _lq_run),
    ("kda lq", 9, {}, _lq_run),
    ("gdn lq4", 12, {}, _lq_run),
    ("gdn lq6", 16, {}, _lq_run),
    ("kda lq4", 17, {}, _lq_run),
    ("kda lq6", 18, {}, _lq_run),
]


@pytest.mark.parametrize("label,idx,over,run", CASES, ids=[c[0].replace(" ", "_") for c in CASES])
def test_nan_in_unwritten_record_slots_changes_nothing(label, idx, over, run):
    w = wl.custom(wl.WORKLOADS[idx], B=2, H=48, steps=2 * wl.WORKLOADS[idx].W, **over)
    say(f"[stale slots] {label}: B=2 H=48 W={w.W}, two windows, records zeroed vs NaN")
    y0, rep0 = run(w, 0.0)
    y1, rep1 = run(w, float("nan"))
    assert torch.isfinite(y0).all(), f"{label}: non-finite output from zeroed record buffers"
    bad = (y0 != y1).any(dim=-1).nonzero()
    assert len(bad) == 0, (f"{label}: {len(bad)} (step, head) outputs differ with NaN in unwritten slots, "
                           f"first at step {int(bad[0, 0])}")
    for name in rep0:
        assert torch.equal(rep0[name], rep1[name]), f"{label}: {name} differs with NaN in unwritten slots"
