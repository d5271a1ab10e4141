"""bench.py's algorithmic byte accounting against sizes and formulas the pages print
(tests/golden/page_figures.json, each entry cited)."""
import json
import os

import pytest

import bench
import workloads as wl

FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _state_part(w):
    """Bytes of a dense step that are state traffic (the rest is q/k/v/gates/y)."""
    d = wl.DK
    other = 3 * d * (2 if w.qkv == "bf16" else 4) + (4 * d if w.per_key_gate else 4) + 4 + 4 * d
    return bench.dense_bytes_per_head(w) - other


def test_one_gib_state_and_two_gib_per_eager_step():
    f = FIG["state_1gib"]
    w = wl.custom(wl.WORKLOADS[2], B=f["B"], H=f["H"])
    assert 4 * f["dk"] * f["dv"] * w.heads == f["state_bytes"]
    assert _state_part(w) * w.heads == f["eager_state_traffic_bytes"]


def test_dense_step_moves_8_bytes_per_state_element():
    f = FIG["dense_intensity"]
    for cid in (1, 2, 3):
        w = wl.WORKLOADS[cid]
        assert _state_part(w) == f["bytes_per_state_element_moved"] * wl.DK * wl.DV
    assert f["flops_per_state"] / f["bytes_per_state_element_moved"] == f["ai"]


def test_request_state_size():
    f = FIG["request_state_144mib"]
    assert f["heads"] * f["dk"] * f["dv"] * 4 == f["bytes"] == 144 * 2 ** 20


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_log_entry_bytes_match_eq9(variant):
    f = FIG["log_entry_bytes"][f"{variant}_bf16"]
    w = wl.custom(wl.WORKLOADS[5], variant=variant)
    eq9 = f["pK"] * wl.DK + f["pU"] * wl.DV + 4 * f["dlambda"]
    assert eq9 == f["per_head"]
    # an append at L+1 reads one more entry than an append at L
    assert bench.log_step_bytes_per_head(w, 1) - bench.log_step_bytes_per_head(w, 0) == eq9


@pytest.mark.parametrize("M", FIG["log_traffic_model"]["M"])
def test_log_cycle_matches_eq10(M):
    """Cycle-averaged log-entry traffic of bench.py equals eq. 10 exactly."""
    w = wl.custom(wl.WORKLOADS[5], M=M)
    d = wl.DK
    c_entry = 2 * d + 4 * d + 4
    per_step = [bench.log_step_bytes_per_head(w, L) for L in range(M)]
    # remove what is not log-entry traffic: base read, lbar, inputs, y, and the merge's base write
    base = 4 * d * d + 4 + (3 * d * 2 + 4 + 4) + 4 * d
    entry_traffic = sum(per_step) - M * base - (4 * d * d + 4) - (M - 1) * 4
    assert entry_traffic / M == pytest.approx(c_entry * ((M - 1) / M + (M - 1) / 2), rel=0, abs=1e-9)


def test_window_buffer_8kib():
    f = FIG["window_buffer_8kib"]
    assert f["W"] * (f["dk"] + f["dv"]) * f["bytes_per_value"] == f["bytes"]
    # bench.py's records hold k in its input dtype, u in fp32 and the gate: at bf16 keys
    w = wl.WORKLOADS[4]
    rec = bench.window_step_bytes_per_head(w, 1) - bench.window_step_bytes_per_head(w, 0)
    assert rec == 2 * wl.DK + 4 * wl.DV + 4
    assert f["W"] * (2 * wl.DK + 2 * wl.DV) == f["bytes"]


def test_headline_workload_bytes():
    w = wl.WORKLOADS[2]
    assert bench.dense_bytes_per_head(w) == 132360
    assert bench.cycle_bytes_per_head(wl.WORKLOADS[4]) == pytest.approx(25754, abs=1)
    assert bench.cycle_bytes_per_head(wl.WORKLOADS[5]) == pytest.approx(78401.5, abs=1e-9)


@pytest.mark.parametrize("variant,M", [("gdn", 1), ("gdn", 2), ("gdn", 8), ("gdn", 64), ("kda", 4), ("kda", 16)])
def test_log_cycle_bytes_follow_the_traffic_model(variant, M):
    """DeltaLog sec. 3.2, eqs. 10-11: per step the base is read (C_state), written once
    per M steps (C_state / M), an entry is appended in M-1 of M steps and (M-1)/2
    entries are replayed on average (C_log(M) = ((M-1)/M + (M-1)/2) C_entry), and the
    cumulative log-decay is read and written (2 C_decay). The rest is T_common (q, k,
    v, gate, beta, y). bench.py's cycle average must be exactly that sum."""
    from fractions import Fraction as Fr
    w = wl.custom(wl.WORKLOADS[5], variant=variant, M=M)
    d = wl.DK
    gdim = d if w.per_key_gate else 1
    c_state = 4 * d * d
    c_entry = d * 2 + 4 * d + 4 * gdim          # bf16 key factor, fp32 value factor, Lam
    c_decay = 4 * gdim
    t_common = 3 * d * 2 + 4 * gdim + 4 + 4 * d  # bf16 q/k/v, gate, beta, fp32 y
    c_log = (Fr(M - 1, M) + Fr(M - 1, 2)) * c_entry
    model = t_common + c_state + Fr(c_state, M) + c_log + 2 * c_decay
    assert Fr(bench.cycle_bytes_per_head(w)) == model
    # a batch at random cycle points moves, per head, what its live-length mix dictates
    w2 = wl.custom(w, B=8, H=16)
    L = bench.slot_lengths(w2)
    per = [bench.log_step_bytes_per_head(w2, int(x)) for x in L]
    assert bench.slots_bytes_per_head(w2) == pytest.approx(sum(per) / len(per), rel=1e-15)


def test_deltaproduct_bytes():
    """DeltaProduct with n = 2 (bf16): the dense step moves the state both ways plus q, two keys,
    two values (bf16), alpha, two betas and y; with n = 1 it is the GDN step's accounting. On
    the window each sub-step is a 772-byte record (bf16 key, fp32 value, fp32 scalar gate)."""
    w = wl.WORKLOADS[14]
    assert bench.dense_bytes_per_head(w) == 131072 + 5 * 256 + 4 + 8 + 512
    assert bench.dense_bytes_per_head(wl.custom(w, n=1)) == bench.dense_bytes_per_head(wl.WORKLOADS[2])
    ww = wl.WORKLOADS[15]
    rec = 256 + 512 + 4
    inputs = 5 * 256 + 4 + 8
    assert bench.window_step_bytes_per_head(ww, 3) == 16384 + 512 + 6 * rec + inputs + 512 + 2 * rec
    last = bench.window_step_bytes_per_head(ww, 15)
    assert last == (16384 + 512 + 30 * rec + inputs + 512 + 2 * rec) + (16384 + 512 + 32 * rec) + (16384 + 512)


def test_lq_low_bit_representation_bytes():
    """LeapQuant's boundary representation per head: the payload (16384, 12288 or 8192
    bytes at 8, 6 or 4 bits), fp32 B and c (512 each) and r fp16 token pairs (r = 4, 4, 8).
    A step at pos 0 reads it with the inputs (3 bf16 vectors, alpha, beta) and writes y and
    one record (bf16 key, fp32 value, fp32 gate)."""
    rec = 256 + 512 + 4
    inputs = 3 * 256 + 4 + 4
    for cid, payload, r in ((6, 16384, 4), (16, 12288, 4), (12, 8192, 8)):
        w = wl.WORKLOADS[cid]
        rep = payload + 512 + 512 + 2 * r * 128 * 2
        assert bench.lq_step_bytes_per_head(w, 0) == rep + inputs + 512 + rec
        assert bench.lq_step_bytes_per_head(w, w.W - 1) == rep + (w.W - 1) * rec + inputs + 512 + rep
