"""STEPQuant's per-step packed state on the GPU (stepq_pack, gdn_stepq_step,
kda_stepq_step through the C ABI) against the fp64 oracle, teacher-forced per step.

Every step's output must match the dense step from the GPU's packed state before it to
the fp32 tolerance. Every packing (of the initial state and after each step) is checked
piece by piece: row factors are the fp16 rounding of the exact sqrt(m_i / w_i), codes are
recomputed from the GPU's row factors, column factors are the fp16 rounding of the
weighted least squares recomputed from the GPU's codes; a difference is allowed only
within a narrow band of a rounding tie (fp32 arithmetic on the GPU against fp64), and
such ties must stay rare.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from parity import DEV, TOL_F32, new_stepq_buffers, rsu, run_stepq, say, stepq_host

pytestmark = pytest.mark.gpu

BASE = wl.WORKLOADS[13]


def _kda(base, **kw):
    return wl.custom(base, variant="kda", gate_lo=0.8, gate_hi=1.0, **kw)


def _assert_ok(err, tol=TOL_F32):
    say(err)
    assert err["y"] < tol
    assert err["r_off"] == 0
    assert err["c_off"] == 0
    assert err["z_maxdiff"] <= 1
    assert err["z_flips_outside_band"] == 0
    assert err["r_ties"] + err["c_ties"] <= max(2, err["rows"] // 100)


@pytest.mark.parametrize("variant", ["gdn", "kda"])
@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_stepq_small_all_heads(variant, qkv):
    w = wl.custom(BASE, B=3, H=5, qkv=qkv)
    if variant == "kda":
        w = _kda(w)
    say(f"stepq {variant} {qkv} B=3 H=5")
    _assert_ok(run_stepq(w, steps=6))


def test_stepq_ragged_grid():
    """100 heads: three whole groups of the XCD head map and a ragged tail."""
    w = wl.custom(BASE, B=10, H=10)
    say("stepq gdn B=10 H=10")
    _assert_ok(run_stepq(w, steps=3))


def test_stepq_full_size_sampled():
    say(f"stepq {BASE.name} sampled")
    _assert_ok(run_stepq(BASE, sample=16, steps=3))


def test_stepq_kda_full_size_sampled():
    w = _kda(BASE, B=128, H=32)
    say("stepq kda B=128 H=32 sampled")
    _assert_ok(run_stepq(w, sample=12, steps=2))


def test_stepq_uniform_influence():
    """omega constant over the rows: every w_i = 1."""
    w = wl.custom(BASE, B=2, H=3)
    say("stepq uniform omega")
    _assert_ok(run_stepq(w, steps=3, om=np.full((w.heads, 128), 3.5, np.float32)))


def test_stepq_extreme_influence_spread():
    """omega log-uniform over 24 decades (w over 6): the row weights' log2 / exp2 path and the
    fp16 factors stay within the oracle's bars."""
    w = wl.custom(BASE, B=2, H=3)
    rng = np.random.default_rng(17)
    om = (10.0 ** rng.uniform(-12, 12, size=(w.heads, 128))).astype(np.float32)
    say("stepq extreme omega")
    _assert_ok(run_stepq(w, steps=3, om=om))


def test_stepq_zero_state():
    """A zero state packs to zero codes and factors; the first step then writes k (beta v)^T."""
    w = wl.custom(BASE, B=2, H=3)
    S0 = np.zeros((w.heads, 128, 128), np.float32)
    m = rsu()
    buf = new_stepq_buffers(w)
    m.stepq_pack(torch.from_numpy(S0).to(DEV).view(w.B, w.H, 128, 128),
                 torch.from_numpy(wl.row_influence(w)).to(DEV).view(w.B, w.H, 128), buf["Z"], buf["R"], buf["C"])
    z, r, c = stepq_host(buf, torch.arange(w.heads, device=DEV))
    assert not z.any() and not r.any() and not c.any()
    say("stepq zero state")
    _assert_ok(run_stepq(w, steps=2, S0=S0))


def test_stepq_zero_rows_and_columns():
    w = wl.custom(BASE, B=2, H=3)
    S0 = wl.initial_state(w)
    S0[:, 7, :] = 0.0
    S0[:, :, 40] = 0.0
    S0[1, :, :] = 0.0
    say("stepq zero rows and columns")
    m = rsu()
    buf = new_stepq_buffers(w)
    m.stepq_pack(torch.from_numpy(S0).to(DEV).view(w.B, w.H, 128, 128),
                 torch.from_numpy(wl.row_influence(w)).to(DEV).view(w.B, w.H, 128), buf["Z"], buf["R"], buf["C"])
    z, r, c = stepq_host(buf, torch.arange(w.heads, device=DEV))
    assert not r[:, 7].any() and not z[:, 7, :].any()
    assert not c[:, 40].any() and not z[:, :, 40].any()
    assert not z[1].any() and not r[1].any() and not c[1].any()
    _assert_ok(run_stepq(w, steps=2, S0=S0))


def test_stepq_tiny_column():
    """A column whose range a_j = max_i |x_ij| / r_i lies near 2^-128, where 7 / a_j overflows
    fp32 (the column's state entries are at most 2^-130): its fp16 column factor, about
    a_j / 7, is zero on both sides, so it decodes to zero whatever its codes; the rest of the
    packing is checked as usual."""
    w = wl.custom(BASE, B=2, H=3)
    S0 = wl.initial_state(w)
    col = 21
    e = np.ceil(np.log2(np.abs(S0[:, :, col]).max(axis=1).astype(np.float64))).astype(np.int32)
    S0[:, :, col] = np.ldexp(S0[:, :, col], (-130 - e)[:, None])
    say("stepq tiny column")
    m = rsu()
    buf = new_stepq_buffers(w)
    m.stepq_pack(torch.from_numpy(S0).to(DEV).view(w.B, w.H, 128, 128),
                 torch.from_numpy(wl.row_influence(w)).to(DEV).view(w.B, w.H, 128), buf["Z"], buf["R"], buf["C"])
    z, r, c = stepq_host(buf, torch.arange(w.heads, device=DEV))
    assert not c[:, col].any()
    err = run_stepq(w, steps=1, S0=S0)
    assert err["tiny_cols"] == w.heads
    _assert_ok(err)


def test_stepq_empty_batch():
    m = rsu()
    w = wl.custom(BASE, B=0, H=4)
    buf = new_stepq_buffers(w)
    om = torch.ones(0, 4, 128, device=DEV)
    q = torch.zeros(0, 4, 128, device=DEV, dtype=torch.bfloat16)
    y = torch.zeros(0, 4, 128, device=DEV)
    m.stepq_pack(torch.zeros(0, 4, 128, 128, device=DEV), om, buf["Z"], buf["R"], buf["C"])
    m.gdn_stepq_step(buf["Z"], buf["R"], buf["C"], om, q, q, q, torch.zeros(0, 4, device=DEV),
                     torch.zeros(0, 4, device=DEV), y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("variant", ["gdn", "kda"])
@pytest.mark.parametrize("shape", [(4, 6), (256, 48)])
def test_stepq_split_equals_fused(variant, shape):
    """The readout on the caller's stream and the repack on a second stream (ordered with
    events, as a caller would overlap it with other work) give y and the new packed state of
    the fused step bit for bit, step after step."""
    from parity import dev_inputs
    m = rsu()
    w = wl.custom(BASE, B=shape[0], H=shape[1])
    if variant == "kda":
        w = _kda(w)
    say(f"stepq split {variant} B={w.B} H={w.H}")
    S0 = torch.from_numpy(wl.initial_state(w)).to(DEV).view(w.B, w.H, 128, 128)
    om = torch.from_numpy(wl.row_influence(w)).to(DEV).view(w.B, w.H, 128)
    a, b = new_stepq_buffers(w), new_stepq_buffers(w)
    m.stepq_pack(S0, om, a["Z"], a["R"], a["C"])
    del S0
    for n in a:
        b[n].copy_(a[n])
    fused = m.kda_stepq_step if variant == "kda" else m.gdn_stepq_step
    readout = m.kda_stepq_readout if variant == "kda" else m.gdn_stepq_readout
    repack = m.kda_stepq_repack if variant == "kda" else m.gdn_stepq_repack
    ya = torch.zeros(w.B, w.H, 128, device=DEV)
    yb = torch.zeros_like(ya)
    u = torch.zeros_like(ya)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for t in range(4):
        d = dev_inputs(w, t)[1]
        fused(a["Z"], a["R"], a["C"], om, d["q"], d["k"], d["v"], d["gate"], d["beta"], ya)
        readout(b["Z"], b["R"], b["C"], d["q"], d["k"], d["v"], d["gate"], d["beta"], u, yb)
        done_read = torch.cuda.Event()
        done_read.record(main)
        with torch.cuda.stream(side):
            side.wait_event(done_read)
            repack(b["Z"], b["R"], b["C"], om, d["k"], d["gate"], u)
            done_pack = torch.cuda.Event()
            done_pack.record(side)
        main.wait_event(done_pack)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), f"step {t}: y differs"
        for n in a:
            assert torch.equal(a[n], b[n]), f"step {t}: {n} differs"
