"""The seeded input generators: reproducible, shaped and distributed as the
workloads prescribe, bf16 values exactly representable."""
import numpy as np
import pytest

import workloads as wl


def _small(cid, **kw):
    return wl.custom(wl.WORKLOADS[cid], **kw)


def test_reproducible_and_step_independent():
    w = _small(2, B=3, H=5)
    a = wl.step_inputs(w, 4)
    b = wl.step_inputs(w, 4)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    c = wl.step_inputs(w, 5)
    assert not np.array_equal(a["q"], c["q"])
    np.testing.assert_array_equal(wl.initial_state(w), wl.initial_state(w))


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_shapes_dtypes_and_ranges(cid):
    w = _small(cid, B=4, H=6)
    x = wl.step_inputs(w, 0)
    n = w.heads
    assert x["q"].shape == (n, 128) and x["k"].shape == (n, 128) and x["v"].shape == (n, 128)
    assert x["gate"].shape == ((n, 128) if w.per_key_gate else (n,))
    assert all(a.dtype == np.float32 for a in x.values())
    assert np.all((x["gate"] >= w.gate_lo) & (x["gate"] <= w.gate_hi))
    assert np.all((x["beta"] >= 0) & (x["beta"] <= 1))
    tol = 1e-6 if w.qkv == "f32" else 1e-2
    np.testing.assert_allclose(np.linalg.norm(x["q"], axis=1), 1.0, atol=tol)
    np.testing.assert_allclose(np.linalg.norm(x["k"], axis=1), 1.0, atol=tol)
    if w.qkv == "bf16":
        for key in ("q", "k", "v"):
            np.testing.assert_array_equal(wl.round_to_bf16(x[key]), x[key])


def test_round_to_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20],
                    dtype=np.float32)
    out = wl.round_to_bf16(vals)
    np.testing.assert_array_equal(out, np.array([1.0, 1 + 2 ** -6, -1.0, 1 + 2 ** -7],
                                                dtype=np.float32))


def test_state_distribution():
    w = _small(2, B=4, H=8)
    S = wl.initial_state(w)
    assert S.shape == (32, 128, 128) and S.dtype == np.float32
    assert abs(S.std() - 0.02) < 2e-4 and abs(S.mean()) < 2e-4


def test_outlier_rows_and_columns():
    w = _small(4, B=2, H=3)
    S = wl.initial_state(w)
    plain = wl.initial_state(wl.custom(w, outliers=False))
    ratio = S / plain
    for h in range(w.heads):
        mask = np.isclose(ratio[h], 50.0)
        rows = np.where(mask.all(axis=1))[0]
        cols = np.where(mask.all(axis=0))[0]
        assert len(rows) == 2 and len(cols) == 2
        expect = np.zeros_like(mask)
        expect[rows, :] = True
        expect[:, cols] = True
        np.testing.assert_array_equal(mask, expect)
        np.testing.assert_array_equal(ratio[h][~mask], 1.0)


def test_sample_heads():
    w = wl.WORKLOADS[2]
    s = wl.sample_heads(w, 64)
    assert s[0] == 0 and s[-1] == w.heads - 1
    assert len(set(s.tolist())) == len(s) and len(s) <= 64
    assert np.all(np.diff(s) > 0)
