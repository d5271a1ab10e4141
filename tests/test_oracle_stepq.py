"""Pins of the STEPQuant packed-state oracle (oracle/stepq.py) against what the notes and
the mathematics fix.

The column factor is the closed-form weighted least squares the notes state (checked
against numpy's least-squares solver on the square-root-weighted system, and by
optimality: no perturbation of c_j lowers the weighted error, and the fitted factors never
do worse than the range-setting factor a_j / qmax); the row weights are omega^(1/8) (what
the notes say the exponent 0.25 amounts to) with geometric mean 1; scaling X by 4 doubles
r and c and keeps every code (the square-root row factor); hand-built ties round to even;
zero rows and zero columns give zero codes and factors; with a huge code range the packed
state reproduces X; and a decode step equals the dense step from the decoded state. A slip
such as dropping w^2 from the fit, swapping the row and column roles, or taking m_i over
the wrong axis fails at least one of them.
"""
import numpy as np
import pytest

import oracle
from oracle import stepq

RNG = np.random.default_rng(4242)


def _state(rng, d=128):
    X = rng.standard_normal((d, d)) * 0.02
    X[5, :] *= 40.0
    X[:, 9] *= 25.0
    return X


def _omega(rng, d=128):
    # log-normal row influence scores: a 90th/10th percentile ratio of about 16
    return np.exp(rng.standard_normal(d) * 1.08)


def test_row_weights_have_unit_geometric_mean_and_the_eighth_power():
    om = _omega(RNG)
    w = stepq.row_weights(om)
    assert abs(np.exp(np.mean(np.log(w))) - 1.0) < 1e-12
    ratio = w / om ** 0.125
    np.testing.assert_allclose(ratio, ratio[0], rtol=1e-12)
    np.testing.assert_allclose(stepq.row_weights(np.full(128, 3.7)), 1.0, rtol=1e-12)


def test_column_factors_are_the_weighted_least_squares_solution():
    X = _state(RNG)
    w = stepq.row_weights(_omega(RNG))
    p = stepq.pack(X, w)
    r, z = p["r"], p["z"].astype(np.float64)
    for j in (0, 9, 77):
        A = (w * r * z[:, j])[:, None]          # sqrt-weighted design column
        b = w * X[:, j]
        sol = np.linalg.lstsq(A, b, rcond=None)[0][0]
        assert abs(sol - p["c_pre"][j]) <= 1e-12 * abs(sol)
    # optimality: the fit beats the range-setting factor and every perturbation of c
    c0 = np.where(p["a"] > 0, p["a"] / stepq.QMAX4, 0.0)
    e_fit = stepq.objective(X, r, p["c_pre"], p["z"], w)
    assert e_fit <= stepq.objective(X, r, c0, p["z"], w) + 1e-18
    for eps in (1e-3, -1e-3):
        assert stepq.objective(X, r, p["c_pre"] * (1 + eps), p["z"], w) > e_fit


def test_scaling_by_four_doubles_both_factors_and_keeps_the_codes():
    X = _state(RNG)
    w = stepq.row_weights(_omega(RNG))
    p, p4 = stepq.pack(X, w), stepq.pack(4.0 * X, w)
    np.testing.assert_array_equal(p4["z"], p["z"])
    np.testing.assert_array_equal(p4["r"], 2.0 * p["r"])
    np.testing.assert_array_equal(p4["c"], 2.0 * p["c"])


def test_row_factor_follows_magnitude_over_influence():
    """r_i = fp16(sqrt(m_i / w_i)) with m_i the mean |X| over the value columns."""
    X = _state(RNG)
    om = _omega(RNG)
    p = stepq.pack(X, stepq.row_weights(om))
    m = np.abs(X).sum(axis=1) / 128.0
    ref = np.sqrt(m / stepq.row_weights(om))
    np.testing.assert_allclose(p["r_pre"], ref, rtol=1e-14)
    np.testing.assert_array_equal(p["r"], ref.astype(np.float16).astype(np.float64))
    # a heavier row gets a wider range, a more influential row a finer one
    Xh = X.copy()
    Xh[3] *= 4.0
    assert stepq.pack(Xh, stepq.row_weights(om))["r"][3] > p["r"][3]
    om2 = om.copy()
    om2[3] *= 16.0
    w2 = stepq.row_weights(om2)
    assert np.sqrt(np.mean(np.abs(X[3])) / w2[3]) < p["r_pre"][3]


def test_exact_ties_in_code_units_round_to_even():
    """Every row has mean |X| = 1 and w = 1, so r_i = 1 exactly after the fp16 rounding, and
    column 0 has range 7: the code of X_i0 is X_i0 itself, so half-integers test the
    rounding, and the clamp holds codes to [-7, 7]."""
    d = 128
    vals = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -2.5, 4.5, 5.5])
    X = np.zeros((d, d))
    X[0, 0] = 7.0
    X[1:9, 0] = vals
    for i in range(d):
        X[i, 1:] = (d - abs(X[i, 0])) / (d - 1)
    p = stepq.pack(X, np.ones(d))
    assert np.all(p["r"] == 1.0)
    assert p["a"][0] == 7.0
    np.testing.assert_array_equal(p["z"][1:9, 0], [0, 2, 2, 4, 0, -2, 4, 6])
    assert np.all(np.abs(p["z"]) <= stepq.QMAX4)


def test_zero_rows_and_columns_give_zero_codes_and_factors():
    X = _state(RNG)
    X[17, :] = 0.0
    X[:, 33] = 0.0
    p = stepq.pack(X, stepq.row_weights(_omega(RNG)))
    assert p["r"][17] == 0.0 and not p["z"][17].any()
    assert p["c"][33] == 0.0 and not p["z"][:, 33].any()
    assert np.isfinite(p["c"]).all() and np.isfinite(p["r"]).all()


def test_huge_code_range_reproduces_the_state():
    X = _state(RNG)
    w = stepq.row_weights(_omega(RNG))
    qmax = 2 ** 22
    p = stepq.pack(X, w, qmax=qmax)
    Xr = stepq.decode(p["z"], p["r"], p["c_pre"])
    np.testing.assert_allclose(Xr, X, rtol=0, atol=4.0 / qmax * np.abs(X).max())


def test_decode_step_is_the_dense_step_from_the_decoded_state():
    nh = 3
    Xs = np.stack([_state(RNG) for _ in range(nh)])
    om = np.stack([_omega(RNG) for _ in range(nh)])
    packs = [stepq.pack(Xs[h], stepq.row_weights(om[h])) for h in range(nh)]
    z = np.stack([p["z"] for p in packs])
    r = np.stack([p["r"] for p in packs])
    c = np.stack([p["c"] for p in packs])
    q = RNG.standard_normal((nh, 128))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = RNG.standard_normal((nh, 128))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = RNG.standard_normal((nh, 128))
    a = RNG.uniform(0.9, 0.999, nh)
    b = RNG.uniform(0, 1, nh)
    y, new, X1 = stepq.step(z, r, c, om, q, k, v, a, b)
    S = stepq.decode(z, r, c)
    y_ref = oracle.dense_step(S, q, k, v, a, b)
    np.testing.assert_array_equal(y, y_ref)
    np.testing.assert_array_equal(X1, S)
    # alpha = 1, beta = 0: the state is the decoded one, y its readout
    y0, _, X0 = stepq.step(z, r, c, om, q, k, v, np.ones(nh), np.zeros(nh))
    Sd = stepq.decode(z, r, c)
    np.testing.assert_allclose(y0, np.einsum("hij,hi->hj", Sd, q), rtol=0, atol=1e-14)
    np.testing.assert_array_equal(X0, Sd)


@pytest.mark.parametrize("seed", [1, 2])
def test_fit_lowers_the_weighted_error_against_per_row_scaling(seed):
    """The point of the dual-axis fit: on a state with strong rows and columns its weighted
    error is below a plain per-row absmax quantizer with the same code range."""
    rng = np.random.default_rng(seed)
    X = _state(rng)
    w = stepq.row_weights(_omega(rng))
    p = stepq.pack(X, w)
    e_dual = stepq.objective(X, p["r"], p["c"], p["z"], w)
    s = np.abs(X).max(axis=1) / 7.0
    zr = np.clip(np.rint(X / s[:, None]), -7, 7)
    e_row = float(np.sum((w ** 2)[:, None] * (X - s[:, None] * zr) ** 2))
    assert e_dual < e_row


def test_column_and_row_permutations_and_sign_are_equivariant():
    """Permuting value columns permutes codes and column factors; permuting key rows together
    with their influence scores permutes codes and row factors; negating X negates the codes.
    A row/column mix-up in the fit breaks at least one of these."""
    rng = np.random.default_rng(7)
    X = _state(rng)
    om = _omega(rng)
    w = stepq.row_weights(om)
    p = stepq.pack(X, w)
    pc = rng.permutation(128)
    q = stepq.pack(X[:, pc], w)
    np.testing.assert_array_equal(q["z"], p["z"][:, pc])
    np.testing.assert_array_equal(q["c"], p["c"][pc])
    np.testing.assert_array_equal(q["r"], p["r"])
    pr = rng.permutation(128)
    q = stepq.pack(X[pr], stepq.row_weights(om[pr]))
    np.testing.assert_array_equal(q["z"], p["z"][pr])
    np.testing.assert_array_equal(q["r"], p["r"][pr])
    np.testing.assert_allclose(q["c"], p["c"], rtol=0, atol=0)
    n = stepq.pack(-X, w)
    np.testing.assert_array_equal(n["z"], -p["z"])
    np.testing.assert_array_equal(n["r"], p["r"])
    np.testing.assert_array_equal(n["c"], p["c"])
