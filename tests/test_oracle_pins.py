"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

Each test below is chosen so that a plausible slip in the oracle -- a dropped
term, a wrong sign, the read taken from the undecayed state, a transposed
operand, an off-by-one in a cumulative decay, the readout taken before the
update, the wrong rounding rule -- fails at least one of them:

dense step (LeapQuant sec. 3.1, App. A; STEPQuant notes, Proposition 1)
  * alpha = 1, beta = 0 leaves S unchanged                     (dropped-term / wrong-gate slips)
  * unit k, alpha = beta = 1: post-update S^T k = v; with q = k, y = v
                                                               (sign, transpose, readout order)
  * equality with the Householder form (I - beta k k^T) Diag(g) S + beta k v^T
                                                               (decay before the read, transposes)
  * beta = 0: pure decay closed form prod_t Diag(g_t) S_0     (gate index)
  * KDA with d = alpha * 1 equals GDN
  * joint linearity in (S_0, v)
  * ||S_t||_F <= ||S_{t-1}||_F + beta ||k|| ||v|| (Proposition 1: ||A_t||_2 <= 1)
  * error recursion E_t = D E_{t-1} - beta k (E_{t-1}^T (g k))^T + eps_t (LeapQuant eq. 8)
quantizer: hand-built ties (round half to even), absmax maps to +-127, zero rows
window path: equals the explicit dequantize / dense steps / requantize schedule
  (eq. 4 unrolls eq. 3); the eq. 9 readout computed independently; on an exactly
  representable state (the identity-quantizer case) the first window is dense decoding;
  the per-window error stays below the per-step error (the page's trend)
log path: equals eager decoding at every step (DeltaLog eq. 7 and closure), M = 1
  reduces to eager, slot reset
tiny cases: the fp64 oracle agrees with exact rational brute force, and the
  identities hold with equality in rationals.
"""
import numpy as np
import pytest

import oracle
from oracle import exact

RNG = np.random.default_rng(12345)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(nh, dk, dv, per_key, rng, glo=0.9, ghi=0.999):
    q = _unit(rng.standard_normal((nh, dk)))
    k = _unit(rng.standard_normal((nh, dk)))
    v = rng.standard_normal((nh, dv))
    gate = rng.uniform(glo, ghi, (nh, dk) if per_key else (nh,))
    beta = rng.uniform(0, 1, nh)
    return q, k, v, gate, beta


def _gmat(gate, h, dk):
    return np.diag(gate[h]) if gate.ndim == 2 else gate[h] * np.eye(dk)


# ---------------------------------------------------------------- dense step

@pytest.mark.parametrize("per_key", [False, True])
def test_identity_gate_one_beta_zero(per_key):
    nh, dk, dv = 5, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv))
    q, k, v, _, _ = _inputs(nh, dk, dv, per_key, RNG)
    gate = np.ones((nh, dk) if per_key else nh)
    S = S0.copy()
    oracle.dense_step(S, q, k, v, gate, np.zeros(nh))
    assert np.array_equal(S, S0)


@pytest.mark.parametrize("per_key", [False, True])
def test_unit_key_writes_value_and_readout_is_post_update(per_key):
    nh, dk, dv = 6, 128, 128
    S = RNG.standard_normal((nh, dk, dv)) * 0.3
    _, k, v, _, _ = _inputs(nh, dk, dv, per_key, RNG)
    gate = np.ones((nh, dk) if per_key else nh)
    y = oracle.dense_step(S, k, k, v, gate, np.ones(nh))
    Stk = np.einsum("hij,hi->hj", S, k)
    np.testing.assert_allclose(Stk, v, rtol=0, atol=1e-12)
    # q = k: the readout of the post-update state returns v itself
    np.testing.assert_allclose(y, v, rtol=0, atol=1e-12)


@pytest.mark.parametrize("per_key", [False, True])
def test_householder_form(per_key):
    nh, dk, dv = 4, 128, 96
    S0 = RNG.standard_normal((nh, dk, dv))
    q, k, v, gate, beta = _inputs(nh, dk, dv, per_key, RNG, 0.5, 1.0)
    # make beta*||k||^2 large enough that a read from the undecayed state is visible
    S = S0.copy()
    y = oracle.dense_step(S, q, k, v, gate, beta)
    for h in range(nh):
        A = np.eye(dk) - beta[h] * np.outer(k[h], k[h])
        ref = A @ (_gmat(gate, h, dk) @ S0[h]) + beta[h] * np.outer(k[h], v[h])
        np.testing.assert_allclose(S[h], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(y[h], ref.T @ q[h], rtol=0, atol=1e-12)


@pytest.mark.parametrize("per_key", [False, True])
def test_beta_zero_is_pure_decay(per_key):
    nh, dk, dv, T = 3, 128, 128, 9
    S0 = RNG.standard_normal((nh, dk, dv))
    S = S0.copy()
    prod = np.ones((nh, dk))
    for _ in range(T):
        q, k, v, gate, _ = _inputs(nh, dk, dv, per_key, RNG)
        oracle.dense_step(S, q, k, v, gate, np.zeros(nh))
        prod *= gate if per_key else gate[:, None]
    np.testing.assert_allclose(S, prod[:, :, None] * S0, rtol=1e-13, atol=0)


def test_kda_with_uniform_gate_equals_gdn():
    nh, dk, dv, T = 4, 128, 128, 5
    S_g = RNG.standard_normal((nh, dk, dv))
    S_k = S_g.copy()
    for _ in range(T):
        q, k, v, alpha, beta = _inputs(nh, dk, dv, False, RNG)
        y_g = oracle.dense_step(S_g, q, k, v, alpha, beta)
        y_k = oracle.dense_step(S_k, q, k, v, np.repeat(alpha[:, None], dk, 1), beta)
        np.testing.assert_array_equal(y_g, y_k)
    np.testing.assert_array_equal(S_g, S_k)


@pytest.mark.parametrize("per_key", [False, True])
def test_joint_linearity_in_state_and_values(per_key):
    nh, dk, dv, T = 3, 128, 128, 6
    S0 = RNG.standard_normal((nh, dk, dv))
    steps = [_inputs(nh, dk, dv, per_key, RNG) for _ in range(T)]
    runs = {}
    for name, s_scale, v_scale in (("both", 1, 1), ("state", 1, 0), ("values", 0, 1)):
        S = S0.copy() * s_scale
        ys = [oracle.dense_step(S, q, k, v * v_scale, g, b) for (q, k, v, g, b) in steps]
        runs[name] = (S, np.array(ys))
    np.testing.assert_allclose(runs["both"][0], runs["state"][0] + runs["values"][0], atol=1e-12)
    np.testing.assert_allclose(runs["both"][1], runs["state"][1] + runs["values"][1], atol=1e-12)


@pytest.mark.parametrize("per_key", [False, True])
def test_frobenius_growth_bound(per_key):
    nh, dk, dv = 8, 128, 128
    S = RNG.standard_normal((nh, dk, dv))
    for _ in range(20):
        q, k, v, gate, beta = _inputs(nh, dk, dv, per_key, RNG, 0.8, 1.0)
        before = np.linalg.norm(S, axis=(1, 2))
        oracle.dense_step(S, q, k, v, gate, beta)
        after = np.linalg.norm(S, axis=(1, 2))
        gmax = gate.max(axis=1) if per_key else gate
        bound = gmax * before + beta * np.linalg.norm(k, axis=1) * np.linalg.norm(v, axis=1)
        assert np.all(after <= bound * (1 + 1e-12))


@pytest.mark.parametrize("per_key", [False, True])
def test_error_recursion_eq8(per_key):
    """Per-step int8 trajectory against the unquantized one (LeapQuant eq. 2, eq. 8)."""
    nh, dk, dv = 4, 128, 128
    S_ref = RNG.standard_normal((nh, dk, dv)) * 0.05
    Z, a = oracle.q8_quantize(S_ref)
    S_hat = oracle.dequant(Z, a)
    E = S_hat - S_ref
    for _ in range(6):
        q, k, v, gate, beta = _inputs(nh, dk, dv, per_key, RNG)
        oracle.dense_step(S_ref, q, k, v, gate, beta)
        X = S_hat.copy()
        oracle.dense_step(X, q, k, v, gate, beta)
        Z, a = oracle.q8_quantize(X)
        S_hat = oracle.dequant(Z, a)
        eps = S_hat - X
        gk = gate * k if per_key else gate[:, None] * k
        pred = np.empty_like(E)
        for h in range(nh):
            pred[h] = _gmat(gate, h, dk) @ E[h] - beta[h] * np.outer(k[h], E[h].T @ gk[h]) + eps[h]
        E = S_hat - S_ref
        np.testing.assert_allclose(E, pred, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- quantizer

def test_quantizer_round_half_even_ties():
    # a = 127 makes the scale exactly 1, so the codes are the values rounded
    row = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.49, -3.51, 126.5, 0.0])
    Z, a = oracle.q8_quantize(row[None, :])
    assert a[0] == np.float32(127.0)
    assert Z[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 3, -4, 126, 0]


@pytest.mark.parametrize("unit_exp", [-149, -130, -100, -71, -64, -40])
def test_quantizer_tiny_rows_keep_exact_codes(unit_exp):
    """Rows whose maximum is subnormal or tiny: values j * 2^e for every odd j in [-127, 127]
    have the exact codes j (a = 127 * 2^e), however small 2^e is. Without the exact 2^64
    rescaling of rows below 2^-64, 127 / a overflows fp32 and every code saturates."""
    j = np.arange(-127, 128, 2).astype(np.float64)
    row = j * 2.0 ** unit_exp
    row[5] = 0.0
    X = np.stack([row, np.linspace(-1.0, 1.0, 128)])
    Z, a = oracle.q8_quantize(X)
    want = j.astype(np.int64)
    want[5] = 0
    assert a[0] == np.float32(127 * 2.0 ** unit_exp)
    assert Z[0].astype(np.int64).tolist() == want.tolist()


def test_quantizer_absmax_zero_rows_and_bound():
    X = RNG.standard_normal((64, 128))
    X[3] = 0.0
    X[5, 17] = -40.0
    Z, a, w = oracle.q8_quantize(X, with_w=True)
    assert a[3] == 0 and not Z[3].any()
    assert Z[5, 17] == -127 and a[5] == np.float32(40.0)
    np.testing.assert_array_equal(a, np.abs(X.astype(np.float32)).max(axis=1))
    assert np.all(np.abs(Z) <= 127)
    for r in range(64):
        j = np.argmax(np.abs(X[r]))
        if a[r] > 0:
            assert abs(Z[r, j]) == 127
    # half-LSB bound of the dequantized value, plus the fp32 rounding of the input
    err = np.abs(oracle.dequant(Z, a) - X)
    assert np.all(err <= a[:, None] / 254.0 * (1 + 1e-6) + np.abs(X) * 2 ** -23)
    # codes are the nearest integers of the exact codes except within fp32 noise of a tie
    frac = np.abs(w - np.round(w))
    bad = (Z != np.round(w)) & (np.abs(frac - 0.5) > 1e-5)
    assert not bad.any()


# ---------------------------------------------------------------- window path

def _explicit_schedule(S0, steps, W):
    """Dequantize, run W eager dense steps, requantize (what eq. 4 unrolls)."""
    Z, a = oracle.q8_quantize(S0)
    S = oracle.dequant(Z, a)
    ys, bounds = [], []
    for t, (q, k, v, g, b) in enumerate(steps):
        ys.append(oracle.dense_step(S, q, k, v, g, b))
        if (t + 1) % W == 0:
            Z, a, w = oracle.q8_quantize(S, with_w=True)
            bounds.append((Z, a, w, S.copy()))
            S = oracle.dequant(Z, a)
    return ys, bounds


@pytest.mark.parametrize("per_key,W,T", [(False, 1, 4), (False, 3, 9), (True, 2, 6),
                                         (False, 16, 40), (True, 16, 32)])
def test_window_equals_explicit_schedule(per_key, W, T):
    nh, dk, dv = 6, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv)) * 0.02
    S0[:, 3, :] *= 50
    S0[:, :, 7] *= 50
    steps = [_inputs(nh, dk, dv, per_key, RNG) for _ in range(T)]
    ys_ref, bounds = _explicit_schedule(S0, steps, W)
    Z, a = oracle.q8_quantize(S0)
    ws = oracle.WindowState(Z, a, W, per_key)
    nb = 0
    for t, (q, k, v, g, b) in enumerate(steps):
        boundary = ws.pos == W - 1
        if boundary:
            y, Sw, w = ws.step(q, k, v, g, b, want_boundary=True)
            Zr, ar, wr, Sr = bounds[nb]
            nb += 1
            np.testing.assert_allclose(Sw, Sr, rtol=0, atol=1e-12)
            np.testing.assert_array_equal(ws.a, ar)
            # codes agree except where the exact code sits within fp64 noise of a tie
            near_tie = np.abs(np.abs(wr - np.trunc(wr)) - 0.5) < 1e-9
            assert np.all((ws.Z == Zr) | near_tie)
        else:
            y = ws.step(q, k, v, g, b)
        np.testing.assert_allclose(y, ys_ref[t], rtol=0, atol=1e-11)


@pytest.mark.parametrize("per_key", [False, True])
def test_window_readout_matches_eq9(per_key):
    """Within a window, y_l = S^_0^T Gamma_{1:l} q + sum_j u_j (k_j^T Gamma_{j+1:l} q)."""
    nh, dk, dv, W = 3, 128, 128, 8
    S0 = RNG.standard_normal((nh, dk, dv)) * 0.1
    Z, a = oracle.q8_quantize(S0)
    base = oracle.dequant(Z, a)
    ws = oracle.WindowState(Z, a, W, per_key)
    for l in range(1, W):
        q, k, v, g, b = _inputs(nh, dk, dv, per_key, RNG)
        y = ws.step(q, k, v, g, b)
        gates = ws.G[:, :l] if per_key else np.repeat(ws.G[:, :l, None], dk, 2)
        for h in range(nh):
            gam = np.prod(gates[h], axis=0)
            ref = base[h].T @ (gam * q[h])
            for j in range(l):
                gj = np.prod(gates[h, j + 1:l], axis=0)
                ref += ws.U[h, j] * (ws.K[h, j] @ (gj * q[h]))
            np.testing.assert_allclose(y[h], ref, rtol=0, atol=1e-11)


# ---------------------------------------------------------------- log path

@pytest.mark.parametrize("per_key,M", [(False, 1), (False, 2), (False, 8), (True, 4), (True, 8),
                                       (False, 64), (True, 32)])
def test_log_equals_eager(per_key, M):
    nh, dk, dv, T = 5, 128, 128, 3 * M + 2
    S0 = RNG.standard_normal((nh, dk, dv)) * 0.02
    S_eager = S0.copy()
    ls = oracle.LogState(S0, M - 1, per_key)
    for t in range(T):
        q, k, v, g, b = _inputs(nh, dk, dv, per_key, RNG)
        y_e = oracle.dense_step(S_eager, q, k, v, g, b)
        y_l = ls.step(q, k, v, g, b)
        np.testing.assert_allclose(y_l, y_e, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ls.logical_state(), S_eager, rtol=0, atol=1e-12)
        if ls.L == 0:
            # right after a merge: the base alone is the state, and lbar is reset
            np.testing.assert_allclose(ls.Sbar, S_eager, rtol=0, atol=1e-12)
            assert not ls.lbar.any()


@pytest.mark.parametrize("per_key", [False, True])
def test_log_slots_equal_eager(per_key):
    """Per-slot live lengths (DeltaLog sec. 4: one live length per request slot): every
    head sits at its own point of its append/merge cycle, merges at its own steps, and
    still decodes exactly like eager dense updates (eq. 7 at every step)."""
    nh, dk, dv, C = 6, 128, 128, 4
    S0 = RNG.standard_normal((nh, dk, dv)) * 0.02
    S_eager = S0.copy()
    ls = oracle.LogState(S0, C, per_key)
    # empty entries (K = U = 0) are a valid log of any length: each head starts elsewhere
    Ls = np.array([0, 1, 2, 3, 4, 4], dtype=np.int32)
    merged = np.zeros(nh, dtype=int)
    for t in range(2 * C + 3):
        q, k, v, g, b = _inputs(nh, dk, dv, per_key, RNG)
        was_full = Ls == C
        y_e = oracle.dense_step(S_eager, q, k, v, g, b)
        y_l = ls.step_slots(Ls, q, k, v, g, b)
        np.testing.assert_allclose(y_l, y_e, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(Ls[was_full], 0)
        merged += was_full
        for h in np.flatnonzero(was_full):
            # right after its merge, a head's base alone is its state
            np.testing.assert_allclose(ls.Sbar[h], S_eager[h], rtol=0, atol=1e-12)
    assert (merged >= 2).all()
    with pytest.raises(ValueError):
        ls.step_slots(np.array([0, 1, 2, 3, 4, 5], dtype=np.int32), q, k, v, g, b)


def test_log_slot_reset_leaves_base():
    nh, dk, dv = 2, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv))
    ls = oracle.LogState(S0, 7, False)
    for _ in range(3):
        ls.step(*_inputs(nh, dk, dv, False, RNG))
    # slot reuse resets only the auxiliary buffers: the logical state is then the base
    ls.lbar[:] = 0
    ls.L = 0
    np.testing.assert_array_equal(ls.logical_state(), ls.Sbar)
    np.testing.assert_array_equal(ls.Sbar, S0)


# ---------------------------------------------------------------- tiny exact cases

def _tiny_steps(rng, T, dk, dv, per_key):
    out = []
    for _ in range(T):
        q = rng.standard_normal(dk)
        k = rng.standard_normal(dk)
        k = k / np.linalg.norm(k)
        v = rng.standard_normal(dv)
        g = rng.uniform(0.8, 1.0, dk) if per_key else np.full(dk, rng.uniform(0.8, 1.0))
        b = rng.uniform(0, 1)
        out.append((q, k, v, g, b))
    return out


def _frac_steps(steps):
    from fractions import Fraction as Fr
    return [(exact.frac_vec(q), exact.frac_vec(k), exact.frac_vec(v), exact.frac_vec(g),
             Fr(float(b))) for (q, k, v, g, b) in steps]


@pytest.mark.parametrize("per_key", [False, True])
def test_exact_householder_and_oracle_agreement(per_key):
    rng = np.random.default_rng(3)
    dk, dv = 4, 3
    S0 = rng.standard_normal((dk, dv))
    steps = _tiny_steps(rng, 5, dk, dv, per_key)
    fs = _frac_steps(steps)
    Sx = exact.frac_mat(S0)
    S64 = S0[None].copy()
    for (q, k, v, g, b), (fq, fk, fv, fg, fb) in zip(steps, fs):
        H = exact.householder_step(Sx, fk, fv, fg, fb)
        Sx, yx = exact.dense_step(Sx, fq, fk, fv, fg, fb)
        assert H == Sx
        gate = g[None] if per_key else np.array([g[0]])
        y64 = oracle.dense_step(S64, q[None], k[None], v[None], gate, np.array([b]))
        np.testing.assert_allclose(S64[0], np.array(Sx, dtype=float), rtol=0, atol=1e-13)
        np.testing.assert_allclose(y64[0], np.array(yx, dtype=float), rtol=0, atol=1e-13)


@pytest.mark.parametrize("W,T", [(1, 4), (2, 6), (3, 6)])
def test_exact_window_unrolling(W, T):
    rng = np.random.default_rng(10 + W)
    dk, dv = 4, 4
    S0 = exact.frac_mat(rng.standard_normal((dk, dv)))
    fs = _frac_steps(_tiny_steps(rng, T, dk, dv, True))
    assert exact.window_run(S0, fs, W) == exact.explicit_schedule_run(S0, fs, W)


@pytest.mark.parametrize("M", [1, 2, 3])
def test_exact_log_equals_eager(M):
    rng = np.random.default_rng(20 + M)
    dk, dv = 4, 3
    S0 = exact.frac_mat(rng.standard_normal((dk, dv)))
    fs = _frac_steps(_tiny_steps(rng, 7, dk, dv, True))
    ys_l, st_l = exact.log_run(S0, fs, M)
    ys_e, st_e = exact.eager_run(S0, fs)
    assert ys_l == ys_e and st_l == st_e


def test_exact_window_matches_fp64_window_oracle():
    rng = np.random.default_rng(31)
    dk, dv, W, T = 4, 4, 3, 6
    S0 = rng.standard_normal((dk, dv))
    steps = _tiny_steps(rng, T, dk, dv, False)
    ys_x, bounds_x = exact.window_run(exact.frac_mat(S0), _frac_steps(steps), W)
    Z, a = oracle.q8_quantize(S0[None])
    ws = oracle.WindowState(Z, a, W, False)
    nb = 0
    for t, (q, k, v, g, b) in enumerate(steps):
        y = ws.step(q[None], k[None], v[None], np.array([g[0]]), np.array([b]))
        # the fp64 path stores the row scale in fp32; the exact one keeps it rational
        np.testing.assert_allclose(y[0], np.array(ys_x[t], dtype=float), rtol=1e-6, atol=1e-7)
        if ws.pos == 0:
            Zx, ax = bounds_x[nb]
            nb += 1
            np.testing.assert_array_equal(ws.Z[0], np.array(Zx))
            np.testing.assert_allclose(ws.a[0], np.array(ax, dtype=float), rtol=1e-7)


@pytest.mark.parametrize("per_key", [False, True])
def test_window_with_an_exactly_representable_state_is_dense(per_key):
    """The identity-quantizer case: rows whose absmax is 127 * 2^e and whose entries are
    integer multiples of 2^e quantize exactly (the scale 127 / a = 2^-e is exact), so until
    the first requantization the window path must reproduce dense decoding from S_0. A slip
    in the readout's scale (/128 for /127, the scale applied twice, a wrong row) breaks it."""
    rng = np.random.default_rng(31)
    nh, dk, dv, W = 4, 128, 128, 8
    codes = rng.integers(-127, 128, size=(nh, dk, dv)).astype(np.float64)
    codes[:, :, 0] = np.where(rng.random((nh, dk)) < 0.5, 127.0, -127.0)   # absmax 127 in every row
    e = rng.integers(-12, -4, size=(nh, dk, 1)).astype(np.float64)
    S0 = codes * 2.0 ** e
    Z, a = oracle.q8_quantize(S0)
    np.testing.assert_array_equal(Z.astype(np.float64), codes)
    np.testing.assert_array_equal(oracle.dequant(Z, a), S0)
    ws = oracle.WindowState(Z, a, W, per_key)
    S = S0.copy()
    for _ in range(W - 1):
        q, k, v, g, b = _inputs(nh, dk, dv, per_key, rng)
        y_w = ws.step(q, k, v, g, b)
        y_d = oracle.dense_step(S, q, k, v, g, b)
        np.testing.assert_allclose(y_w, y_d, rtol=0, atol=1e-12 * np.abs(y_d).max())


def test_window_error_is_below_per_step_error():
    """LeapQuant's point about windows: against the fp32-exact trajectory, quantizing once per
    window of 16 leaves less output error than quantizing after every step (W = 1), because
    rounding enters 16 times less often. A trend the page reports, checked on one seeded run."""
    rng = np.random.default_rng(8)
    nh, dk, dv, T = 6, 128, 128, 64
    S0 = rng.standard_normal((nh, dk, dv)) * 0.02
    S0[:, 3, :] *= 50
    steps = [_inputs(nh, dk, dv, False, rng) for _ in range(T)]
    S = S0.copy()
    ref = [oracle.dense_step(S, *x) for x in steps]
    err = {}
    for W in (1, 16):
        Z, a = oracle.q8_quantize(S0)
        ws = oracle.WindowState(Z, a, W, False)
        e = [np.linalg.norm(ws.step(*x) - r) / np.linalg.norm(r) for x, r in zip(steps, ref)]
        err[W] = float(np.mean(e))
    assert err[16] < err[1]
