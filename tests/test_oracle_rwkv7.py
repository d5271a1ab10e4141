"""Pins of the RWKV7 oracle against what the pages and the mathematics fix.

LeapQuant App. A writes RWKV7's transition Diag(w) - kappa (a * kappa)^T as two sub-steps of
eq. 1: an erase along kappa with v = 0 and read vector a * kappa, then a pure write k v^T.
Pins: the product form of the transition (written as a matrix, numpy), the reduction to
the RWKV6 step at a = 0, an exact substitution onto the (separately pinned) KDA step
(kappa = k, a = beta d, v -> beta v gives (I - beta k k^T) Diag(d) S + beta k v^T), the
erase removing the kappa direction completely at w = 1, a = 1, joint linearity, and exact
rational brute force. A slip such as reading the erase from the decayed state, dropping
the erase rate or swapping the order of the two sub-steps fails at least one of them.

On the per-window int8 representation each token is two records (App. A: the same
treatment as a DeltaProduct token with n = 2): gates w and 1, keys kappa and k, values
-S^T (a * kappa) and v. Pins: the window equals the explicit dequantize / dense steps /
requantize schedule (fp64 for W in {1, 2, 3, 16}, and with equality in exact rationals),
and a = 0 leaves erase records that only decay (the single-record RWKV6 readout).
"""
import numpy as np
import pytest

import oracle
from oracle import exact

RNG = np.random.default_rng(7070)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(nh, dk, dv, rng):
    q = _unit(rng.standard_normal((nh, dk)))
    k = _unit(rng.standard_normal((nh, dk)))
    v = rng.standard_normal((nh, dv))
    w = rng.uniform(0.8, 1.0, (nh, dk))
    kappa = _unit(rng.standard_normal((nh, dk)))
    a = rng.uniform(0.0, 1.0, (nh, dk))
    return q, k, v, w, kappa, a


def test_transition_product_form():
    nh, dk, dv = 3, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv))
    q, k, v, w, kappa, a = _inputs(nh, dk, dv, RNG)
    S = S0.copy()
    y = oracle.rwkv7_step(S, q, k, v, w, kappa, a)
    for h in range(nh):
        T = np.diag(w[h]) - np.outer(kappa[h], a[h] * kappa[h])
        ref = T @ S0[h] + np.outer(k[h], v[h])
        np.testing.assert_allclose(S[h], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(y[h], ref.T @ q[h], rtol=0, atol=1e-12)


def test_zero_erase_rate_is_the_rwkv6_step():
    nh, dk, dv = 2, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv))
    q, k, v, w, kappa, _ = _inputs(nh, dk, dv, RNG)
    S7, S6 = S0.copy(), S0.copy()
    y7 = oracle.rwkv7_step(S7, q, k, v, w, kappa, np.zeros((nh, dk)))
    y6 = oracle.rwkv6_step(S6, q, k, v, w)
    np.testing.assert_array_equal(S7, S6)
    np.testing.assert_array_equal(y7, y6)


def test_substitution_onto_the_kda_step():
    """kappa = k, a = beta d, w = d and v -> beta v: Diag(d) S - k (beta d * k)^T S + beta k v^T,
    which is the KDA step (I - beta k k^T) Diag(d) S + beta k v^T."""
    nh, dk, dv = 3, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv)) * 0.02
    q, k, v, d, _, _ = _inputs(nh, dk, dv, RNG)
    beta = RNG.uniform(0, 1, nh)
    S7, Sk = S0.copy(), S0.copy()
    y7 = oracle.rwkv7_step(S7, q, k, beta[:, None] * v, d, k, beta[:, None] * d)
    yk = oracle.dense_step(Sk, q, k, v, d, beta)
    np.testing.assert_allclose(S7, Sk, rtol=0, atol=1e-13)
    np.testing.assert_allclose(y7, yk, rtol=0, atol=1e-13)


def test_full_erase_removes_the_kappa_direction():
    """w = 1, a = 1 and unit kappa: the erase is the projection I - kappa kappa^T, so with
    no write kappa^T S = 0 afterwards, and a second erase changes nothing."""
    nh, dk, dv = 2, 128, 128
    S = RNG.standard_normal((nh, dk, dv))
    q, _, _, _, kappa, _ = _inputs(nh, dk, dv, RNG)
    ones, zk, zv = np.ones((nh, dk)), np.zeros((nh, dk)), np.zeros((nh, dv))
    oracle.rwkv7_step(S, q, zk, zv, ones, kappa, ones)
    assert np.abs(np.einsum("hij,hi->hj", S, kappa)).max() < 1e-12
    S2 = S.copy()
    oracle.rwkv7_step(S2, q, zk, zv, ones, kappa, ones)
    np.testing.assert_allclose(S2, S, rtol=0, atol=1e-12)


def test_joint_linearity_in_state_and_values():
    nh, dk, dv = 2, 128, 128
    q, k, v1, w, kappa, a = _inputs(nh, dk, dv, RNG)
    v2 = RNG.standard_normal((nh, dv))
    S1, S2 = RNG.standard_normal((2, nh, dk, dv))
    c1, c2 = 0.6, -1.7
    Sa, Sb, Sc = S1.copy(), S2.copy(), c1 * S1 + c2 * S2
    ya = oracle.rwkv7_step(Sa, q, k, v1, w, kappa, a)
    yb = oracle.rwkv7_step(Sb, q, k, v2, w, kappa, a)
    yc = oracle.rwkv7_step(Sc, q, k, c1 * v1 + c2 * v2, w, kappa, a)
    np.testing.assert_allclose(Sc, c1 * Sa + c2 * Sb, rtol=0, atol=1e-12)
    np.testing.assert_allclose(yc, c1 * ya + c2 * yb, rtol=0, atol=1e-12)


def test_exact_rationals_match_the_fp64_oracle():
    rng = np.random.default_rng(71)
    dk, dv = 4, 3
    S0 = rng.standard_normal((dk, dv))
    Sx, S64 = exact.frac_mat(S0), S0[None].copy()
    for _ in range(5):
        q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
        w, kappa, a = rng.uniform(0.8, 1, dk), rng.standard_normal(dk), rng.uniform(0, 1, dk)
        Sx, yx = exact.rwkv7_step(Sx, *(exact.frac_vec(x) for x in (q, k, v, w, kappa, a)))
        y64 = oracle.rwkv7_step(S64, q[None], k[None], v[None], w[None], kappa[None], a[None])
        np.testing.assert_allclose(S64[0], np.array(Sx, dtype=float), rtol=0, atol=1e-13)
        np.testing.assert_allclose(y64[0], np.array(yx, dtype=float), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- two records per token

def _explicit_schedule(S0, steps, W):
    """Dequantize, run W dense RWKV7 steps, requantize (what eq. 4 over 2W records unrolls)."""
    Z, a = oracle.q8_quantize(S0)
    S = oracle.dequant(Z, a)
    ys, bounds = [], []
    for t, st in enumerate(steps):
        ys.append(oracle.rwkv7_step(S, *st))
        if (t + 1) % W == 0:
            Z, a, w = oracle.q8_quantize(S, with_w=True)
            bounds.append((Z, a, w, S.copy()))
            S = oracle.dequant(Z, a)
    return ys, bounds


@pytest.mark.parametrize("W,T", [(1, 4), (2, 6), (3, 9), (16, 40)])
def test_window_with_two_records_per_token_equals_explicit_schedule(W, T):
    nh, dk, dv = 5, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv)) * 0.02
    S0[:, 5, :] *= 50
    S0[:, :, 9] *= 50
    steps = [_inputs(nh, dk, dv, RNG) for _ in range(T)]
    ys_ref, bounds = _explicit_schedule(S0, steps, W)
    Z, a = oracle.q8_quantize(S0)
    ws = oracle.Rwkv7WindowState(Z, a, W)
    nb = 0
    for t, st in enumerate(steps):
        if ws.pos == W - 1:
            y, Sw, w = ws.step(*st, want_boundary=True)
            Zr, ar, wr, Sr = bounds[nb]
            nb += 1
            np.testing.assert_allclose(Sw, Sr, rtol=0, atol=1e-12)
            np.testing.assert_array_equal(ws.a, ar)
            near_tie = np.abs(np.abs(wr - np.trunc(wr)) - 0.5) < 1e-9
            assert np.all((ws.Z == Zr) | near_tie)
        else:
            y = ws.step(*st)
            # the token's two records: (w, kappa, -S^T (a kappa)) and (1, k, v)
            p = ws.pos - 1
            np.testing.assert_array_equal(ws.G[:, 2 * p], st[3])
            np.testing.assert_array_equal(ws.K[:, 2 * p], st[4])
            np.testing.assert_array_equal(ws.G[:, 2 * p + 1], 1.0)
            np.testing.assert_array_equal(ws.K[:, 2 * p + 1], st[1])
            np.testing.assert_array_equal(ws.U[:, 2 * p + 1], st[2])
        np.testing.assert_allclose(y, ys_ref[t], rtol=0, atol=1e-11)


def test_window_with_zero_erase_rate_has_pure_decay_erase_records():
    """a = 0: every erase record carries u = 0, so it only decays (the single-record
    RWKV6 form inside the window)."""
    nh, dk, dv, W = 3, 128, 128, 4
    S0 = RNG.standard_normal((nh, dk, dv)) * 0.02
    Z, a = oracle.q8_quantize(S0)
    ws = oracle.Rwkv7WindowState(Z, a, W)
    S = oracle.dequant(Z, a)
    for _ in range(W - 1):
        q, k, v, w, kappa, _ = _inputs(nh, dk, dv, RNG)
        y = ws.step(q, k, v, w, kappa, np.zeros((nh, dk)))
        y6 = oracle.rwkv6_step(S, q, k, v, w)
        np.testing.assert_allclose(y, y6, rtol=0, atol=1e-12)
        assert not ws.U[:, 2 * (ws.pos - 1)].any()


@pytest.mark.parametrize("W,T", [(1, 3), (2, 4), (3, 6)])
def test_exact_window_with_two_records_equals_explicit_schedule(W, T):
    rng = np.random.default_rng(90 + W)
    dk, dv = 4, 3
    S0 = exact.frac_mat(rng.standard_normal((dk, dv)))
    fs = []
    for _ in range(T):
        q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
        w, kappa, er = rng.uniform(0.8, 1, dk), rng.standard_normal(dk), rng.uniform(0, 1, dk)
        fs.append(tuple(exact.frac_vec(x) for x in (q, k, v, w, kappa, er)))
    assert exact.rwkv7_window_run(S0, fs, W) == exact.rwkv7_explicit_run(S0, fs, W)
