"""Pins of the DeltaProduct oracle against what the pages and the mathematics fix.

LeapQuant App. A (Table 4) lists DeltaProduct as n delta-rule sub-steps of eq. 1 per token.
The reading built here: each sub-step i has its own key k_i, value v_i and strength beta_i;
the token's scalar gate alpha decays the state once, in the first sub-step; the output is
read after the last sub-step. Pins: the token equals the product of generalized Householder
transforms written as matrices (numpy); n = 1 is the (separately pinned) GDN step; n = 2
with alpha = 1 on the second sub-step is two chained GDN steps; unit keys with beta = 1
make the last sub-step's key read back its value exactly; exact rational brute force.
A slip such as decaying every sub-step, reading the second sub-step from the state before
the first write or dropping a beta fails at least one of them.

On the per-window int8 representation each sub-step is one record (LeapQuant sec. 3.2 with
App. A: "the same treatment as a DeltaProduct token with n = 2"): gates alpha, 1, ..., 1.
Pins: the window equals the explicit dequantize / tokens / requantize schedule (fp64 for
several W and n, and with equality in exact rationals), and a state the quantizer
represents exactly gives dense DeltaProduct decoding through the first window.
"""
import numpy as np
import pytest

import oracle
from oracle import exact

RNG = np.random.default_rng(5150)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(nh, n, dk, dv, rng):
    q = _unit(rng.standard_normal((nh, dk)))
    k = _unit(rng.standard_normal((nh, n, dk)))
    v = rng.standard_normal((nh, n, dv))
    alpha = rng.uniform(0.9, 0.999, nh)
    beta = rng.uniform(0.0, 1.0, (nh, n))
    return q, k, v, alpha, beta


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_token_is_a_product_of_householder_transforms(n):
    nh, dk, dv = 3, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv))
    q, k, v, alpha, beta = _inputs(nh, n, dk, dv, RNG)
    S = S0.copy()
    y = oracle.deltaproduct_step(S, q, k, v, alpha, beta)
    I = np.eye(dk)
    for h in range(nh):
        ref = alpha[h] * S0[h]
        for i in range(n):
            ref = (I - beta[h, i] * np.outer(k[h, i], k[h, i])) @ ref + beta[h, i] * np.outer(k[h, i], v[h, i])
        np.testing.assert_allclose(S[h], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(y[h], ref.T @ q[h], rtol=0, atol=1e-12)


def test_one_sub_step_is_the_gdn_step():
    nh, dk, dv = 4, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv))
    q, k, v, alpha, beta = _inputs(nh, 1, dk, dv, RNG)
    Sa, Sb = S0.copy(), S0.copy()
    ya = oracle.deltaproduct_step(Sa, q, k, v, alpha, beta)
    yb = oracle.dense_step(Sb, q, k[:, 0], v[:, 0], alpha, beta[:, 0])
    np.testing.assert_array_equal(Sa, Sb)
    np.testing.assert_array_equal(ya, yb)


def test_two_sub_steps_are_two_chained_gdn_steps():
    nh, dk, dv = 4, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv))
    q, k, v, alpha, beta = _inputs(nh, 2, dk, dv, RNG)
    Sa, Sb = S0.copy(), S0.copy()
    ya = oracle.deltaproduct_step(Sa, q, k, v, alpha, beta)
    oracle.dense_step(Sb, q, k[:, 0], v[:, 0], alpha, beta[:, 0])
    yb = oracle.dense_step(Sb, q, k[:, 1], v[:, 1], np.ones(nh), beta[:, 1])
    np.testing.assert_allclose(Sa, Sb, rtol=0, atol=1e-13)
    np.testing.assert_allclose(ya, yb, rtol=0, atol=1e-13)


def test_last_key_reads_back_its_value():
    """Unit keys and beta = 1 in the last sub-step: after the token S^T k_n = v_n (the
    delta rule's exact write along its key, whatever came before)."""
    nh, dk, dv, n = 3, 128, 128, 3
    S = RNG.standard_normal((nh, dk, dv))
    q, k, v, alpha, beta = _inputs(nh, n, dk, dv, RNG)
    beta[:, -1] = 1.0
    oracle.deltaproduct_step(S, q, k, v, alpha, beta)
    got = np.einsum("hij,hi->hj", S, k[:, -1])
    np.testing.assert_allclose(got, v[:, -1], rtol=0, atol=1e-12)


def test_exact_rationals_match_the_fp64_oracle():
    rng = np.random.default_rng(515)
    dk, dv, n = 4, 3, 2
    S0 = rng.standard_normal((dk, dv))
    Sx, S64 = exact.frac_mat(S0), S0[None].copy()
    for _ in range(4):
        q = rng.standard_normal(dk)
        k = rng.standard_normal((n, dk))
        v = rng.standard_normal((n, dv))
        alpha, beta = rng.uniform(0.8, 1), rng.uniform(0, 1, n)
        Sx = exact.deltaproduct_householder(Sx, [exact.frac_vec(x) for x in k], [exact.frac_vec(x) for x in v],
                                            exact.F(float(alpha)), [exact.F(float(b)) for b in beta])
        yx = [sum(Sx[i][j] * exact.F(float(q[i])) for i in range(dk)) for j in range(dv)]
        y64 = oracle.deltaproduct_step(S64, q[None], k[None], v[None], np.array([alpha]), beta[None])
        np.testing.assert_allclose(S64[0], np.array(Sx, dtype=float), rtol=0, atol=1e-13)
        np.testing.assert_allclose(y64[0], np.array(yx, dtype=float), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- one record per sub-step

def _explicit_schedule(S0, steps, W):
    """Dequantize, run W dense DeltaProduct tokens, requantize (what eq. 4 over nW records unrolls)."""
    Z, a = oracle.q8_quantize(S0)
    S = oracle.dequant(Z, a)
    ys, bounds = [], []
    for t, st in enumerate(steps):
        ys.append(oracle.deltaproduct_step(S, *st))
        if (t + 1) % W == 0:
            Z, a, w = oracle.q8_quantize(S, with_w=True)
            bounds.append((Z, a, w, S.copy()))
            S = oracle.dequant(Z, a)
    return ys, bounds


@pytest.mark.parametrize("n,W,T", [(2, 1, 4), (2, 2, 6), (2, 3, 9), (2, 16, 40), (3, 5, 12), (1, 4, 9)])
def test_window_with_one_record_per_sub_step_equals_explicit_schedule(n, W, T):
    nh, dk, dv = 5, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv)) * 0.02
    S0[:, 5, :] *= 50
    S0[:, :, 9] *= 50
    steps = [_inputs(nh, n, dk, dv, RNG) for _ in range(T)]
    ys_ref, bounds = _explicit_schedule(S0, steps, W)
    Z, a = oracle.q8_quantize(S0)
    ws = oracle.DeltaProductWindowState(Z, a, W, n)
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
            p = ws.pos - 1                                   # the token's records: gates alpha, 1, ..
            np.testing.assert_array_equal(ws.G[:, n * p], st[3])
            for i in range(1, n):
                np.testing.assert_array_equal(ws.G[:, n * p + i], 1.0)
            for i in range(n):
                np.testing.assert_array_equal(ws.K[:, n * p + i], st[1][:, i])
        np.testing.assert_allclose(y, ys_ref[t], rtol=0, atol=1e-11)


def test_window_from_an_exactly_quantized_state_is_dense_decoding():
    """Row absmax 127 * 2^-8 and entries multiples of 2^-8: the quantizer represents the
    state exactly, so through the first window the int8 path is dense DeltaProduct decoding."""
    nh, dk, dv, n, W = 3, 128, 128, 2, 6
    Zi = RNG.integers(-127, 128, (nh, dk, dv))
    Zi[:, :, 0] = 127
    S0 = Zi * 2.0 ** -8
    Z, a = oracle.q8_quantize(S0)
    np.testing.assert_array_equal(oracle.dequant(Z, a), S0)
    ws = oracle.DeltaProductWindowState(Z, a, W, n)
    S = S0.copy()
    for _ in range(W - 1):
        st = _inputs(nh, n, dk, dv, RNG)
        np.testing.assert_allclose(ws.step(*st), oracle.deltaproduct_step(S, *st), rtol=0, atol=1e-11)


@pytest.mark.parametrize("W,T", [(1, 3), (2, 4), (3, 6)])
def test_exact_window_with_sub_step_records_equals_explicit_schedule(W, T):
    rng = np.random.default_rng(60 + W)
    dk, dv, n = 4, 3, 2
    S0 = exact.frac_mat(rng.standard_normal((dk, dv)))
    fs = []
    for _ in range(T):
        q = exact.frac_vec(rng.standard_normal(dk))
        ks = [exact.frac_vec(x) for x in rng.standard_normal((n, dk))]
        vs = [exact.frac_vec(x) for x in rng.standard_normal((n, dv))]
        fs.append((q, ks, vs, exact.F(float(rng.uniform(0.8, 1))), [exact.F(float(b)) for b in rng.uniform(0, 1, n)]))
    assert exact.deltaproduct_window_run(S0, fs, W) == exact.deltaproduct_explicit_run(S0, fs, W)
