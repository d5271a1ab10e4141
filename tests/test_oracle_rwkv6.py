"""Pins of the RWKV6 oracle (dense step and base + log) against what the pages and the
mathematics fix.

The update is the pages' common form without the delta read (DeltaLog Table 1, the RWKV6
row: state transform D(lambda) S, update pair (k, v), per-key decay; LeapQuant App. A
eq. 1 with read vector b = 0 and output S_t^T q_t). Each pin below fails on a plausible
slip: a decay applied to the written pair or on the value side (zero-key and no-decay
closed forms), a stray correction term (equality with the KDA step on a state whose
columns are orthogonal to the decayed key, where the delta read vanishes), a transposed
write (linear attention closed form), and in the log path a decay snapshot taken at the
wrong time (log = eager at every step, also in exact rationals).
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import exact

RNG = np.random.default_rng(6060)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(nh, dk, dv, rng, lo=0.8, hi=1.0):
    q = _unit(rng.standard_normal((nh, dk)))
    k = _unit(rng.standard_normal((nh, dk)))
    v = rng.standard_normal((nh, dv))
    w = rng.uniform(lo, hi, (nh, dk))
    return q, k, v, w


def test_no_decay_from_zero_is_linear_attention():
    """w = 1 and S_0 = 0: S_T = sum_t k_t v_t^T = K^T V, and y_t reads S_t."""
    nh, dk, dv, T = 3, 128, 128, 6
    S = np.zeros((nh, dk, dv))
    Ks, Vs = [], []
    for _ in range(T):
        q, k, v, _ = _inputs(nh, dk, dv, RNG)
        y = oracle.rwkv6_step(S, q, k, v, np.ones((nh, dk)))
        Ks.append(k)
        Vs.append(v)
        Kt, Vt = np.stack(Ks, 1), np.stack(Vs, 1)              # [nh, t, dk], [nh, t, dv]
        ref = np.matmul(Kt.transpose(0, 2, 1), Vt)
        np.testing.assert_allclose(S, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(y, np.matmul(q[:, None, :], ref)[:, 0], rtol=0, atol=1e-12)


def test_zero_key_is_pure_decay_on_the_key_rows():
    nh, dk, dv = 2, 128, 128
    S0 = RNG.standard_normal((nh, dk, dv))
    S = S0.copy()
    prod = np.ones((nh, dk))
    for _ in range(4):
        q, _, v, w = _inputs(nh, dk, dv, RNG)
        y = oracle.rwkv6_step(S, q, np.zeros((nh, dk)), v, w)
        prod *= w
        ref = prod[:, :, None] * S0
        np.testing.assert_allclose(S, ref, rtol=1e-13, atol=0)
        np.testing.assert_allclose(y, np.einsum("hij,hi->hj", ref, q), rtol=1e-12, atol=1e-14)


def test_equals_kda_with_beta_one_when_the_delta_read_vanishes():
    """The KDA step is Diag(d) S + k (beta (v - S^T (d k)))^T; on a state whose columns
    are orthogonal to d k the read is zero, and with beta = 1 it is the RWKV6 step."""
    nh, dk, dv = 3, 128, 128
    q, k, v, w = _inputs(nh, dk, dv, RNG)
    R = RNG.standard_normal((nh, dk, dv))
    x = w * k
    P = np.eye(dk)[None] - x[:, :, None] * x[:, None, :] / np.sum(x * x, 1)[:, None, None]
    S = np.matmul(P, R)
    assert np.abs(np.einsum("hij,hi->hj", S, x)).max() < 1e-12
    S_kda, S_rw = S.copy(), S.copy()
    y_kda = oracle.dense_step(S_kda, q, k, v, w, np.ones(nh))
    y_rw = oracle.rwkv6_step(S_rw, q, k, v, w)
    np.testing.assert_allclose(S_rw, S_kda, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y_rw, y_kda, rtol=0, atol=1e-12)


def test_joint_linearity_in_state_and_values():
    nh, dk, dv = 2, 128, 128
    q, k, v1, w = _inputs(nh, dk, dv, RNG)
    v2 = RNG.standard_normal((nh, dv))
    S1, S2 = RNG.standard_normal((2, nh, dk, dv))
    a, b = 0.7, -1.3
    Sa, Sb, Sc = S1.copy(), S2.copy(), a * S1 + b * S2
    ya = oracle.rwkv6_step(Sa, q, k, v1, w)
    yb = oracle.rwkv6_step(Sb, q, k, v2, w)
    yc = oracle.rwkv6_step(Sc, q, k, a * v1 + b * v2, w)
    np.testing.assert_allclose(Sc, a * Sa + b * Sb, rtol=0, atol=1e-12)
    np.testing.assert_allclose(yc, a * ya + b * yb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("M", [1, 2, 4, 8, 64])
def test_log_equals_eager(M):
    nh, dk, dv, T = 4, 128, 128, 3 * M + 2
    S0 = RNG.standard_normal((nh, dk, dv)) * 0.02
    S_eager = S0.copy()
    ls = oracle.LogState(S0, M - 1, True, rwkv6=True)
    for _ in range(T):
        q, k, v, w = _inputs(nh, dk, dv, RNG)
        y_e = oracle.rwkv6_step(S_eager, q, k, v, w)
        y_l = ls.step(q, k, v, w)
        np.testing.assert_allclose(y_l, y_e, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ls.logical_state(), S_eager, rtol=0, atol=1e-12)
        if ls.L == 0:
            np.testing.assert_allclose(ls.Sbar, S_eager, rtol=0, atol=1e-12)
            assert not ls.lbar.any()
        else:
            # the value-side factor of the newest entry is the raw value
            np.testing.assert_array_equal(ls.U[:, ls.L - 1], v)


def test_log_slots_equal_eager():
    nh, dk, dv, C = 5, 128, 128, 3
    S0 = RNG.standard_normal((nh, dk, dv)) * 0.02
    S_eager = S0.copy()
    ls = oracle.LogState(S0, C, True, rwkv6=True)
    Ls = np.array([0, 1, 2, 3, 3], dtype=np.int32)
    merged = np.zeros(nh, dtype=int)
    for _ in range(2 * C + 3):
        q, k, v, w = _inputs(nh, dk, dv, RNG)
        was_full = Ls == C
        y_e = oracle.rwkv6_step(S_eager, q, k, v, w)
        y_l = ls.step_slots(Ls, q, k, v, w)
        np.testing.assert_allclose(y_l, y_e, rtol=0, atol=1e-12)
        merged += was_full
        for h in np.flatnonzero(was_full):
            np.testing.assert_allclose(ls.Sbar[h], S_eager[h], rtol=0, atol=1e-12)
    assert (merged >= 2).all()


def _tiny(rng, T, dk, dv):
    out = []
    for _ in range(T):
        out.append((rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv),
                    rng.uniform(0.8, 1.0, dk)))
    return out


def _frac(steps):
    return [(exact.frac_vec(q), exact.frac_vec(k), exact.frac_vec(v), exact.frac_vec(w), Fr(0))
            for (q, k, v, w) in steps]


@pytest.mark.parametrize("M", [1, 2, 3])
def test_exact_log_equals_eager(M):
    rng = np.random.default_rng(70 + M)
    dk, dv = 4, 3
    S0 = exact.frac_mat(rng.standard_normal((dk, dv)))
    fs = _frac(_tiny(rng, 7, dk, dv))
    assert exact.log_run(S0, fs, M, delta=False) == exact.eager_run(S0, fs, delta=False)


def test_exact_matches_fp64_oracle():
    rng = np.random.default_rng(77)
    dk, dv = 4, 3
    S0 = rng.standard_normal((dk, dv))
    steps = _tiny(rng, 6, dk, dv)
    Sx, S64 = exact.frac_mat(S0), S0[None].copy()
    ls = oracle.LogState(S0[None], 2, True, rwkv6=True)
    for (q, k, v, w), (fq, fk, fv, fw, _) in zip(steps, _frac(steps)):
        Sx, yx = exact.rwkv6_step(Sx, fq, fk, fv, fw)
        y64 = oracle.rwkv6_step(S64, q[None], k[None], v[None], w[None])
        yl = ls.step(q[None], k[None], v[None], w[None])
        np.testing.assert_allclose(S64[0], np.array(Sx, dtype=float), rtol=0, atol=1e-13)
        np.testing.assert_allclose(y64[0], np.array(yx, dtype=float), rtol=0, atol=1e-13)
        np.testing.assert_allclose(yl[0], np.array(yx, dtype=float), rtol=0, atol=1e-13)
