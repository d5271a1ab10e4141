"""Exact rational brute force of the three state representations, for tiny heads.

TEST INFRASTRUCTURE (same rules as the rest of ``oracle/``). Everything is
``fractions.Fraction``, so the algebraic identities the pages state -- window
unrolling (LeapQuant eq. 4 and App. B.2) and the base+log invariant (DeltaLog
eq. 7 and its closure argument) -- must hold with equality, not to a tolerance.
Decays are kept as exact products of the gates; the exponential of a sum of
log-decays in DeltaLog is the same product, which rationals can hold exactly.

Matrices are lists of rows; vectors are lists.
"""
from __future__ import annotations

from fractions import Fraction as F
from typing import List, Sequence

Mat = List[List[F]]
Vec = List[F]


def frac_vec(x: Sequence[float]) -> Vec:
    return [F(float(t)) for t in x]


def frac_mat(x) -> Mat:
    return [frac_vec(row) for row in x]


def dense_step(S: Mat, q: Vec, k: Vec, v: Vec, g: Vec, beta: F):
    """Decay, read along k from the decayed state, delta write, post-update readout
    (LeapQuant App. A). Returns (S_new, y); S is not modified."""
    dk, dv = len(S), len(S[0])
    Sd = [[g[i] * S[i][j] for j in range(dv)] for i in range(dk)]
    u = [beta * (v[j] - sum(Sd[i][j] * k[i] for i in range(dk))) for j in range(dv)]
    Sn = [[Sd[i][j] + k[i] * u[j] for j in range(dv)] for i in range(dk)]
    y = [sum(Sn[i][j] * q[i] for i in range(dk)) for j in range(dv)]
    return Sn, y


def householder_step(S: Mat, k: Vec, v: Vec, g: Vec, beta: F) -> Mat:
    """(I - beta k k^T) Diag(g) S + beta k v^T: the left-hand side of the GDN and
    KDA expansions in LeapQuant App. A (for a scalar gate Diag(g) = alpha I commutes)."""
    dk, dv = len(S), len(S[0])
    Sd = [[g[i] * S[i][j] for j in range(dv)] for i in range(dk)]
    A = [[(1 if i == m else 0) - beta * k[i] * k[m] for m in range(dk)] for i in range(dk)]
    return [[sum(A[i][m] * Sd[m][j] for m in range(dk)) + beta * k[i] * v[j]
             for j in range(dv)] for i in range(dk)]


def _rne(x: F) -> int:
    """Round to nearest integer, ties to even."""
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def quantize(S: Mat):
    """Per-row symmetric int8: a_i = max_j |S_ij|, z = clamp(rne(S*127/a), -127, 127)."""
    Z, a = [], []
    for row in S:
        ai = max(abs(x) for x in row)
        a.append(ai)
        Z.append([0 if ai == 0 else max(-127, min(127, _rne(x * 127 / ai))) for x in row])
    return Z, a


def dequant(Z, a) -> Mat:
    return [[F(z) * a[i] / 127 for z in Z[i]] for i in range(len(Z))]


def window_run(S0: Mat, inputs, W: int):
    """Per-window quantization by eq. 4: S_l = Gamma_{1:l} S^_0 + sum Gamma_{j+1:l} k_j u_j^T,
    u_l from S_{l-1} read along the decayed key, y_l = S_l^T q_l, requantize at l = W.
    inputs: list of (q, k, v, g, beta). Returns (ys, [(Z, a) at each boundary])."""
    dk, dv = len(S0), len(S0[0])
    Z, a = quantize(S0)
    base = dequant(Z, a)
    recs = []
    ys, bounds = [], []

    def mat(l):
        out = []
        for i in range(dk):
            gam0 = F(1)
            for (g, _, _) in recs[:l]:
                gam0 *= g[i]
            row = [gam0 * base[i][j] for j in range(dv)]
            for m in range(l):
                c = recs[m][1][i]
                for (g, _, _) in recs[m + 1:l]:
                    c *= g[i]
                for j in range(dv):
                    row[j] += c * recs[m][2][j]
            out.append(row)
        return out

    for (q, k, v, g, beta) in inputs:
        l = len(recs) + 1
        Sp = mat(l - 1)
        u = [beta * (v[j] - sum(g[i] * Sp[i][j] * k[i] for i in range(dk))) for j in range(dv)]
        recs.append((g, k, u))
        Sl = mat(l)
        ys.append([sum(Sl[i][j] * q[i] for i in range(dk)) for j in range(dv)])
        if l == W:
            Z, a = quantize(Sl)
            bounds.append((Z, a))
            base = dequant(Z, a)
            recs = []
    return ys, bounds


def explicit_schedule_run(S0: Mat, inputs, W: int):
    """Dequantize, W eager dense steps, requantize -- the schedule eq. 4 unrolls."""
    Z, a = quantize(S0)
    S = dequant(Z, a)
    ys, bounds = [], []
    for t, (q, k, v, g, beta) in enumerate(inputs):
        S, y = dense_step(S, q, k, v, g, beta)
        ys.append(y)
        if (t + 1) % W == 0:
            Z, a = quantize(S)
            bounds.append((Z, a))
            S = dequant(Z, a)
    return ys, bounds


def rwkv6_step(S: Mat, q: Vec, k: Vec, v: Vec, w: Vec):
    """RWKV6 in the pages' common form: S <- Diag(w) S + k v^T, y = S^T q."""
    dk, dv = len(S), len(S[0])
    Sn = [[w[i] * S[i][j] + k[i] * v[j] for j in range(dv)] for i in range(dk)]
    return Sn, [sum(Sn[i][j] * q[i] for i in range(dk)) for j in range(dv)]


def rwkv7_step(S: Mat, q: Vec, k: Vec, v: Vec, w: Vec, kappa: Vec, a: Vec):
    """RWKV7 as the product of its transition: S <- (Diag(w) - kappa (a * kappa)^T) S + k v^T."""
    dk, dv = len(S), len(S[0])
    T = [[(w[i] if i == m else 0) - kappa[i] * a[m] * kappa[m] for m in range(dk)] for i in range(dk)]
    Sn = [[sum(T[i][m] * S[m][j] for m in range(dk)) + k[i] * v[j] for j in range(dv)] for i in range(dk)]
    return Sn, [sum(Sn[i][j] * q[i] for i in range(dk)) for j in range(dv)]


def rwkv7_window_run(S0: Mat, inputs, W: int):
    """RWKV7 on the per-window representation with exact arithmetic: two records per token
    (erase: gate w, key kappa, u = -S^T (a * kappa); write: gate 1, key k, u = v), the state
    materialized by eq. 4 from the window-start state and the records, requantized at
    every window end. inputs: (q, k, v, w, kappa, a) per token. Returns (ys, boundaries)."""
    dk, dv = len(S0), len(S0[0])
    Z, a = quantize(S0)
    ys, bounds = [], []
    recs = []          # (gate vector, key, u)

    def mat(base):
        out = []
        for i in range(dk):
            g = F(1)
            for (gv, _, _) in recs:
                g *= gv[i]
            row = [g * base[i][j] for j in range(dv)]
            for m, (_, km, um) in enumerate(recs):
                c = km[i]
                for (gv, _, _) in recs[m + 1:]:
                    c *= gv[i]
                for j in range(dv):
                    row[j] += c * um[j]
            out.append(row)
        return out

    for t, (q, k, v, w, kappa, er) in enumerate(inputs):
        base = dequant(Z, a)
        S = mat(base)
        ue = [-sum(S[i][j] * er[i] * kappa[i] for i in range(dk)) for j in range(dv)]
        recs.append((list(w), list(kappa), ue))
        recs.append(([F(1)] * dk, list(k), list(v)))
        S = mat(base)
        ys.append([sum(S[i][j] * q[i] for i in range(dk)) for j in range(dv)])
        if (t + 1) % W == 0:
            Z, a = quantize(S)
            bounds.append((Z, a))
            recs = []
    return ys, bounds


def rwkv7_explicit_run(S0: Mat, inputs, W: int):
    """Dequantize at each window start, run dense RWKV7 steps, requantize at its end."""
    Z, a = quantize(S0)
    ys, bounds = [], []
    S = dequant(Z, a)
    for t, (q, k, v, w, kappa, er) in enumerate(inputs):
        S, y = rwkv7_step(S, q, k, v, w, kappa, er)
        ys.append(y)
        if (t + 1) % W == 0:
            Z, a = quantize(S)
            bounds.append((Z, a))
            S = dequant(Z, a)
    return ys, bounds


def deltaproduct_householder(S: Mat, ks, vs, alpha: F, betas) -> Mat:
    """A DeltaProduct token as the product of its generalized Householder sub-steps
    (LeapQuant App. A, Table 4; each sub-step the left-hand side of the GDN expansion):
    S <- (I - b_n k_n k_n^T)(... ((I - b_1 k_1 k_1^T) alpha S + b_1 k_1 v_1^T) ...) + b_n k_n v_n^T."""
    dk = len(S)
    for s, (k, v, b) in enumerate(zip(ks, vs, betas)):
        S = householder_step(S, k, v, [alpha if s == 0 else F(1)] * dk, b)
    return S


def deltaproduct_window_run(S0: Mat, inputs, W: int):
    """DeltaProduct on the per-window representation with exact arithmetic: one record per
    sub-step (gate alpha for the first, 1 for the others; u = beta (v - (d S_cur)^T k)), the
    state materialized by eq. 4 from the window-start state and the records, requantized at
    every window end. inputs: (q, ks, vs, alpha, betas) per token. Returns (ys, boundaries)."""
    dk, dv = len(S0), len(S0[0])
    Z, a = quantize(S0)
    ys, bounds = [], []
    recs = []          # (scalar gate, key, u)

    def mat(base):
        out = []
        for i in range(dk):
            g = F(1)
            for (gr, _, _) in recs:
                g *= gr
            row = [g * base[i][j] for j in range(dv)]
            for m, (_, km, um) in enumerate(recs):
                c = km[i]
                for (gr, _, _) in recs[m + 1:]:
                    c *= gr
                for j in range(dv):
                    row[j] += c * um[j]
            out.append(row)
        return out

    for t, (q, ks, vs, alpha, betas) in enumerate(inputs):
        base = dequant(Z, a)
        for s, (k, v, b) in enumerate(zip(ks, vs, betas)):
            d = alpha if s == 0 else F(1)
            S = mat(base)
            u = [b * (v[j] - sum(d * S[i][j] * k[i] for i in range(dk))) for j in range(dv)]
            recs.append((d, list(k), u))
        S = mat(base)
        ys.append([sum(S[i][j] * q[i] for i in range(dk)) for j in range(dv)])
        if (t + 1) % W == 0:
            Z, a = quantize(S)
            bounds.append((Z, a))
            recs = []
    return ys, bounds


def deltaproduct_explicit_run(S0: Mat, inputs, W: int):
    """Dequantize at each window start, run DeltaProduct tokens as products of Householder
    sub-steps, requantize at its end."""
    Z, a = quantize(S0)
    ys, bounds = [], []
    S = dequant(Z, a)
    for t, (q, ks, vs, alpha, betas) in enumerate(inputs):
        S = deltaproduct_householder(S, ks, vs, alpha, betas)
        ys.append([sum(S[i][j] * q[i] for i in range(len(S))) for j in range(len(S[0]))])
        if (t + 1) % W == 0:
            Z, a = quantize(S)
            bounds.append((Z, a))
            S = dequant(Z, a)
    return ys, bounds


def log_run(S0: Mat, inputs, M: int, delta: bool = True):
    """Base + log (DeltaLog Alg. 1, eqs. 4-7) with decays as exact gate products:
    D(lbar) is the product of the gates since the last merge and D(lbar - Lam_m) the
    product of the gates after entry m. Without the delta rule (RWKV6) the value-side
    factor is v itself. Returns (ys, logical states after each step)."""
    dk, dv = len(S0), len(S0[0])
    C = M - 1
    Sbar = [row[:] for row in S0]
    dec = [F(1)] * dk                   # exp(lbar)
    log_entries = []                    # (K, U, exp(Lam))
    ys, states = [], []

    def logical(decay, entries):
        out = []
        for i in range(dk):
            row = [decay[i] * Sbar[i][j] for j in range(dv)]
            for (Km, Um, Em) in entries:
                c = decay[i] / Em[i] * Km[i]
                for j in range(dv):
                    row[j] += c * Um[j]
            out.append(row)
        return out

    for (q, k, v, g, beta) in inputs:
        Sold = logical(dec, log_entries)
        if delta:
            b = [beta * (v[j] - sum(g[i] * Sold[i][j] * k[i] for i in range(dk))) for j in range(dv)]
        else:
            b = list(v)
        dec = [dec[i] * g[i] for i in range(dk)]
        Snew = logical(dec, log_entries)
        Snew = [[Snew[i][j] + k[i] * b[j] for j in range(dv)] for i in range(dk)]
        ys.append([sum(Snew[i][j] * q[i] for i in range(dk)) for j in range(dv)])
        if len(log_entries) < C:
            log_entries.append((k, b, dec[:]))
        else:
            Sbar = Snew
            dec = [F(1)] * dk
            log_entries = []
        states.append(logical(dec, log_entries))
    return ys, states


def eager_run(S0: Mat, inputs, delta: bool = True):
    S = [row[:] for row in S0]
    ys, states = [], []
    for (q, k, v, g, beta) in inputs:
        S, y = dense_step(S, q, k, v, g, beta) if delta else rwkv6_step(S, q, k, v, g)
        ys.append(y)
        states.append(S)
    return ys, states
