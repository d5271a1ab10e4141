"""Pins of the LeapQuant-format oracle (oracle/lq.py) against what the pages and the
mathematics fix: the fit against the SVD (LeapQuant eqs. 5-6 define the tokens as the
best rank-r approximation), exact recovery of a rank-r state, smoothing without
quantization being the identity (sec. 3.4), the eq. 10 readout against dense decoding
from the represented state, the reduction to a plain per-value-channel quantizer, the
rounding rule on hand-built ties, and the 1.19 bytes per element of sec. 4.3."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import lq

RNG = np.random.default_rng(20261202)
FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _gapped(d=128, sig=(10.0, 8.0, 6.0, 4.0), noise=0.01, rng=RNG):
    """A state with a clear rank-4 part: top singular values sig, then noise."""
    A = np.linalg.qr(rng.standard_normal((d, d)))[0]
    Bm = np.linalg.qr(rng.standard_normal((d, d)))[0]
    S = (A[:, :4] * np.array(sig)) @ Bm[:, :4].T
    return S + noise * rng.standard_normal((d, d))


def test_walsh_start_is_orthonormal_and_dense():
    V = lq.walsh_start()
    np.testing.assert_allclose(V.T @ V, np.eye(4), atol=1e-15)
    assert np.all(np.abs(np.abs(V) - 1 / np.sqrt(128)) < 1e-15)
    np.testing.assert_array_equal(V[:, 0] > 0, True)


def test_mgs_matches_qr_up_to_signs():
    W = RNG.standard_normal((128, 4))
    Q = lq.mgs(W)
    Qr, Rr = np.linalg.qr(W)
    Qr = Qr * np.sign(np.diag(Rr))[None, :]     # positive-diagonal convention = Gram-Schmidt's
    np.testing.assert_allclose(Q, Qr, atol=1e-12)
    W[:, 2] = 0.0
    assert not lq.mgs(W)[:, 2].any()


def test_fit_converges_to_the_truncated_svd():
    """Eq. 5 / eq. 6: the tokens minimise ||S - K U^T||_F, i.e. the rank-4 SVD truncation."""
    S = _gapped()
    K, U = lq.fit(S, lq.walsh_start(), 60)
    u, s, vt = np.linalg.svd(S)
    best = (u[:, :4] * s[:4]) @ vt[:4]
    np.testing.assert_allclose(K @ U.T, best, atol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(S - K @ U.T), np.sqrt(np.sum(s[4:] ** 2)), rtol=1e-9)
    np.testing.assert_allclose(U.T @ U, np.eye(4), atol=1e-12)


def test_fit_recovers_an_exact_rank4_state_in_one_iteration():
    S = _gapped(noise=0.0)
    K, U = lq.fit(S, lq.walsh_start(), 1)
    np.testing.assert_allclose(K @ U.T, S, atol=1e-12)


def test_smoothing_without_quantization_is_the_identity():
    """Sec. 3.4: C (C^-1 R) = R, and adding the unchanged tokens back recovers S."""
    S = _gapped(noise=0.05)
    K, U = lq.fit(S, lq.walsh_start(), 2)
    K16, U16 = lq.to_fp16(K), lq.to_fp16(U)
    R = S - K16 @ U16.T
    c = np.maximum(np.sqrt(np.mean(np.abs(R), axis=1)), lq.C_FLOOR)
    X = R / c[:, None]
    np.testing.assert_allclose(c[:, None] * X + K16 @ U16.T, S, atol=1e-14)


def test_quantized_representation_error_is_bounded_by_half_a_step():
    """Every reconstructed element is within half a code step (c_i B_j / 254) of S."""
    S = _gapped(noise=0.05)
    out = lq.boundary(S, lq.walsh_start(), 3)
    S0 = lq.represent(out["Z"], out["B"], out["c"], out["K16"], out["U16"])
    step = out["c"][:, None] * out["B"][None, :] / 127.0
    assert np.all(np.abs(S0 - S) <= 0.5 * step * (1 + 1e-6) + 1e-15)
    # B is the fp32-rounded absmax, so the largest code value is 127 within fp32 rounding
    assert np.max(np.abs(out["w"])) <= 127.0 * (1 + 2.0 ** -23)


def test_no_tokens_no_smoothing_is_a_per_value_channel_quantizer():
    """r = 0 and c = 1: the payload is plain symmetric per-column int8 of S."""
    S = RNG.standard_normal((128, 128)) * 0.02
    zero = np.zeros((128, 0))
    R = S - zero @ zero.T
    B = np.abs(R).max(axis=0).astype(np.float32).astype(np.float64)
    ref = np.empty_like(S)
    for j in range(128):        # independent column-by-column quantizer
        for i in range(128):
            x = S[i, j] * 127.0 / B[j]
            f = np.floor(x)
            ref[i, j] = f + 1 if (x - f > 0.5 or (x - f == 0.5 and f % 2 == 1)) else f
    Z, Bq, c, _ = lq.smooth_quantize(S, zero, zero)
    # lq smooths; undo it here by quantizing the already smoothed residual's definition
    X = S / c[:, None]
    Bx = np.abs(X).max(axis=0)
    np.testing.assert_allclose(Bq, Bx.astype(np.float32), rtol=0)
    Zc = np.clip(np.rint(X * 127.0 / Bq[None, :]), -127, 127)
    np.testing.assert_array_equal(Z, Zc.astype(np.int8))
    # and with c forced to 1 the same rule is exactly the plain quantizer above
    Z1 = np.clip(np.rint(S * 127.0 / B[None, :]), -127, 127)
    np.testing.assert_array_equal(Z1, ref)


def test_rounding_ties_go_to_even_and_zero_columns_give_zero():
    """Rows built so that every mean |R_i| is exactly 1 (so c = 1); column 0 holds values
    on the half-integer grid with absmax 127, so its exact code values are ties."""
    S = np.zeros((128, 128))
    t = np.concatenate([[127.0], (np.arange(127) - 63) + 0.5])
    S[:, 0] = t
    S[:, 1] = 128.0 - np.abs(t)          # row abs-sum 128 -> mean 1 -> c = 1 exactly
    zero = np.zeros((128, 0))
    Z, B, c, w = lq.smooth_quantize(S, zero, zero)
    np.testing.assert_array_equal(c, 1.0)
    assert B[0] == 127.0
    np.testing.assert_array_equal(w[:, 0], t)
    halves = t[1:]
    even = np.where(np.floor(halves) % 2 == 0, np.floor(halves), np.ceil(halves))
    np.testing.assert_array_equal(Z[1:, 0], even.astype(np.int8))
    assert Z[0, 0] == 127
    assert not Z[:, 5].any() and B[5] == 0.0


def test_eq10_readout_equals_dense_decoding_from_the_represented_state():
    """App. B.3 eq. 10 evaluated term by term (payload read, token pairs, records)
    equals the output of dense steps from the represented state (LeapQuant eq. 7)."""
    d, W = 128, 6
    S = _gapped(noise=0.05)
    rep = lq.boundary(S, lq.walsh_start(), 2)
    S0 = lq.represent(rep["Z"], rep["B"], rep["c"], rep["K16"], rep["U16"])
    Sd = S0[None].copy()
    recs = []
    for t in range(W):
        q = RNG.standard_normal((1, d))
        k = RNG.standard_normal((1, d))
        k /= np.linalg.norm(k)
        v = RNG.standard_normal((1, d))
        g = np.array([RNG.uniform(0.9, 0.999)])
        b = np.array([RNG.uniform(0.0, 1.0)])
        y_dense = oracle.dense_step(Sd, q, k, v, g, b)[0]
        # eq. 10 with l = t + 1: Gamma_{1:l} = prod of gates so far (scalar for GDN)
        gam_all = np.prod([r[2] for r in recs]) * g[0]

        def read(x):
            out = (rep["B"] / 127.0) * (rep["Z"].astype(np.float64).T @ (rep["c"] * gam_all * x))
            out += rep["U16"] @ (rep["K16"].T @ (gam_all * x))
            for j, (kj, uj, gj) in enumerate(recs):
                dec = np.prod([r[2] for r in recs[j + 1:]]) * g[0]
                out += uj * (kj @ (dec * x))
            return out
        p = read(k[0])                       # the delta read of S_{l-1} along g * k
        u = b[0] * (v[0] - p)
        y_eq10 = read(q[0]) + u * (k[0] @ q[0])
        np.testing.assert_allclose(y_eq10, y_dense, rtol=0, atol=1e-11)
        recs.append((k[0], u, g[0]))


@pytest.mark.parametrize("bits,r", [(8, 4), (6, 4), (4, 8)])
def test_eq10_readout_with_per_key_decays_equals_dense_kda_decoding(bits, r):
    """Eq. 10 with KDA's per-key gates: Gamma is diagonal over the key rows, so it scales
    the read vector row by row (payload and token keys alike) and each record's key;
    term by term this equals dense KDA decoding from the represented state (at each code
    width: /127 with 4 tokens, /31 with 4, /7 with 8)."""
    d, W = 128, 5
    qmax = lq.qmax_of(bits)
    S = _gapped(noise=0.05) if r == 4 else _gapped8(noise=0.05)
    rep = lq.boundary(S, lq.walsh_start(r=r), 1, qmax=qmax)
    assert np.abs(rep["Z"]).max() == qmax
    S0 = lq.represent(rep["Z"], rep["B"], rep["c"], rep["K16"], rep["U16"], qmax=qmax)
    Sd = S0[None].copy()
    recs = []
    for t in range(W):
        q = RNG.standard_normal((1, d))
        k = RNG.standard_normal((1, d))
        k /= np.linalg.norm(k)
        v = RNG.standard_normal((1, d))
        g = RNG.uniform(0.8, 1.0, (1, d))
        b = np.array([RNG.uniform(0.0, 1.0)])
        y_dense = oracle.dense_step(Sd, q, k, v, g, b)[0]
        gam_all = np.prod([rr[2] for rr in recs] + [g[0]], axis=0)        # per key row

        def read(x):
            out = (rep["B"] / float(qmax)) * (rep["Z"].astype(np.float64).T @ (rep["c"] * gam_all * x))
            out += rep["U16"] @ (rep["K16"].T @ (gam_all * x))
            for j, (kj, uj, _) in enumerate(recs):
                dec = np.prod([rr[2] for rr in recs[j + 1:]] + [g[0]], axis=0)
                out += uj * (kj @ (dec * x))
            return out
        p = read(k[0])
        u = b[0] * (v[0] - p)
        np.testing.assert_allclose(read(q[0]) + u * (k[0] @ q[0]), y_dense, rtol=0, atol=1e-11)
        recs.append((k[0], u, g[0]))


def test_boundary_bytes_per_element_match_the_page():
    f = FIG["leapquant_boundary_bytes"]
    bpe = lq.bytes_per_element(f["dk"], f["r"])
    assert round(bpe, 2) == f["bytes_per_element_printed"]
    assert round(f["fp32_bytes_per_element"] / bpe, 1) == f["reduction_printed"]


# ---------------------------------------------------------------- 4 bits, r = 8 tokens
# (LeapQuant sec. 4.1 uses r = 8 compensator tokens at 4 bits; codes in [-7, 7], /7)

def _gapped8(d=128, noise=0.01, rng=RNG):
    sig = np.array([12.0, 10.0, 9.0, 8.0, 6.0, 5.0, 4.0, 3.0])
    A = np.linalg.qr(rng.standard_normal((d, d)))[0]
    Bm = np.linalg.qr(rng.standard_normal((d, d)))[0]
    return (A[:, :8] * sig) @ Bm[:, :8].T + noise * rng.standard_normal((d, d))


def test_eight_token_fit_converges_to_the_truncated_svd():
    S = _gapped8()
    V0 = lq.walsh_start(r=8)
    np.testing.assert_allclose(V0.T @ V0, np.eye(8), atol=1e-15)
    K, U = lq.fit(S, V0, 80)
    u, s, vt = np.linalg.svd(S)
    np.testing.assert_allclose(K @ U.T, (u[:, :8] * s[:8]) @ vt[:8], atol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(S - K @ U.T), np.sqrt(np.sum(s[8:] ** 2)), rtol=1e-9)


def test_4bit_representation_error_is_bounded_by_half_a_step():
    S = _gapped8(noise=0.05)
    out = lq.boundary(S, lq.walsh_start(r=8), 2, qmax=lq.QMAX4)
    assert out["Z"].min() >= -7 and out["Z"].max() <= 7
    S0 = lq.represent(out["Z"], out["B"], out["c"], out["K16"], out["U16"], qmax=lq.QMAX4)
    step = out["c"][:, None] * out["B"][None, :] / 7.0
    assert np.all(np.abs(S0 - S) <= 0.5 * step * (1 + 1e-6) + 1e-15)


def test_4bit_without_tokens_is_a_per_column_int4_quantizer():
    """r = 0: codes rne(X_ij * 7 / B_j) on the smoothed state, written out column by column."""
    S = RNG.standard_normal((128, 128)) * 0.02
    zero = np.zeros((128, 0))
    Z, Bq, c, _ = lq.smooth_quantize(S, zero, zero, qmax=lq.QMAX4)
    X = S / c[:, None]
    for j in range(128):
        B = float(np.float32(np.abs(X[:, j]).max()))
        assert Bq[j] == B
        for i in range(0, 128, 7):
            x = X[i, j] * 7.0 / B
            f = np.floor(x)
            r = f + 1 if (x - f > 0.5 or (x - f == 0.5 and f % 2 == 1)) else f
            assert Z[i, j] == max(-7, min(7, int(r)))


def test_4bit_ties_round_to_even():
    """c = 1 by construction (row mean |R| = 1); column 0 on the half grid with absmax 7."""
    S = np.zeros((128, 128))
    t = np.concatenate([[7.0], ((np.arange(127) % 15) - 7) + 0.5])
    t[t > 7] = 6.5
    S[:, 0] = t
    S[:, 1] = 128.0 - np.abs(t)
    zero = np.zeros((128, 0))
    Z, B, c, w = lq.smooth_quantize(S, zero, zero, qmax=lq.QMAX4)
    np.testing.assert_array_equal(c, 1.0)
    assert B[0] == 7.0
    np.testing.assert_array_equal(w[:, 0], t)
    halves = t[1:]
    even = np.where(np.floor(halves) % 2 == 0, np.floor(halves), np.ceil(halves))
    np.testing.assert_array_equal(Z[1:, 0], even.astype(np.int8))


def test_nibble_packing_layout_and_round_trip():
    Z = np.array([[-7, 7, -1, 0, 3, -3, 1, -8 + 1]], dtype=np.int8)
    P = lq.pack_nibbles(Z)
    # column 0 in the low nibble, column 1 in the high nibble, two's complement
    np.testing.assert_array_equal(P[0], [0x79, 0x0F, 0xD3, 0x9 << 4 | 0x1])
    np.testing.assert_array_equal(lq.unpack_nibbles(P), Z)
    R = RNG.integers(-7, 8, size=(5, 128)).astype(np.int8)
    np.testing.assert_array_equal(lq.unpack_nibbles(lq.pack_nibbles(R)), R)


def test_eq10_readout_at_4_bits_with_8_tokens_equals_dense_decoding():
    d, W = 128, 4
    S = _gapped8(noise=0.05)
    rep = lq.boundary(S, lq.walsh_start(r=8), 1, qmax=lq.QMAX4)
    S0 = lq.represent(rep["Z"], rep["B"], rep["c"], rep["K16"], rep["U16"], qmax=lq.QMAX4)
    Sd = S0[None].copy()
    recs = []
    for _ in range(W):
        q = RNG.standard_normal((1, d))
        k = RNG.standard_normal((1, d))
        k /= np.linalg.norm(k)
        v = RNG.standard_normal((1, d))
        g = np.array([RNG.uniform(0.9, 0.999)])
        b = np.array([RNG.uniform(0.0, 1.0)])
        y_dense = oracle.dense_step(Sd, q, k, v, g, b)[0]
        gam_all = np.prod([r[2] for r in recs]) * g[0]

        def read(x):
            out = (rep["B"] / 7.0) * (rep["Z"].astype(np.float64).T @ (rep["c"] * gam_all * x))
            out += rep["U16"] @ (rep["K16"].T @ (gam_all * x))
            for j, (kj, uj, _) in enumerate(recs):
                out += uj * (kj @ (np.prod([r[2] for r in recs[j + 1:]]) * g[0] * x))
            return out
        u = b[0] * (v[0] - read(k[0]))
        np.testing.assert_allclose(read(q[0]) + u * (k[0] @ q[0]), y_dense, rtol=0, atol=1e-11)
        recs.append((k[0], u, g[0]))


# ---------------------------------------------------------------- 6 bits, r = 4 tokens
# (LeapQuant sec. 4.1 and Table 1 evaluate a 6-bit group; codes in [-31, 31], /31; the
# token count stays at the default r = 4, since only 4 bits is given r = 8)

def test_6bit_representation_error_is_bounded_by_half_a_step():
    S = _gapped(noise=0.05)
    out = lq.boundary(S, lq.walsh_start(), 2, qmax=lq.QMAX6)
    assert out["Z"].min() >= -31 and out["Z"].max() <= 31
    assert np.abs(out["Z"]).max() == 31
    S0 = lq.represent(out["Z"], out["B"], out["c"], out["K16"], out["U16"], qmax=lq.QMAX6)
    step = out["c"][:, None] * out["B"][None, :] / 31.0
    assert np.all(np.abs(S0 - S) <= 0.5 * step * (1 + 1e-6) + 1e-15)
    # finer than the 4-bit grid on the same state, coarser than the 8-bit one
    err = {b: np.linalg.norm(lq.represent(*(lambda o: (o["Z"], o["B"], o["c"], o["K16"], o["U16"]))(
        lq.boundary(S, lq.walsh_start(), 2, qmax=lq.qmax_of(b))), qmax=lq.qmax_of(b)) - S) for b in (4, 6, 8)}
    assert err[8] < err[6] < err[4]


def test_6bit_without_tokens_is_a_per_column_int6_quantizer():
    """r = 0: codes rne(X_ij * 31 / B_j) on the smoothed state, written out column by column."""
    S = RNG.standard_normal((128, 128)) * 0.02
    zero = np.zeros((128, 0))
    Z, Bq, c, _ = lq.smooth_quantize(S, zero, zero, qmax=lq.QMAX6)
    X = S / c[:, None]
    for j in range(0, 128, 3):
        B = float(np.float32(np.abs(X[:, j]).max()))
        assert Bq[j] == B
        for i in range(0, 128, 5):
            x = X[i, j] * 31.0 / B
            f = np.floor(x)
            r = f + 1 if (x - f > 0.5 or (x - f == 0.5 and f % 2 == 1)) else f
            assert Z[i, j] == max(-31, min(31, int(r)))


def test_6bit_ties_round_to_even():
    """c = 1 by construction (row mean |R| = 1); column 0 on the half grid with absmax 31."""
    S = np.zeros((128, 128))
    t = np.concatenate([[31.0], ((np.arange(127) % 62) - 31) + 0.5])
    S[:, 0] = t
    S[:, 1] = 128.0 - np.abs(t)
    zero = np.zeros((128, 0))
    Z, B, c, w = lq.smooth_quantize(S, zero, zero, qmax=lq.QMAX6)
    np.testing.assert_array_equal(c, 1.0)
    assert B[0] == 31.0
    np.testing.assert_array_equal(w[:, 0], t)
    halves = t[1:]
    even = np.where(np.floor(halves) % 2 == 0, np.floor(halves), np.ceil(halves))
    np.testing.assert_array_equal(Z[1:, 0], even.astype(np.int8))


def test_6bit_packing_layout_and_round_trip():
    Z = np.zeros((1, 128), dtype=np.int8)
    Z[0, :4] = [-31, 31, -1, 5]   # = 4 (-8) + 1, 4 (7) + 3, 4 (-1) + 3, 4 (1) + 1
    P = lq.pack6(Z)
    assert P.shape == (1, 96) and P.dtype == np.uint8
    # high parts as nibbles (column 0 low), then the low parts four per byte (column 0 lowest)
    np.testing.assert_array_equal(P[0, :2], [0x78, 0x1F])
    assert P[0, 64] == 0b01_11_11_01
    assert not P[0, 2:64].any() and not P[0, 65:].any()
    np.testing.assert_array_equal(lq.unpack6(P), Z)
    R = RNG.integers(-31, 32, size=(5, 128)).astype(np.int8)
    np.testing.assert_array_equal(lq.unpack6(lq.pack6(R)), R)


def test_eq10_readout_at_6_bits_equals_dense_decoding():
    d, W = 128, 4
    S = _gapped(noise=0.05)
    rep = lq.boundary(S, lq.walsh_start(), 1, qmax=lq.QMAX6)
    S0 = lq.represent(rep["Z"], rep["B"], rep["c"], rep["K16"], rep["U16"], qmax=lq.QMAX6)
    Sd = S0[None].copy()
    recs = []
    for _ in range(W):
        q = RNG.standard_normal((1, d))
        k = RNG.standard_normal((1, d))
        k /= np.linalg.norm(k)
        v = RNG.standard_normal((1, d))
        g = np.array([RNG.uniform(0.9, 0.999)])
        b = np.array([RNG.uniform(0.0, 1.0)])
        y_dense = oracle.dense_step(Sd, q, k, v, g, b)[0]
        gam_all = np.prod([r[2] for r in recs]) * g[0]

        def read(x):
            out = (rep["B"] / 31.0) * (rep["Z"].astype(np.float64).T @ (rep["c"] * gam_all * x))
            out += rep["U16"] @ (rep["K16"].T @ (gam_all * x))
            for j, (kj, uj, _) in enumerate(recs):
                out += uj * (kj @ (np.prod([r[2] for r in recs[j + 1:]]) * g[0] * x))
            return out
        u = b[0] * (v[0] - read(k[0]))
        np.testing.assert_allclose(read(q[0]) + u * (k[0] @ q[0]), y_dense, rtol=0, atol=1e-11)
        recs.append((k[0], u, g[0]))
