"""GPU parity of LeapQuant's window-boundary format (compensator tokens, residual
smoothing, per-value-channel int8; eq. 10 readout) against the fp64 oracle, teacher-forced
per window (the oracle restarts from the GPU's representation at every window start and
recomputes each refit's payload from the GPU's own fp16 tokens).

Bars: outputs within 1e-4 norm-wise relative error; the token product Kt Ut^T within
2e-3 (fp16 rounding of the tokens, 2^-11, plus fp32 iteration error), each key token
within 4e-3 of the largest and each value-vector entry within 2e-3 absolute; c^2 and B
within 1e-5 of the uncancelled magnitude |S| + |Kt Ut^T| they are computed from (the
residual cancels the outliers the tokens hold, which amplifies the fp32 state's
rounding relative to the residual itself); payload codes, recomputed from the GPU's c
and B, within 1 LSB and different only near a rounding tie (1e-3 LSB plus the fp32
error of the uncancelled value, 1e-6 of it, in LSB units)."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity import DEV, TOL_Q8, check_lq_refit, lq_host, new_lq_buffers, rsu, run_lq, say

pytestmark = pytest.mark.gpu


def _check(err, name, boundaries=True):
    say(f"[lq] {name}: {err}")
    assert err["y"] < TOL_Q8
    assert err["tok"] < 2e-3 and err["tok_k"] < 4e-3 and err["tok_u"] < 2e-3
    assert err["c"] < 1e-5 and err["B"] < 1e-5
    assert err["z_maxdiff"] <= 1 and err["z_flips_outside_band"] == 0
    if boundaries:
        assert err["boundaries"] > 0


@pytest.mark.parametrize("W,B,H,n_iter", [(16, 2, 5, 1), (16, 3, 4, 2), (5, 2, 3, 1), (1, 2, 2, 0),
                                          (16, 10, 10, 1)])
def test_lq_windows_small(W, B, H, n_iter):
    w = wl.custom(wl.WORKLOADS[6], B=B, H=H, W=W, steps=2 * W + min(W, 3))
    _check(run_lq(w, n_iter=n_iter), f"W={W} B={B} H={H} n_iter={n_iter}")


@pytest.mark.parametrize("W,B,H,n_iter", [(16, 2, 5, 1), (16, 3, 4, 2), (7, 2, 3, 1), (1, 2, 2, 0)])
def test_lq_kda_windows_small(W, B, H, n_iter):
    """Per-key gates (KDA): Gamma of eq. 10 is diagonal over the key rows."""
    w = wl.custom(wl.WORKLOADS[9], B=B, H=H, W=W, steps=2 * W + min(W, 3))
    _check(run_lq(w, n_iter=n_iter), f"kda W={W} B={B} H={H} n_iter={n_iter}")


def test_lq_kda_b128_h32_full_size_sampled():
    """The KDA LeapQuant workload (B=128, H=32, W=16), 64 sampled heads, 3 windows."""
    w = wl.WORKLOADS[9]
    say(f"[lq] {w.name}: full size, 64 sampled heads, 48 steps")
    _check(run_lq(w, n_iter=1, sample=64, steps=48), w.name)


@pytest.mark.parametrize("W,B,H,n_iter", [(16, 2, 5, 1), (16, 3, 4, 2), (5, 2, 3, 1), (1, 2, 2, 0)])
def test_lq4_windows_small(W, B, H, n_iter):
    """4-bit codes (two per byte, /7) with 8 tokens (LeapQuant sec. 4.1)."""
    w = wl.custom(wl.WORKLOADS[12], B=B, H=H, W=W, steps=2 * W + min(W, 3))
    _check(run_lq(w, n_iter=n_iter), f"4-bit W={W} B={B} H={H} n_iter={n_iter}")


@pytest.mark.parametrize("n_iter0", [0, 3])
def test_lq4_quantize_start_iterations(n_iter0):
    w = wl.custom(wl.WORKLOADS[12], B=3, H=11, W=16, steps=0)
    _check(run_lq(w, n_iter0=n_iter0, steps=0), f"4-bit quantize n_iter0={n_iter0}", boundaries=False)


def test_lq4_ragged_batch():
    """100 heads: the head order's last group of 32 is cut short."""
    w = wl.custom(wl.WORKLOADS[12], B=10, H=10, W=16, steps=35)
    _check(run_lq(w, n_iter=1), "4-bit B=10 H=10")


def test_lq4_zero_state_gives_zero_tokens_and_payload():
    m = rsu()
    S = torch.zeros(1, 2, 128, 128, device=DEV)
    w = wl.custom(wl.WORKLOADS[12], B=1, H=2, W=16)
    buf = new_lq_buffers(w)
    buf["C"].fill_(7.0)
    buf["Z"].fill_(0x5A)
    m.gdn_lq4_quantize(S, 4, buf["Z"], buf["B"], buf["C"], buf["Kc"], buf["Uc"])
    assert not buf["Z"].any() and not buf["B"].any() and not buf["Kc"].any()
    np.testing.assert_array_equal(buf["C"].cpu().numpy(), np.float32(1e-6))


def test_lq4_b256_h48_full_size_sampled():
    w = wl.WORKLOADS[12]
    say(f"[lq] {w.name}: full size, 64 sampled heads, 48 steps")
    _check(run_lq(w, n_iter=1, sample=64, steps=48), w.name)


@pytest.mark.parametrize("W,B,H,n_iter", [(16, 2, 5, 1), (16, 3, 4, 2), (5, 2, 3, 1), (1, 2, 2, 0)])
def test_lq6_windows_small(W, B, H, n_iter):
    """6-bit codes (high parts as nibbles, low 2-bit parts four per byte, /31) with 4 tokens."""
    w = wl.custom(wl.WORKLOADS[16], B=B, H=H, W=W, steps=2 * W + min(W, 3))
    _check(run_lq(w, n_iter=n_iter), f"6-bit W={W} B={B} H={H} n_iter={n_iter}")


@pytest.mark.parametrize("n_iter0", [0, 3])
def test_lq6_quantize_start_iterations(n_iter0):
    w = wl.custom(wl.WORKLOADS[16], B=3, H=11, W=16, steps=0)
    _check(run_lq(w, n_iter0=n_iter0, steps=0), f"6-bit quantize n_iter0={n_iter0}", boundaries=False)


def test_lq6_ragged_batch():
    """100 heads: the head order's last group of 32 is cut short."""
    w = wl.custom(wl.WORKLOADS[16], B=10, H=10, W=16, steps=35)
    _check(run_lq(w, n_iter=1), "6-bit B=10 H=10")


def test_lq6_zero_state_gives_zero_tokens_and_payload():
    m = rsu()
    S = torch.zeros(1, 2, 128, 128, device=DEV)
    w = wl.custom(wl.WORKLOADS[16], B=1, H=2, W=16)
    buf = new_lq_buffers(w)
    buf["C"].fill_(7.0)
    buf["Z"].fill_(0x5A)
    m.gdn_lq6_quantize(S, 4, buf["Z"], buf["B"], buf["C"], buf["Kc"], buf["Uc"])
    assert not buf["Z"].any() and not buf["B"].any() and not buf["Kc"].any()
    np.testing.assert_array_equal(buf["C"].cpu().numpy(), np.float32(1e-6))


def test_lq6_extreme_codes_round_trip():
    """A state whose smoothed residual puts codes at -31, 31 and every value between in each
    column: the payload's two parts decode to the oracle's codes exactly."""
    m = rsu()
    from oracle import lq as lqo
    rng = np.random.default_rng(61)
    S = (rng.standard_normal((2, 3, 128, 128)) * 0.02).astype(np.float32)
    S[..., 5, :] *= 40.0   # a heavy row the smoothing scales down
    Sd = torch.from_numpy(S).to(DEV)
    w = wl.custom(wl.WORKLOADS[16], B=2, H=3, W=16)
    buf = new_lq_buffers(w)
    m.gdn_lq6_quantize(Sd, 2, buf["Z"], buf["B"], buf["C"], buf["Kc"], buf["Uc"])
    hd = torch.arange(6, device=DEV)
    rep = lq_host(buf, hd)
    assert (np.abs(rep[0]).max(axis=1) == 31).all()          # each column's absmax code
    assert set(np.unique(rep[0]).tolist()) == set(range(-31, 32))  # every code, both signs
    err = {"tok": 0.0, "tok_k": 0.0, "tok_u": 0.0, "c": 0.0, "B": 0.0, "z_maxdiff": 0, "z_flips": 0,
           "z_flips_outside_band": 0}
    from parity import check_lq_refit
    check_lq_refit(S.reshape(6, 128, 128).astype(np.float64), np.broadcast_to(lqo.walsh_start(), (6, 128, 4)),
                   2, rep, err, qmax=31)
    say(f"[lq] 6-bit extremes: {err}")
    assert err["z_maxdiff"] <= 1 and err["z_flips_outside_band"] == 0


def test_lq6_b256_h48_full_size_sampled():
    w = wl.WORKLOADS[16]
    say(f"[lq] {w.name}: full size, 64 sampled heads, 48 steps")
    _check(run_lq(w, n_iter=1, sample=64, steps=48), w.name)


@pytest.mark.parametrize("cid", [17, 18])
@pytest.mark.parametrize("W,B,H,n_iter", [(16, 2, 5, 1), (16, 3, 4, 2), (7, 2, 3, 1), (1, 2, 2, 0)])
def test_lq_low_bit_kda_windows_small(cid, W, B, H, n_iter):
    """KDA's per-key gates at 4 bits (8 tokens) and 6 bits (4 tokens)."""
    w = wl.custom(wl.WORKLOADS[cid], B=B, H=H, W=W, steps=2 * W + min(W, 3))
    _check(run_lq(w, n_iter=n_iter), f"kda {w.bits}-bit W={W} B={B} H={H} n_iter={n_iter}")


@pytest.mark.parametrize("cid", [17, 18])
def test_lq_low_bit_kda_b128_h32_full_size_sampled(cid):
    """The KDA LeapQuant workloads at 4 and 6 bits (B=128, H=32, W=16), 64 sampled heads,
    3 windows."""
    w = wl.WORKLOADS[cid]
    say(f"[lq] {w.name}: full size, 64 sampled heads, 48 steps")
    _check(run_lq(w, n_iter=1, sample=64, steps=48), w.name)


@pytest.mark.parametrize("n_iter0", [0, 3])
def test_lq_quantize_start_iterations(n_iter0):
    w = wl.custom(wl.WORKLOADS[6], B=2, H=3, W=16, steps=0)
    _check(run_lq(w, n_iter0=n_iter0, steps=0), f"quantize n_iter0={n_iter0}", boundaries=False)


@pytest.mark.parametrize("cid,fn", [(6, "gdn_lq_quantize"), (16, "gdn_lq6_quantize"), (12, "gdn_lq4_quantize"),
                                    (9, "kda_lq_quantize"), (18, "kda_lq6_quantize"), (17, "kda_lq4_quantize")])
def test_lq_quantize_tiny_column(cid, fn):
    """A value column whose smoothed maximum B lies near 2^-123, where qmax / B overflows fp32
    (the column's state entries are at most 2^-126: subnormal or nearly; no outliers, so the
    smoothing factors c lie in [0.11, 0.14]). The column is quantized after scaling by 2^64:
    its codes follow the oracle's like any other column's, and its largest code is qmax."""
    from oracle import lq as lqo
    m = rsu()
    w = wl.custom(wl.WORKLOADS[cid], B=1, H=3, W=16, steps=0, outliers=False)
    S0 = wl.initial_state(w)
    col = 9
    e = np.ceil(np.log2(np.abs(S0[:, :, col]).max(axis=1).astype(np.float64))).astype(np.int32)
    S0[:, :, col] = np.ldexp(S0[:, :, col], (-126 - e)[:, None])
    say(f"[lq] {fn}: tiny column {col}")
    buf = new_lq_buffers(w)
    getattr(m, fn)(torch.from_numpy(S0).to(DEV).view(1, 3, 128, 128), 8, buf["Z"], buf["B"], buf["C"],
                   buf["Kc"], buf["Uc"])
    hd = torch.arange(w.heads, device=DEV)
    rep = lq_host(buf, hd)
    qmax = lqo.qmax_of(w.bits)
    Bg = rep[1][:, col]
    assert np.all(Bg > 0) and np.all(Bg < 2.0 ** -121.4), Bg
    assert np.all(np.abs(rep[0][:, :, col]).max(axis=1) == qmax)
    err = {"tok": 0.0, "tok_k": 0.0, "tok_u": 0.0, "c": 0.0, "B": 0.0, "z_maxdiff": 0, "z_flips": 0,
           "z_flips_outside_band": 0}
    walsh = np.broadcast_to(lqo.walsh_start(r=8 if w.bits == 4 else 4), (w.heads, 128, 8 if w.bits == 4 else 4))
    check_lq_refit(S0.astype(np.float64), walsh, 8, rep, err, qmax=qmax)
    _check(dict(err, y=0.0), f"{fn} tiny column", boundaries=False)


def test_lq_zero_state_gives_zero_tokens_and_payload():
    m = rsu()
    S = torch.zeros(1, 2, 128, 128, device=DEV)
    w = wl.custom(wl.WORKLOADS[6], B=1, H=2, W=16)
    buf = new_lq_buffers(w)
    buf["C"].fill_(7.0)
    m.gdn_lq_quantize(S, 4, buf["Z"], buf["B"], buf["C"], buf["Kc"], buf["Uc"])
    assert not buf["Z"].any() and not buf["B"].any() and not buf["Kc"].any()
    np.testing.assert_array_equal(buf["C"].cpu().numpy(), np.float32(1e-6))


def test_lq_b256_h48_full_size_sampled():
    """The int8 workload's inputs (B=256, H=48, W=16) in LeapQuant's format, 64 sampled
    heads, 3 windows, one warm-started iteration per refit."""
    w = wl.WORKLOADS[6]
    say(f"[lq] {w.name}: full size, 64 sampled heads, 48 steps")
    _check(run_lq(w, n_iter=1, sample=64, steps=48), w.name)
