"""Maximum sizes: 135,168 heads (B=2048, H=66). The dense fp32 state is then 8.86 GB, past
2^31 fp32 elements, and the int8 codes 2.2 GB, past 2^31 bytes, so every head offset beyond
those limits must be formed in 64 bits.

Generating seeded inputs for every head on the host would take minutes, and heads are
independent: the bulk of the state and of the step inputs is filled on the GPU by torch's own
generator (values of the workloads' distributions), and the sampled heads -- the first, the
last, the first head past 2^31 state elements, and a few more -- get the seeded values of a
small workload of the same kind, which the oracle then checks.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import (DEV, TOL_F32, TOL_Q8, check_stepq_pack, new_stepq_buffers, rel_err, rsu, say,
                    stepq_host)

pytestmark = pytest.mark.gpu

B, H = 2048, 66
N = B * H


def _heads():
    rng = np.random.default_rng(99)
    extra = rng.choice(N, size=4, replace=False)
    return np.array(sorted({0, 131072, 131073, N - 1, *extra.tolist()}), dtype=np.int64)


def _small(base, n):
    return wl.custom(base, B=1, H=n)


def _inputs(w, ws, hd, t):
    """Device inputs of the big workload for step t: torch-filled, the sampled heads from ws."""
    g = torch.Generator(device=DEV)
    g.manual_seed(5000 + t)
    n = w.heads

    def unit(x):
        return x / x.norm(dim=1, keepdim=True)

    d = {"q": unit(torch.randn(n, 128, device=DEV, generator=g)),
         "k": unit(torch.randn(n, 128, device=DEV, generator=g)),
         "v": torch.randn(n, 128, device=DEV, generator=g)}
    gshape = (n, 128) if w.per_key_gate else (n,)
    d["gate"] = w.gate_lo + (w.gate_hi - w.gate_lo) * torch.rand(gshape, device=DEV, generator=g)
    d["beta"] = torch.rand(n, device=DEV, generator=g)
    x = wl.step_inputs(ws, t)
    for name in d:
        d[name][hd] = torch.from_numpy(x[name]).to(DEV)
    dt = torch.bfloat16 if w.qkv == "bf16" else torch.float32
    out = {nm: d[nm].to(dt).view(B, H, 128) for nm in ("q", "k", "v")}
    out["gate"] = d["gate"].view((B, H, 128) if w.per_key_gate else (B, H))
    out["beta"] = d["beta"].view(B, H)
    return x, out


def _state(ws, hd, std):
    g = torch.Generator(device=DEV)
    g.manual_seed(4000)
    S = torch.empty(N, 128, 128, device=DEV).normal_(0.0, std, generator=g)
    S0 = wl.initial_state(ws)
    S[hd] = torch.from_numpy(S0).to(DEV)
    return S.view(B, H, 128, 128), S0.astype(np.float64)


def _host(x):
    return x["q"], x["k"], x["v"], x["gate"], x["beta"]


def test_dense_gdn_past_2e31_state_elements():
    m = rsu()
    heads = _heads()
    hd = torch.from_numpy(heads).to(DEV)
    w = wl.custom(wl.WORKLOADS[2], B=B, H=H)
    ws = _small(w, len(heads))
    say(f"max size dense: {N} heads, sampled {heads.tolist()}")
    S, S_ref = _state(ws, hd, w.state_std)
    y = torch.empty(B, H, 128, device=DEV)
    worst = 0.0
    for t in range(2):
        x, d = _inputs(w, ws, hd, t)
        m.gdn_decode_step(S, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
        y_ref = oracle.dense_step(S_ref, *_host(x))
        worst = max(worst, rel_err(y.view(N, 128)[hd].cpu().numpy(), y_ref))
    eS = rel_err(S.view(N, 128, 128)[hd].cpu().numpy(), S_ref)
    say(f"  y {worst:.2e}  S {eS:.2e}")
    assert worst < TOL_F32 and eS < TOL_F32
    del S
    torch.cuda.empty_cache()


def test_int8_window_past_2e31_code_bytes():
    """W = 2: one in-window step and one boundary (requantization) per head."""
    m = rsu()
    heads = _heads()
    hd = torch.from_numpy(heads).to(DEV)
    w = wl.custom(wl.WORKLOADS[4], B=B, H=H, W=2)
    ws = _small(w, len(heads))
    say(f"max size int8 window: {N} heads")
    S, S_ref = _state(ws, hd, w.state_std)
    Z = torch.empty(B, H, 128, 128, device=DEV, dtype=torch.int8)
    A = torch.empty(B, H, 128, device=DEV)
    m.q8_quantize(S, Z, A)
    del S
    torch.cuda.empty_cache()
    Zr, ar = oracle.q8_quantize(S_ref)
    assert np.array_equal(Z.view(N, 128, 128)[hd].cpu().numpy(), Zr)
    assert np.array_equal(A.view(N, 128)[hd].cpu().numpy(), ar)
    Kb = torch.zeros(B, H, 2, 128, device=DEV, dtype=torch.bfloat16)
    Ub = torch.zeros(B, H, 2, 128, device=DEV)
    Gb = torch.zeros(B, H, 2, device=DEV)
    y = torch.empty(B, H, 128, device=DEV)
    ref = oracle.WindowState(Zr, ar, 2, False)
    worst = 0.0
    for t in range(2):
        x, d = _inputs(w, ws, hd, t)
        m.gdn_q8_window(2, t, Z, A, Kb, Ub, Gb, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
        if t == 1:
            y_ref, _, wcode = ref.step(*_host(x), want_boundary=True)
        else:
            y_ref = ref.step(*_host(x))
        worst = max(worst, rel_err(y.view(N, 128)[hd].cpu().numpy(), y_ref))
    Zg = Z.view(N, 128, 128)[hd].cpu().numpy().astype(np.int32)
    diff = Zg - ref.Z.astype(np.int32)
    near = np.abs(np.abs(wcode - np.floor(wcode)) - 0.5) < 1e-3
    say(f"  y {worst:.2e}  code flips {int((diff != 0).sum())}")
    assert worst < TOL_Q8
    assert int(np.abs(diff).max()) <= 1 and int(((diff != 0) & ~near).sum()) == 0
    ag = A.view(N, 128)[hd].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(ag - ref.a) / np.maximum(ref.a, 1e-30)) < 1e-5


def test_stepq_at_the_largest_batch():
    from oracle import stepq as sqo
    m = rsu()
    heads = _heads()
    hd = torch.from_numpy(heads).to(DEV)
    w = wl.custom(wl.WORKLOADS[13], B=B, H=H)
    ws = _small(w, len(heads))
    say(f"max size packed state: {N} heads")
    S, S_ref = _state(ws, hd, w.state_std)
    g = torch.Generator(device=DEV)
    g.manual_seed(4100)
    om = torch.exp(1.08 * torch.randn(N, 128, device=DEV, generator=g))
    om_s = wl.row_influence(ws)
    om[hd] = torch.from_numpy(om_s).to(DEV)
    om = om.view(B, H, 128)
    buf = new_stepq_buffers(w)
    m.stepq_pack(S, om, buf["Z"], buf["R"], buf["C"])
    del S
    torch.cuda.empty_cache()
    err = {"y": 0.0, "r_off": 0, "r_ties": 0, "z_maxdiff": 0, "z_flips": 0, "z_flips_outside_band": 0,
           "c_off": 0, "c_ties": 0, "rows": 0, "steps": 0}
    om64 = om_s.astype(np.float64)
    check_stepq_pack(S_ref, np.abs(S_ref), om64, stepq_host(buf, hd), err)
    y = torch.empty(B, H, 128, device=DEV)
    for t in range(2):
        z, r, c = stepq_host(buf, hd)
        x, d = _inputs(w, ws, hd, t)
        m.gdn_stepq_step(buf["Z"], buf["R"], buf["C"], om, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
        y_ref, _, Xt = sqo.step(z, r, c, om64, *_host(x))
        err["y"] = max(err["y"], rel_err(y.view(N, 128)[hd].cpu().numpy(), y_ref))
        Xp = sqo.decode(z, r, c)
        gX = Xp * np.asarray(x["gate"], np.float64)[:, None, None]
        check_stepq_pack(Xt, np.abs(gX) + np.abs(Xt - gX), om64, stepq_host(buf, hd), err)
    say(f"  {err}")
    assert err["y"] < TOL_F32 and err["r_off"] == 0 and err["c_off"] == 0
    assert err["z_maxdiff"] <= 1 and err["z_flips_outside_band"] == 0
