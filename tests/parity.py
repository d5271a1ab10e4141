"""Helpers of the GPU parity tests: upload seeded inputs, run the HIP path through
the C ABI, run the fp64 oracle on the same inputs (all heads, or sampled heads
at full size), and measure the error as the pages' tolerances define it.

Error metric: for every (head, step), two relative errors over the head's output
vector (or state matrix): the norm-wise ||x_gpu - x_ref||_2 / ||x_ref||_2 and the
element-wise max|x_gpu - x_ref| / max|x_ref|. The larger of the two, maximised over
heads and steps, is compared with the tolerance.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads as wl

DEV = "cuda"
TOL_F32 = 1e-5      # fp32 state and outputs
TOL_Q8 = 1e-4       # outputs of the int8 path against the oracle's same schedule


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rsu():
    import recurrent_state_update_head_amd as m
    return m


def qkv_dtype(w: wl.Workload):
    return torch.bfloat16 if w.qkv == "bf16" else torch.float32


def dev_inputs(w: wl.Workload, t: int):
    """Host inputs of step t (fp32 numpy) and their device tensors in the workload dtype."""
    x = wl.step_inputs(w, t)
    B, H, dt = w.B, w.H, qkv_dtype(w)
    sub = (w.n,) if w.variant == "deltaproduct" else ()   # DeltaProduct: one key, value, beta per sub-step
    d = {"q": torch.from_numpy(x["q"]).to(DEV).to(dt).view(B, H, 128)}
    for n in ("k", "v"):
        d[n] = torch.from_numpy(x[n]).to(DEV).to(dt).view((B, H) + sub + (128,))
    d["gate"] = torch.from_numpy(x["gate"]).to(DEV).view((B, H, 128) if w.per_key_gate else (B, H))
    d["beta"] = torch.from_numpy(x["beta"]).to(DEV).view((B, H) + sub)
    if "kappa" in x:
        d["kappa"] = torch.from_numpy(x["kappa"]).to(DEV).to(dt).view(B, H, 128)
        d["a"] = torch.from_numpy(x["a"]).to(DEV).view(B, H, 128)
    return x, d


def host_slice(x: dict, heads: np.ndarray):
    return tuple(x[n][heads] for n in ("q", "k", "v", "gate", "beta"))


def rel_err_parts(gpu: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    """Both error figures over the trailing axes, maximised over the leading index (one
    head's vector or state matrix at one step): the norm-wise ||gpu - ref||_2 / ||ref||_2
    and the element-wise max|gpu - ref| / max|ref|."""
    g = gpu.reshape(gpu.shape[0], -1).astype(np.float64)
    r = ref.reshape(ref.shape[0], -1).astype(np.float64)
    d = g - r
    norm = np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-300)
    elem = np.max(np.abs(d), axis=1) / np.maximum(np.max(np.abs(r), axis=1), 1e-300)
    return float(np.max(norm)), float(np.max(elem))


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """The larger of the two figures of rel_err_parts: every tolerance bounds both the
    norm-wise error of a head's vector or matrix and its worst single element."""
    return max(rel_err_parts(gpu, ref))


def take(t: torch.Tensor, heads_dev: torch.Tensor, inner) -> np.ndarray:
    return t.reshape((-1,) + tuple(inner))[heads_dev].cpu().numpy()


def run_dense(w: wl.Workload, sample: int | None = None):
    """Dense GDN/KDA/RWKV6 steps on the GPU against the eager oracle; returns (max y err, final S err)."""
    m = rsu()
    B, H = w.B, w.H
    S0 = wl.initial_state(w)
    heads = np.arange(w.heads) if sample is None else wl.sample_heads(w, sample)
    hd = torch.from_numpy(heads).to(DEV)
    S = torch.from_numpy(S0).to(DEV).view(B, H, 128, 128)
    S_ref = S0[heads].astype(np.float64)
    del S0
    y = torch.empty(B, H, 128, device=DEV)
    fn = m.kda_decode_step if w.per_key_gate else m.gdn_decode_step
    worst_y = 0.0
    for t in range(w.steps):
        x, d = dev_inputs(w, t)
        if w.variant == "rwkv6":
            m.rwkv6_decode_step(S, d["q"], d["k"], d["v"], d["gate"], y)
            y_ref = oracle.rwkv6_step(S_ref, *host_slice(x, heads)[:4])
        elif w.variant == "rwkv7":
            m.rwkv7_decode_step(S, d["q"], d["k"], d["v"], d["kappa"], d["gate"], d["a"], y)
            y_ref = oracle.rwkv7_step(S_ref, *host_slice(x, heads)[:4], x["kappa"][heads], x["a"][heads])
        elif w.variant == "deltaproduct":
            m.deltaproduct_decode_step(S, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
            y_ref = oracle.deltaproduct_step(S_ref, *host_slice(x, heads))
        else:
            fn(S, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
            y_ref = oracle.dense_step(S_ref, *host_slice(x, heads))
        worst_y = max(worst_y, rel_err(take(y, hd, (128,)), y_ref))
    worst_S = rel_err(take(S, hd, (128, 128)), S_ref)
    return worst_y, worst_S


def new_log_buffers(w: wl.Workload, C: int):
    B, H = w.B, w.H
    per_key = w.per_key_gate
    cap = max(C, 1)
    return {
        "lbar": torch.zeros((B, H, 128) if per_key else (B, H), device=DEV),
        "Klog": torch.zeros(B, H, cap, 128, device=DEV, dtype=qkv_dtype(w)),
        "Ulog": torch.zeros(B, H, cap, 128, device=DEV,
                            dtype=qkv_dtype(w) if w.variant == "rwkv6" else torch.float32),
        "Lam": torch.zeros((B, H, cap, 128) if per_key else (B, H, cap), device=DEV),
    }


def log_step(w: wl.Workload, C: int, L: int, Sbase, buf, d, y):
    """One base+log step through the C ABI; returns the next L."""
    m = rsu()
    kda = w.per_key_gate
    Klog, Ulog, Lam = (buf["Klog"], buf["Ulog"], buf["Lam"]) if C > 0 else (None, None, None)
    if w.variant == "rwkv6":
        fn = m.rwkv6_log_append if L < C else m.rwkv6_log_merge
        fn(C, L, Sbase, buf["lbar"], Klog, Ulog, Lam, d["q"], d["k"], d["v"], d["gate"], y)
        return L + 1 if L < C else 0
    if L < C:
        (m.kda_log_append if kda else m.gdn_log_append)(
            C, L, Sbase, buf["lbar"], Klog, Ulog, Lam, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
        return L + 1
    (m.kda_log_merge if kda else m.gdn_log_merge)(
        C, L, Sbase, buf["lbar"], Klog, Ulog, Lam, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
    return 0


def run_log(w: wl.Workload, sample: int | None = None, steps: int | None = None):
    """Base+log steps on the GPU against the oracle's base+log steps (which equal eager
    decoding, a pinned property). Returns a dict of max errors."""
    B, H = w.B, w.H
    C = w.M - 1
    steps = w.steps if steps is None else steps
    S0 = wl.initial_state(w)
    heads = np.arange(w.heads) if sample is None else wl.sample_heads(w, sample)
    hd = torch.from_numpy(heads).to(DEV)
    Sbase = torch.from_numpy(S0).to(DEV).view(B, H, 128, 128)
    ref = oracle.LogState(S0[heads].astype(np.float64), C, w.per_key_gate, rwkv6=w.variant == "rwkv6")
    del S0
    buf = new_log_buffers(w, C)
    y = torch.empty(B, H, 128, device=DEV)
    err = {"y": 0.0, "Sbase": 0.0, "lbar": 0.0, "Ulog": 0.0, "Klog": 0.0, "Lam": 0.0}
    L = 0
    for t in range(steps):
        x, d = dev_inputs(w, t)
        L = log_step(w, C, L, Sbase, buf, d, y)
        y_ref = ref.step(*host_slice(x, heads))
        assert L == ref.L
        err["y"] = max(err["y"], rel_err(take(y, hd, (128,)), y_ref))
        if L == 0:
            err["Sbase"] = max(err["Sbase"], rel_err(take(Sbase, hd, (128, 128)), ref.Sbar))
        else:
            m = L - 1
            gd = (128,) if w.per_key_gate else ()
            Ug = take(buf["Ulog"][:, :, m].float(), hd, (128,))
            err["Ulog"] = max(err["Ulog"], rel_err(Ug, ref.U[:, m]))
            Kg = take(buf["Klog"][:, :, m].float(), hd, (128,))
            err["Klog"] = max(err["Klog"], float(np.abs(Kg - ref.K[:, m]).max()))
            lam_g = take(buf["Lam"][:, :, m], hd, gd)
            err["Lam"] = max(err["Lam"], float(np.abs(lam_g - ref.Lam[:, m]).max()))
        lb_g = take(buf["lbar"], hd, (128,) if w.per_key_gate else ())
        err["lbar"] = max(err["lbar"], float(np.abs(lb_g - ref.lbar).max()))
    return err


def run_log_slots(w: wl.Workload, sample: int | None = None, steps: int | None = None,
                  L0: np.ndarray | None = None):
    """Per-slot live lengths: the GPU's *_log_step_slots against the oracle's per-slot
    steps (which equal eager decoding, a pinned property). Heads start at staggered
    points of their cycle (empty entries, K = U = 0, are a valid log of any length),
    so appends and merges of different heads share every launch."""
    m = rsu()
    B, H = w.B, w.H
    C = w.M - 1
    steps = w.steps if steps is None else steps
    S0 = wl.initial_state(w)
    heads = np.arange(w.heads) if sample is None else wl.sample_heads(w, sample)
    hd = torch.from_numpy(heads).to(DEV)
    Sbase = torch.from_numpy(S0).to(DEV).view(B, H, 128, 128)
    ref = oracle.LogState(S0[heads].astype(np.float64), C, w.per_key_gate, rwkv6=w.variant == "rwkv6")
    del S0
    L_all = (np.arange(w.heads, dtype=np.int32) * 5) % (C + 1) if L0 is None else L0.astype(np.int32)
    Ld = torch.from_numpy(L_all.copy()).to(DEV).view(B, H)
    Lref = np.ascontiguousarray(L_all[heads])
    buf = new_log_buffers(w, C)
    Klog, Ulog, Lam = (buf["Klog"], buf["Ulog"], buf["Lam"]) if C > 0 else (None, None, None)
    fn = m.kda_log_step_slots if w.per_key_gate else m.gdn_log_step_slots
    if w.variant == "rwkv6":
        def fn(C, L, Sb, lb, K, U, Lm, q, k, v, g, b, y):
            return m.rwkv6_log_step_slots(C, L, Sb, lb, K, U, Lm, q, k, v, g, y)
    y = torch.empty(B, H, 128, device=DEV)
    err = {"y": 0.0, "Sbase": 0.0, "lbar": 0.0, "Ulog": 0.0, "Klog": 0.0, "Lam": 0.0, "L": 0,
           "merges": 0, "appends": 0}
    gd = (128,) if w.per_key_gate else ()
    for t in range(steps):
        x, d = dev_inputs(w, t)
        fn(C, Ld, Sbase, buf["lbar"], Klog, Ulog, Lam, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
        y_ref = ref.step_slots(Lref, *host_slice(x, heads))
        Lg = take(Ld, hd, ())
        err["L"] = max(err["L"], int(np.abs(Lg - Lref).max()))
        err["y"] = max(err["y"], rel_err(take(y, hd, (128,)), y_ref))
        merged = np.flatnonzero(Lref == 0)
        appended = np.flatnonzero(Lref > 0)
        err["merges"] += len(merged)
        err["appends"] += len(appended)
        if len(merged):
            Sg = take(Sbase, hd[torch.from_numpy(merged).to(DEV)], (128, 128))
            err["Sbase"] = max(err["Sbase"], rel_err(Sg, ref.Sbar[merged]))
        for i in appended:
            mm = int(Lref[i]) - 1
            h = hd[i:i + 1]
            err["Ulog"] = max(err["Ulog"], rel_err(take(buf["Ulog"][:, :, mm].float(), h, (128,)),
                                                   ref.U[i:i + 1, mm]))
            err["Klog"] = max(err["Klog"], float(np.abs(take(buf["Klog"][:, :, mm].float(), h, (128,)) -
                                                         ref.K[i:i + 1, mm]).max()))
            err["Lam"] = max(err["Lam"], float(np.abs(take(buf["Lam"][:, :, mm], h, gd) -
                                                      ref.Lam[i:i + 1, mm]).max()))
        err["lbar"] = max(err["lbar"], float(np.abs(take(buf["lbar"], hd, gd) - ref.lbar).max()))
    return err


def new_lq_buffers(w: wl.Workload):
    B, H, W = w.B, w.H, w.W
    r = 8 if w.bits == 4 else 4
    return {
        "Z": (torch.zeros(B, H, 128, 128 * w.bits // 8, device=DEV, dtype=torch.uint8) if w.bits != 8 else
              torch.zeros(B, H, 128, 128, device=DEV, dtype=torch.int8)),
        "B": torch.zeros(B, H, 128, device=DEV),
        "C": torch.zeros(B, H, 128, device=DEV),
        "Kc": torch.zeros(B, H, r, 128, device=DEV, dtype=torch.float16),
        "Uc": torch.zeros(B, H, r, 128, device=DEV, dtype=torch.float16),
        "Kbuf": torch.zeros(B, H, W, 128, device=DEV, dtype=qkv_dtype(w)),
        "Ubuf": torch.zeros(B, H, W, 128, device=DEV),
        "Gbuf": torch.zeros((B, H, W, 128) if w.per_key_gate else (B, H, W), device=DEV),
    }


def lq_host(buf, hd):
    """The GPU's representation of the sampled heads: Z, B, c, and the tokens as [n, 128, r]
    (4-bit codes unpacked from their nibbles, 6-bit codes from their two parts)."""
    from oracle import lq as lqo
    if buf["Z"].dtype == torch.uint8 and buf["Z"].shape[-1] == 96:
        Z = lqo.unpack6(take(buf["Z"], hd, (128, 96))).astype(np.int64)
    elif buf["Z"].dtype == torch.uint8:
        Z = lqo.unpack_nibbles(take(buf["Z"], hd, (128, 64))).astype(np.int64)
    else:
        Z = take(buf["Z"], hd, (128, 128)).astype(np.int64)
    r = buf["Kc"].shape[2]
    Bc = take(buf["B"], hd, (128,)).astype(np.float64)
    C = take(buf["C"], hd, (128,)).astype(np.float64)
    K16 = np.transpose(take(buf["Kc"].float(), hd, (r, 128)), (0, 2, 1)).astype(np.float64)
    U16 = np.transpose(take(buf["Uc"].float(), hd, (r, 128)), (0, 2, 1)).astype(np.float64)
    return Z, Bc, C, K16, U16


def check_lq_refit(S_ref, V0, n_iter, rep, err, tie_band=1e-3, mat_rel=1e-6, qmax=127):
    """Teacher-forced check of one refit.

    Tokens: against the oracle's fit of the same state from the same start (the
    product K U^T, each key token, each value-vector entry; fp16 rounding level).
    Residual pieces: recomputed by the oracle from the GPU's own fp16 tokens. The
    residual R = S - K U^T cancels most of S where the tokens sit (the outlier rows
    and columns), so the GPU's fp32 state error, relative to the uncancelled
    magnitude m = |S| + |K U^T|, is what the GPU's c and B inherit: their errors are
    measured against m (mean of m per row for c^2, max of m / c per column for B).
    Codes are recomputed from the GPU's own c and B; a code may differ by 1 only where
    the exact code lies within 1e-3 LSB of a tie, widened by mat_rel * m in LSB units."""
    from oracle import lq as lqo
    Z, Bc, C, K16, U16 = rep
    for i in range(S_ref.shape[0]):
        K, U = lqo.fit(S_ref[i], V0[i], n_iter)
        Kr, Ur = lqo.to_fp16(K), lqo.to_fp16(U)
        Pg, Pr = K16[i] @ U16[i].T, Kr @ Ur.T
        err["tok"] = max(err["tok"], float(np.linalg.norm(Pg - Pr) / max(np.linalg.norm(Pr), 1e-300)))
        kmax = max(np.linalg.norm(Kr, axis=0).max(), 1e-300)
        err["tok_k"] = max(err["tok_k"], float(np.linalg.norm(K16[i] - Kr, axis=0).max() / kmax))
        err["tok_u"] = max(err["tok_u"], float(np.abs(U16[i] - Ur).max()))
        R = S_ref[i] - Pg
        mag = np.abs(S_ref[i]) + np.abs(Pg)
        c_ref = np.maximum(np.sqrt(np.mean(np.abs(R), axis=1)), lqo.C_FLOOR)
        err["c"] = max(err["c"], float(np.max(np.abs(C[i] ** 2 - c_ref ** 2) / np.mean(mag, axis=1))))
        X = R / C[i][:, None]
        B_ref = np.max(np.abs(X), axis=0)
        xmag = np.max(mag / C[i][:, None], axis=0)
        err["B"] = max(err["B"], float(np.max(np.abs(Bc[i] - B_ref) / np.maximum(xmag, 1e-300))))
        nz = Bc[i] > 0
        w = np.zeros_like(X)
        w[:, nz] = X[:, nz] * float(qmax) / Bc[i][nz][None, :]
        Zr = np.clip(np.rint(w), -qmax, qmax).astype(np.int64)
        dz = np.abs(Z[i] - Zr)
        err["z_maxdiff"] = max(err["z_maxdiff"], int(dz.max()))
        flips = dz > 0
        err["z_flips"] += int(flips.sum())
        band = np.full_like(w, tie_band)
        band[:, nz] += mat_rel * float(qmax) * (mag[:, nz] / C[i][:, None]) / Bc[i][nz][None, :]
        near = np.abs(np.abs(w - np.floor(w)) - 0.5) < band
        err["z_flips_outside_band"] += int((flips & ~near).sum())


def run_lq(w: wl.Workload, n_iter: int = 1, n_iter0: int = 8, sample: int | None = None,
           steps: int | None = None):
    """LeapQuant's format on the GPU against the oracle, teacher-forced per window: the
    conversion of the initial state, every in-window output against dense decoding from
    the GPU's window-start representation, and every boundary refit."""
    from oracle import lq as lqo
    m = rsu()
    B, H, W = w.B, w.H, w.W
    steps = w.steps if steps is None else steps
    S0 = wl.initial_state(w)
    heads = np.arange(w.heads) if sample is None else wl.sample_heads(w, sample)
    hd = torch.from_numpy(heads).to(DEV)
    buf = new_lq_buffers(w)
    Sd = torch.from_numpy(S0).to(DEV).view(B, H, 128, 128)
    quantize = m.kda_lq_quantize if w.per_key_gate else m.gdn_lq_quantize
    window = m.kda_lq_window if w.per_key_gate else m.gdn_lq_window
    if w.bits == 4:
        quantize, window = ((m.kda_lq4_quantize, m.kda_lq4_window) if w.per_key_gate else
                            (m.gdn_lq4_quantize, m.gdn_lq4_window))
    if w.bits == 6:
        quantize, window = ((m.kda_lq6_quantize, m.kda_lq6_window) if w.per_key_gate else
                            (m.gdn_lq6_quantize, m.gdn_lq6_window))
    qmax = lqo.qmax_of(w.bits)
    r = 8 if w.bits == 4 else 4
    quantize(Sd, n_iter0, buf["Z"], buf["B"], buf["C"], buf["Kc"], buf["Uc"])
    err = {"y": 0.0, "tok": 0.0, "tok_k": 0.0, "tok_u": 0.0, "c": 0.0, "B": 0.0, "z_maxdiff": 0,
           "z_flips": 0, "z_flips_outside_band": 0, "boundaries": 0}
    S_ref = S0[heads].astype(np.float64)
    del Sd, S0
    walsh = np.broadcast_to(lqo.walsh_start(r=r), (len(heads), 128, r))
    check_lq_refit(S_ref, walsh, n_iter0, lq_host(buf, hd), err, qmax=qmax)
    y = torch.empty(B, H, 128, device=DEV)
    for t0 in range(0, steps, W):
        rep = lq_host(buf, hd)
        S = np.stack([lqo.represent(rep[0][i], rep[1][i], rep[2][i], rep[3][i], rep[4][i], qmax=qmax)
                      for i in range(len(heads))])
        n = min(W, steps - t0)
        for pos in range(n):
            x, d = dev_inputs(w, t0 + pos)
            window(W, pos, n_iter, buf["Z"], buf["B"], buf["C"], buf["Kc"], buf["Uc"], buf["Kbuf"],
                   buf["Ubuf"], buf["Gbuf"], d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
            y_ref = oracle.dense_step(S, *host_slice(x, heads))
            err["y"] = max(err["y"], rel_err(take(y, hd, (128,)), y_ref))
        if n == W:
            check_lq_refit(S, rep[4], n_iter, lq_host(buf, hd), err, qmax=qmax)
            err["boundaries"] += 1
    return err


def new_window_buffers(w: wl.Workload):
    B, H, W = w.B, w.H, w.W
    if w.variant == "rwkv7":   # two records per token, per-key gates
        return {
            "Z": torch.zeros(B, H, 128, 128, device=DEV, dtype=torch.int8),
            "A": torch.zeros(B, H, 128, device=DEV),
            "Kbuf": torch.zeros(B, H, 2 * W, 128, device=DEV, dtype=qkv_dtype(w)),
            "Ubuf": torch.zeros(B, H, 2 * W, 128, device=DEV),
            "Gbuf": torch.zeros(B, H, 2 * W, 128, device=DEV),
        }
    if w.variant == "deltaproduct":   # one record per sub-step, scalar gates
        R = w.n * W
        return {
            "Z": torch.zeros(B, H, 128, 128, device=DEV, dtype=torch.int8),
            "A": torch.zeros(B, H, 128, device=DEV),
            "Kbuf": torch.zeros(B, H, R, 128, device=DEV, dtype=qkv_dtype(w)),
            "Ubuf": torch.zeros(B, H, R, 128, device=DEV),
            "Gbuf": torch.zeros(B, H, R, device=DEV),
        }
    return {
        "Z": torch.zeros(B, H, 128, 128, device=DEV, dtype=torch.int8),
        "A": torch.zeros(B, H, 128, device=DEV),
        "Kbuf": torch.zeros(B, H, W, 128, device=DEV, dtype=qkv_dtype(w)),
        "Ubuf": torch.zeros(B, H, W, 128, device=DEV),
        "Gbuf": torch.zeros((B, H, W, 128) if w.per_key_gate else (B, H, W), device=DEV),
    }


def window_step(w: wl.Workload, pos: int, buf, d, y):
    m = rsu()
    if w.variant == "rwkv7":
        m.rwkv7_q8_window(w.W, pos, buf["Z"], buf["A"], buf["Kbuf"], buf["Ubuf"], buf["Gbuf"], d["q"], d["k"],
                          d["v"], d["kappa"], d["gate"], d["a"], y)
        return
    if w.variant == "deltaproduct":
        m.deltaproduct_q8_window(w.W, pos, buf["Z"], buf["A"], buf["Kbuf"], buf["Ubuf"], buf["Gbuf"], d["q"],
                                 d["k"], d["v"], d["gate"], d["beta"], y)
        return
    fn = m.kda_q8_window if w.per_key_gate else m.gdn_q8_window
    fn(w.W, pos, buf["Z"], buf["A"], buf["Kbuf"], buf["Ubuf"], buf["Gbuf"], d["q"], d["k"], d["v"],
       d["gate"], d["beta"], y)


def run_window(w: wl.Workload, sample: int | None = None, steps: int | None = None,
               tie_band: float = 1e-3, a_abs: float = 0.0):
    """Int8 per-window path on the GPU against the oracle, teacher-forced per window:
    at every window start the oracle restarts from the GPU's (Z, a), so a 1-LSB
    rounding-tie flip at one boundary is not carried into later windows.
    Returns a dict: max y error, max row-scale relative error (beyond an absolute slack
    a_abs), and code statistics at the boundaries (max |dZ|, flips, flips outside the tie
    band)."""
    m = rsu()
    B, H, W = w.B, w.H, w.W
    steps = w.steps if steps is None else steps
    S0 = wl.initial_state(w)
    heads = np.arange(w.heads) if sample is None else wl.sample_heads(w, sample)
    hd = torch.from_numpy(heads).to(DEV)
    buf = new_window_buffers(w)
    S0_dev = torch.from_numpy(S0).to(DEV).view(B, H, 128, 128)
    m.q8_quantize(S0_dev, buf["Z"], buf["A"])
    Zr, ar = oracle.q8_quantize(S0[heads].astype(np.float64))
    del S0, S0_dev
    st = {"init_codes_equal": bool(np.array_equal(take(buf["Z"], hd, (128, 128)), Zr)),
          "init_scales_equal": bool(np.array_equal(take(buf["A"], hd, (128,)), ar)),
          "y": 0.0, "a": 0.0, "z_maxdiff": 0, "z_flips": 0, "z_flips_outside_band": 0,
          "boundaries": 0}
    y = torch.empty(B, H, 128, device=DEV)
    ref = None
    for t in range(steps):
        pos = t % W
        if pos == 0:
            Zs, As = take(buf["Z"], hd, (128, 128)), take(buf["A"], hd, (128,))
            if w.variant == "rwkv7":
                ref = oracle.Rwkv7WindowState(Zs, As, W)
            elif w.variant == "deltaproduct":
                ref = oracle.DeltaProductWindowState(Zs, As, W, w.n)
            else:
                ref = oracle.WindowState(Zs, As, W, w.per_key_gate)
        x, d = dev_inputs(w, t)
        window_step(w, pos, buf, d, y)
        args = host_slice(x, heads)
        if w.variant == "rwkv7":
            args = args[:4] + (x["kappa"][heads], x["a"][heads])
        if pos == W - 1:
            y_ref, _, wcode = ref.step(*args, want_boundary=True)
            Zg = take(buf["Z"], hd, (128, 128)).astype(np.int32)
            ag = take(buf["A"], hd, (128,)).astype(np.float64)
            aref = ref.a.astype(np.float64)
            st["a"] = max(st["a"], float(np.max(np.maximum(np.abs(ag - aref) - a_abs, 0.0) /
                                                np.maximum(aref, 1e-300))))
            diff = Zg - ref.Z.astype(np.int32)
            flips = diff != 0
            near_tie = np.abs(np.abs(wcode - np.floor(wcode)) - 0.5) < tie_band
            st["z_maxdiff"] = max(st["z_maxdiff"], int(np.abs(diff).max()))
            st["z_flips"] += int(flips.sum())
            st["z_flips_outside_band"] += int((flips & ~near_tie).sum())
            st["boundaries"] += 1
        else:
            y_ref = ref.step(*args)
        st["y"] = max(st["y"], rel_err(take(y, hd, (128,)), y_ref))
    return st


def new_stepq_buffers(w: wl.Workload):
    B, H = w.B, w.H
    return {
        "Z": torch.zeros(B, H, 128, 64, device=DEV, dtype=torch.uint8),
        "R": torch.zeros(B, H, 128, device=DEV, dtype=torch.float16),
        "C": torch.zeros(B, H, 128, device=DEV, dtype=torch.float16),
    }


def stepq_host(buf, hd):
    """The GPU's packed state of the sampled heads: codes [n, 128, 128], R, C (fp64)."""
    from oracle import lq as lqo
    z = lqo.unpack_nibbles(take(buf["Z"], hd, (128, 64))).astype(np.int64)
    r = take(buf["R"].float(), hd, (128,)).astype(np.float64)
    c = take(buf["C"].float(), hd, (128,)).astype(np.float64)
    return z, r, c


def _fp16_rounding_ok(got, exact, rel_band):
    """got == fp16(exact), or exact lies within rel_band * |exact| of the midpoint between
    got and fp16(exact) (a tie the GPU's fp32 arithmetic may round either way). Returns the
    masks (off: wrong outside the band, tie: differs inside it)."""
    from oracle import stepq as sqo
    ref = sqo.to_fp16(exact)
    diff = got != ref
    near = np.abs(exact - 0.5 * (got + ref)) <= rel_band * np.abs(exact)
    return diff & ~near, diff & near


def check_stepq_pack(X, mag, omega, rep, err, tie_band=1e-4, mat_rel=1e-6, rel_band=2e-5):
    """Teacher-forced check of the packing of the fp64 states X [n, 128, 128].

    mag bounds the magnitude the GPU's fp32 X was formed from (|X| itself for a packed
    input state; |g X_prev| + |k u^T| after a step): the GPU's elements carry errors of
    about mat_rel * mag. Row factors: the GPU's R is the fp16 rounding of the exact
    sqrt(m_i / w_i), except within a relative band of a rounding midpoint. Codes:
    recomputed from the GPU's own R; a code may differ by 1 only within tie_band (plus
    mat_rel * mag in code units) of a tie. Column factors: recomputed in fp64 from the
    GPU's own R and codes; the GPU's C is their fp16 rounding up to a band at midpoints.
    A column whose range a_j is below 2^-64 has a column factor of about a_j / 7, which is
    zero in fp16 on both sides (and checked as such), so it decodes to zero whatever its
    codes: those codes are not compared (the GPU caps 7 / a_j where it overflows fp32)."""
    from oracle import stepq as sqo
    z, r, c = rep
    W = sqo.row_weights(omega)
    qmax = sqo.QMAX4
    for i in range(X.shape[0]):
        p = sqo.pack(X[i], W[i])
        m = np.mean(np.abs(X[i]), axis=1)
        band_r = rel_band + mat_rel * np.mean(mag[i], axis=1) / np.maximum(m, 1e-300)
        off, tie = _fp16_rounding_ok(r[i], p["r_pre"], band_r)
        err["r_off"] += int(off.sum())
        err["r_ties"] += int(tie.sum())
        live = r[i] > 0
        U = np.zeros_like(X[i])
        U[live] = X[i][live] / r[i][live][:, None]
        a = np.max(np.abs(U), axis=0)
        cols = a > 0
        code = np.zeros_like(U)
        code[:, cols] = U[:, cols] * (qmax / a[cols])[None, :]
        Zr = np.clip(np.rint(code), -qmax, qmax).astype(np.int64)
        dz = np.abs(z[i] - Zr)
        dz[:, a < 2.0 ** -64] = 0
        err["z_maxdiff"] = max(err["z_maxdiff"], int(dz.max()))
        flips = dz > 0
        err["z_flips"] += int(flips.sum())
        band = np.full_like(code, tie_band)
        rr = np.where(live, r[i], np.inf)[:, None]
        band[:, cols] += mat_rel * qmax * (mag[i][:, cols] / rr) / a[cols][None, :]
        near = np.abs(np.abs(code - np.floor(code)) - 0.5) < band
        tiny = a < 2.0 ** -64
        flips[:, tiny] = False
        err["tiny_cols"] = err.get("tiny_cols", 0) + int(tiny.sum())
        err["z_flips_outside_band"] += int((flips & ~near).sum())
        zf = z[i].astype(np.float64)
        cp = sqo.column_factors(X[i], r[i], zf, W[i])
        wr = (W[i] ** 2 * r[i])[:, None]
        num_abs = np.sum(wr * np.abs(zf) * mag[i], axis=0)
        num = np.abs(np.sum(wr * zf * X[i], axis=0))
        band_c = rel_band + mat_rel * num_abs / np.maximum(num, 1e-300)
        off, tie = _fp16_rounding_ok(c[i], cp, band_c)
        err["c_off"] += int(off.sum())
        err["c_ties"] += int(tie.sum())
        err["rows"] += X.shape[1]


def run_stepq(w: wl.Workload, sample: int | None = None, steps: int | None = None, S0=None, om=None):
    """The packed state on the GPU against the oracle, teacher-forced per step: the packing
    of the initial state, then for every step the output against the dense step from the
    GPU's packed state before it, and the packing of the resulting state."""
    from oracle import stepq as sqo
    m = rsu()
    B, H = w.B, w.H
    steps = w.steps if steps is None else steps
    if S0 is None:
        S0 = wl.initial_state(w)
    if om is None:
        om = wl.row_influence(w)
    heads = np.arange(w.heads) if sample is None else wl.sample_heads(w, sample)
    hd = torch.from_numpy(heads).to(DEV)
    buf = new_stepq_buffers(w)
    omega = torch.from_numpy(om).to(DEV).view(B, H, 128)
    Sd = torch.from_numpy(S0).to(DEV).view(B, H, 128, 128)
    m.stepq_pack(Sd, omega, buf["Z"], buf["R"], buf["C"])
    err = {"y": 0.0, "r_off": 0, "r_ties": 0, "z_maxdiff": 0, "z_flips": 0, "z_flips_outside_band": 0,
           "c_off": 0, "c_ties": 0, "rows": 0, "steps": 0}
    X0 = S0[heads].astype(np.float64)
    del Sd, S0
    om_s = om[heads].astype(np.float64)
    check_stepq_pack(X0, np.abs(X0), om_s, stepq_host(buf, hd), err)
    step = m.kda_stepq_step if w.per_key_gate else m.gdn_stepq_step
    y = torch.empty(B, H, 128, device=DEV)
    for t in range(steps):
        z, r, c = stepq_host(buf, hd)
        x, d = dev_inputs(w, t)
        step(buf["Z"], buf["R"], buf["C"], omega, d["q"], d["k"], d["v"], d["gate"], d["beta"], y)
        q, k, v, g, b = host_slice(x, heads)
        y_ref, _, Xt = sqo.step(z, r, c, om_s, q, k, v, g, b)
        err["y"] = max(err["y"], rel_err(take(y, hd, (128,)), y_ref))
        Xp = sqo.decode(z, r, c)
        gX = Xp * (np.asarray(g, np.float64)[:, :, None] if g.ndim == 2 else np.asarray(g, np.float64)[:, None, None])
        check_stepq_pack(Xt, np.abs(gX) + np.abs(Xt - gX), om_s, stepq_host(buf, hd), err)
        err["steps"] += 1
    return err
