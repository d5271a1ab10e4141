#!/usr/bin/env python3
"""Benchmark of the batched decode-step update + readout of delta-rule states on one GPU.

Default workload: Gated DeltaNet dense fp32 state, B=256 requests x H=48 heads,
128x128 state per head (805 MB), bf16 q/k/v, 16 distinct steps of seeded
synthetic inputs resident in HBM (cycled when more steps are timed).

One "step" is one decode step of the whole batch: one launch of the dense step
kernel (gate, k-read, correction, rank-one update, readout) over all B*H heads.

Prints ONE JSON line on stdout:
  value = state head-updates per second (B*H*K / timed seconds),
  roofline = algorithmic HBM bytes per launch / average launch time vs 8 TB/s,
  hbm_ceiling = read-only and write-only stream rates of the same tile pattern over the
    state's size, and the step time they imply (bytes read / R + bytes written / W),
  other_configs = GPU-only lines of the KDA, int8-window and base+log workloads,
  cpu_baseline = the fp64 oracle timed on the host cores on a bounded sample.
Other workloads (--workload kda|q8|log|lq|kda_lq|lq4|rwkv6|rwkv6_log|rwkv7|rwkv7_q8|
stepq|dp|dp_q8|gdn_small) report the same fields for their own kernels, with the CPU baseline
timing the oracle of their own path; they are measurements, not the headline line.
Per-launch timing of window positions / log lengths goes to "phases", a launch-by-launch
pass to "step_time_distribution"; --graph replays the timed steps as one HIP graph and
--split (stepq) runs the readout and the repack on two streams.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "state head-updates/sec and achieved HBM GB/s (% of peak), B=256 H=48 decode"
PEAK_HBM_GBS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "counters_gdn_dense_b256_h48.txt")
KERNEL_SOURCES = {
    "dense": ["recurrent_state_update_head_amd/csrc/dense.hip",
              "recurrent_state_update_head_amd/csrc/rsu_device.hpp"],
}

WORKLOAD_BY_FLAG = {"gdn": 2, "gdn_small": 1, "kda": 3, "q8": 4, "log": 5, "lq": 6, "rwkv6": 7,
                    "rwkv6_log": 8, "kda_lq": 9, "rwkv7": 10, "rwkv7_q8": 11, "lq4": 12,
                    "stepq": 13, "dp": 14, "dp_q8": 15, "lq6": 16, "kda_lq4": 17, "kda_lq6": 18}
LQ_TOKENS = 4


# ----------------------------------------------------------------- byte accounting

def _in_bytes(w: wl.Workload) -> int:
    return 2 if w.qkv == "bf16" else 4


def _beta_bytes(w: wl.Workload) -> int:
    return 0 if w.variant in ("rwkv6", "rwkv7") else 4     # RWKV6 / RWKV7 have no write strength


def dense_bytes_per_head(w: wl.Workload) -> int:
    """State read + write (fp32), q/k/v in their dtype, gate, beta, y (fp32)."""
    d = wl.DK
    gate = 4 * d if w.per_key_gate else 4
    if w.variant == "deltaproduct":   # n keys, n values and n betas per token
        return 2 * 4 * d * d + (1 + 2 * w.n) * d * _in_bytes(w) + gate + 4 * w.n + 4 * d
    extra = d * _in_bytes(w) + 4 * d if w.variant == "rwkv7" else 0     # RWKV7's kappa and erase rate a
    return 2 * 4 * d * d + 3 * d * _in_bytes(w) + gate + _beta_bytes(w) + 4 * d + extra


def window_step_bytes_per_head(w: wl.Workload, pos: int) -> int:
    """Int8 window step at position pos: codes + row scales, the pos records read,
    the step inputs, y, and either the record write or (at the boundary) the
    requantized codes and scales."""
    d = wl.DK
    gdim = d if w.per_key_gate else 1
    rec = d * _in_bytes(w) + 4 * d + 4 * gdim
    inputs = 3 * d * _in_bytes(w) + 4 * gdim + 4
    if w.variant == "rwkv7":
        return rwkv7_window_step_bytes_per_head(w, pos)
    if w.variant == "deltaproduct":
        return dp_window_step_bytes_per_head(w, pos)
    rd = d * d + 4 * d + pos * rec + inputs
    wr = 4 * d + ((d * d + 4 * d) if pos == w.W - 1 else rec)
    return rd + wr


def rwkv7_window_step_bytes_per_head(w: wl.Workload, pos: int) -> int:
    """RWKV7 on the int8 window, two records per token: the step reads codes + row scales,
    its 2 pos records (key in the input dtype, value and per-key gate fp32), q, k, v, kappa,
    w and a, and writes y and its two records; at the last token a second pass reads the
    codes, scales and all 2W records and writes the requantized codes and scales."""
    d = wl.DK
    rec = d * _in_bytes(w) + 4 * d + 4 * d
    inputs = 4 * d * _in_bytes(w) + 2 * 4 * d
    rd = d * d + 4 * d + 2 * pos * rec + inputs
    wr = 4 * d + 2 * rec
    if pos == w.W - 1:
        rd += d * d + 4 * d + 2 * w.W * rec
        wr += d * d + 4 * d
    return rd + wr


def dp_window_step_bytes_per_head(w: wl.Workload, pos: int) -> int:
    """DeltaProduct on the int8 window, one record per sub-step (key in the input dtype, value
    fp32, scalar gate fp32): the step reads codes + row scales, its n pos records, q, the n
    keys, values and betas and alpha, and writes y and its n records; at the last token a
    second pass reads the codes, scales and all nW records and writes the requantized codes
    and scales."""
    d, n = wl.DK, w.n
    rec = d * _in_bytes(w) + 4 * d + 4
    inputs = (1 + 2 * n) * d * _in_bytes(w) + 4 + 4 * n
    rd = d * d + 4 * d + n * pos * rec + inputs
    wr = 4 * d + n * rec
    if pos == w.W - 1:
        rd += d * d + 4 * d + n * w.W * rec
        wr += d * d + 4 * d
    return rd + wr


def lq_step_bytes_per_head(w: wl.Workload, pos: int) -> int:
    """LeapQuant-format window step at position pos: payload codes, per-column absmax and
    per-row smoothing scales, the fp16 token pairs, the pos records, the step inputs, y,
    and either the record write or (at the boundary) the whole new representation."""
    d = wl.DK
    gdim = d if w.per_key_gate else 1
    rec = d * _in_bytes(w) + 4 * d + 4 * gdim
    inputs = 3 * d * _in_bytes(w) + 4 * gdim + 4
    r = 8 if w.bits == 4 else LQ_TOKENS
    rep = d * d * w.bits // 8 + 4 * d + 4 * d + 2 * r * d * 2
    rd = rep + pos * rec + inputs
    wr = 4 * d + (rep if pos == w.W - 1 else rec)
    return rd + wr


def stepq_bytes_per_head(w: wl.Workload) -> int:
    """Packed-state step: the 4-bit codes and the fp16 row and column factors read and
    written, the fp32 row influence scores read, the step inputs, y."""
    d = wl.DK
    gate = 4 * d if w.per_key_gate else 4
    packed = d * d // 2 + 2 * d + 2 * d
    return 2 * packed + 4 * d + 3 * d * _in_bytes(w) + gate + _beta_bytes(w) + 4 * d


def log_step_bytes_per_head(w: wl.Workload, L: int) -> int:
    """Base+log step with L live entries: base read, L entries read, lbar, inputs,
    y, and either the entry + lbar write (append) or the base + lbar write (merge).
    Entries hold k in the input dtype, the value factor in fp32 (delta rule) or in the
    input dtype (RWKV6's raw value), and the log-decay snapshot."""
    d = wl.DK
    C = w.M - 1
    gdim = d if w.per_key_gate else 1
    ubytes = _in_bytes(w) if w.variant == "rwkv6" else 4
    ent = d * _in_bytes(w) + ubytes * d + 4 * gdim
    inputs = 3 * d * _in_bytes(w) + 4 * gdim + _beta_bytes(w)
    rd = 4 * d * d + L * ent + 4 * gdim + inputs
    wr = 4 * d + (4 * d * d + 4 * gdim if L == C else ent + 4 * gdim)
    return rd + wr


def slot_lengths(w: wl.Workload) -> np.ndarray:
    """Initial per-slot live lengths of the mixed-phase log benchmark: every request-head
    at a seeded random point of its cycle (requests admitted at unrelated times), so
    about 1/M of the heads merge at each step, spread over the whole grid."""
    rng = np.random.Generator(np.random.SFC64(np.random.SeedSequence([w.seed, 77])))
    return rng.integers(0, w.M, size=w.heads).astype(np.int32)


def slots_bytes_per_head(w: wl.Workload) -> float:
    """Average algorithmic bytes per head-update of a mixed-phase step (the multiset of
    live lengths is the same at every step)."""
    counts = np.bincount(slot_lengths(w), minlength=w.M)
    return float(sum(int(counts[L]) * log_step_bytes_per_head(w, L) for L in range(w.M))) / w.heads


def cycle_bytes_per_head(w: wl.Workload) -> float:
    """Average algorithmic bytes per head-update over one window / merge cycle."""
    if w.path == "dense":
        return float(dense_bytes_per_head(w))
    if w.path == "stepq":
        return float(stepq_bytes_per_head(w))
    if w.path == "q8_window":
        return sum(window_step_bytes_per_head(w, p) for p in range(w.W)) / w.W
    if w.path == "lq_window":
        return sum(lq_step_bytes_per_head(w, p) for p in range(w.W)) / w.W
    return sum(log_step_bytes_per_head(w, L) for L in range(w.M)) / w.M


# ----------------------------------------------------------------- counters on file

def kernel_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(bytes_per_launch: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    kv = {}
    for line in open(PROFILE_COUNTERS):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_hash") != kernel_hash("dense"):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------- GPU runs

def _dev_inputs(w, steps, torch, dev):
    """All steps' inputs stacked on the device: dict of [steps, B, H, ...] tensors."""
    dt = torch.bfloat16 if w.qkv == "bf16" else torch.float32
    B, H = w.B, w.H
    names = ("q", "k", "v", "gate", "beta") + (("kappa", "a") if w.variant == "rwkv7" else ())
    sub = (w.n,) if w.variant == "deltaproduct" else ()   # DeltaProduct: per-sub-step k, v, beta
    out = {n: [] for n in names}
    for t in range(steps):
        x = wl.step_inputs(w, t)
        for n in ("q", "k", "v") + (("kappa",) if w.variant == "rwkv7" else ()):
            shape = (B, H) + (sub if n in ("k", "v") else ()) + (128,)
            out[n].append(torch.from_numpy(x[n]).to(dev).to(dt).view(shape))
        if w.variant == "rwkv7":
            out["a"].append(torch.from_numpy(x["a"]).to(dev).view(B, H, 128))
        out["gate"].append(torch.from_numpy(x["gate"]).to(dev).view((B, H, 128) if w.per_key_gate else (B, H)))
        out["beta"].append(torch.from_numpy(x["beta"]).to(dev).view((B, H) + sub))
    return {n: torch.stack(v) for n, v in out.items()}


def dense_rw_bytes_per_head(w: wl.Workload) -> tuple[int, int]:
    """(bytes read, bytes written) of one dense step per head: the state both ways, the
    inputs read, y written."""
    total = dense_bytes_per_head(w)
    written = 4 * wl.DK * wl.DK + 4 * wl.DK
    return total - written, written


def _time_calls(torch, call, reps: int = 10, trials: int = 3) -> float:
    """Median over trials of the average launch time (s) of `reps` back-to-back calls, with
    HIP events on the stream the calls launch on (torch's current stream)."""
    stream = torch.cuda.current_stream()
    call()
    torch.cuda.synchronize()
    out = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / 1e3 / reps)
    return float(np.median(out))


def hbm_ceiling(torch, rsu, tiles: int, read_bytes: float, write_bytes: float, step_sec: float) -> dict:
    """The HBM read rate R and write rate W of streams with the dense step's tile pattern
    over `tiles` 64 KiB tiles (the size of the step's state), and the time a step that
    reads read_bytes and writes write_bytes would take at those rates one after the
    other: read_bytes / R + write_bytes / W. A copy into a second buffer is reported
    beside them; it is not a bound of the in-place step."""
    src = torch.empty(tiles, 128, 128, device="cuda").uniform_()
    sums = torch.empty(tiles, 128, device="cuda")
    dst = torch.empty_like(src)
    nbytes = tiles * 128 * 128 * 4
    t_r = _time_calls(torch, lambda: rsu.read_f32(src, sums))
    t_w = _time_calls(torch, lambda: rsu.fill_f32(dst, 0.5))
    t_c = _time_calls(torch, lambda: rsu.copy_f32(src, dst))
    del src, sums, dst
    R, W = nbytes / t_r, nbytes / t_w
    ceil_sec = read_bytes / R + write_bytes / W
    return {"read_GBps": R / 1e9, "write_GBps": W / 1e9, "copy_GBps": 2 * nbytes / t_c / 1e9,
            "bytes_read_per_step": read_bytes, "bytes_written_per_step": write_bytes,
            "ceiling_us": ceil_sec * 1e6, "step_us": step_sec * 1e6, "frac_of_ceiling": ceil_sec / step_sec,
            "ceiling_GBps": (read_bytes + write_bytes) / ceil_sec / 1e9,
            "probes": "rsu_read_f32 / rsu_fill_f32 / rsu_copy_f32 over the state's size, same tile pattern"}


def run_gpu(w: wl.Workload, steps: int, warmup: int, slots: bool = False, n_iter: int = 1, graph: bool = False,
            split: bool = False, measure_ceiling: bool = True, layers: int = 1):
    import torch
    import recurrent_state_update_head_amd as rsu
    dev = "cuda"
    B, H = w.B, w.H
    n_inputs = {"dense": w.steps, "stepq": w.steps, "q8_window": w.W, "lq_window": w.W, "log": w.M}[w.path]
    n_inputs = min(n_inputs, max(1, w.steps))
    x = _dev_inputs(w, n_inputs, torch, dev)
    # the per-step views, made once: indexing five or six tensors in every step costs the host
    # a few microseconds, which matters beside launches of 20-30 us
    xv = [{name: t[i] for name, t in x.items()} for i in range(n_inputs)]
    y = torch.empty(B, H, 128, device=dev)
    S0 = torch.from_numpy(wl.initial_state(w)).to(dev).view(B, H, 128, 128)
    kda = w.per_key_gate
    state = {"t": 0}
    drain = None  # set where launches can still run on another stream when a step returns

    if w.path == "dense" and w.variant == "rwkv7":
        S = S0

        def step():
            i = state["t"] % n_inputs
            rsu.rwkv7_decode_step(S, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["kappa"], xv[i]["gate"], xv[i]["a"], y)
            state["t"] += 1
    elif w.path == "dense" and w.variant == "deltaproduct":
        S = S0

        def step():
            i = state["t"] % n_inputs
            rsu.deltaproduct_decode_step(S, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["gate"], xv[i]["beta"], y)
            state["t"] += 1
    elif w.path == "dense" and w.variant == "rwkv6":
        S = S0

        def step():
            i = state["t"] % n_inputs
            rsu.rwkv6_decode_step(S, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["gate"], y)
            state["t"] += 1
    elif w.path == "dense":
        fn = rsu.kda_decode_step if kda else rsu.gdn_decode_step
        S = S0

        def step():
            i = state["t"] % n_inputs
            fn(S, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["gate"], xv[i]["beta"], y)
            state["t"] += 1
    elif w.path == "stepq":
        Z = torch.empty(B, H, 128, 64, device=dev, dtype=torch.uint8)
        R = torch.empty(B, H, 128, device=dev, dtype=torch.float16)
        Cf = torch.empty(B, H, 128, device=dev, dtype=torch.float16)
        om = torch.from_numpy(wl.row_influence(w)).to(dev).view(B, H, 128)
        rsu.stepq_pack(S0, om, Z, R, Cf)
        del S0
        # `layers` independent packed states (a model's layers, the same inputs): a step runs
        # each of them once
        packs = [(Z, R, Cf)] + [(Z.clone(), R.clone(), Cf.clone()) for _ in range(layers - 1)]
        fn = rsu.kda_stepq_step if kda else rsu.gdn_stepq_step
        if split:
            # the readout on this stream, the repack on a second one ordered by events: a
            # layer's next readout waits for its repack, which can run beside the readouts of
            # the other layers (with one layer nothing else runs to hide the repack behind)
            readout = rsu.kda_stepq_readout if kda else rsu.gdn_stepq_readout
            repack = rsu.kda_stepq_repack if kda else rsu.gdn_stepq_repack
            us = [torch.empty(B, H, 128, device=dev) for _ in range(layers)]
            ys = [y] + [torch.empty(B, H, 128, device=dev) for _ in range(layers - 1)]
            u = us[0]
            side = torch.cuda.Stream()
            main = torch.cuda.current_stream()
            done = [None] * layers  # each layer's last repack

            def step():
                i = state["t"] % n_inputs
                for l, (Zl, Rl, Cl) in enumerate(packs):
                    if done[l] is not None:
                        main.wait_event(done[l])
                    readout(Zl, Rl, Cl, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["gate"], xv[i]["beta"], us[l], ys[l])
                    r1 = torch.cuda.Event()
                    r1.record(main)
                    with torch.cuda.stream(side):
                        side.wait_event(r1)
                        repack(Zl, Rl, Cl, om, xv[i]["k"], xv[i]["gate"], us[l])
                        done[l] = torch.cuda.Event()
                        done[l].record(side)
                state["t"] += 1

            def drain():
                for e in done:
                    if e is not None:
                        main.wait_event(e)

            def split_phases(reps=32):
                """Each half alone, launched back to back on one stream (the readout only reads the
                packed state; repeated repacks keep stepping it): average launch times."""
                out = {}
                for key, call in (("readout_us", lambda: readout(Z, R, Cf, x["q"][0], x["k"][0], x["v"][0],
                                                                   x["gate"][0], x["beta"][0], u, y)),
                                  ("repack_us", lambda: repack(Z, R, Cf, om, x["k"][0], x["gate"][0], u))):
                    call()
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(main)
                    for _ in range(reps):
                        call()
                    b.record(main)
                    torch.cuda.synchronize()
                    out[key] = round(a.elapsed_time(b) * 1e3 / reps, 2)
                return out
        else:
            def step():
                i = state["t"] % n_inputs
                for Zl, Rl, Cl in packs:
                    fn(Zl, Rl, Cl, om, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["gate"], xv[i]["beta"], y)
                state["t"] += 1
    elif w.path == "q8_window" and w.variant == "rwkv7":
        W = w.W
        Z = torch.empty(B, H, 128, 128, device=dev, dtype=torch.int8)
        A = torch.empty(B, H, 128, device=dev)
        rsu.q8_quantize(S0, Z, A)
        del S0
        Kb = torch.zeros(B, H, 2 * W, 128, device=dev, dtype=x["q"].dtype)
        Ub = torch.zeros(B, H, 2 * W, 128, device=dev)
        Gb = torch.zeros(B, H, 2 * W, 128, device=dev)

        def step():
            t = state["t"]
            i = t % n_inputs
            rsu.rwkv7_q8_window(W, t % W, Z, A, Kb, Ub, Gb, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["kappa"],
                                xv[i]["gate"], xv[i]["a"], y)
            state["t"] += 1
    elif w.path == "q8_window" and w.variant == "deltaproduct":
        W, R = w.W, w.n * w.W
        Z = torch.empty(B, H, 128, 128, device=dev, dtype=torch.int8)
        A = torch.empty(B, H, 128, device=dev)
        rsu.q8_quantize(S0, Z, A)
        del S0
        Kb = torch.zeros(B, H, R, 128, device=dev, dtype=x["q"].dtype)
        Ub = torch.zeros(B, H, R, 128, device=dev)
        Gb = torch.zeros(B, H, R, device=dev)

        def step():
            t = state["t"]
            i = t % n_inputs
            rsu.deltaproduct_q8_window(W, t % W, Z, A, Kb, Ub, Gb, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["gate"],
                                       xv[i]["beta"], y)
            state["t"] += 1
    elif w.path == "q8_window":
        W = w.W
        Z = torch.empty(B, H, 128, 128, device=dev, dtype=torch.int8)
        A = torch.empty(B, H, 128, device=dev)
        rsu.q8_quantize(S0, Z, A)
        del S0
        Kb = torch.zeros(B, H, W, 128, device=dev, dtype=x["q"].dtype)
        Ub = torch.zeros(B, H, W, 128, device=dev)
        Gb = torch.zeros((B, H, W, 128) if kda else (B, H, W), device=dev)
        fn = rsu.kda_q8_window if kda else rsu.gdn_q8_window

        def step():
            t = state["t"]
            i = t % n_inputs
            fn(W, t % W, Z, A, Kb, Ub, Gb, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["gate"], xv[i]["beta"], y)
            state["t"] += 1
    elif w.path == "lq_window":
        W = w.W
        four = w.bits == 4
        Z = (torch.empty(B, H, 128, 128 * w.bits // 8, device=dev, dtype=torch.uint8) if w.bits != 8 else
             torch.empty(B, H, 128, 128, device=dev, dtype=torch.int8))
        Bc = torch.empty(B, H, 128, device=dev)
        Cs = torch.empty(B, H, 128, device=dev)
        Kc = torch.empty(B, H, 8 if four else LQ_TOKENS, 128, device=dev, dtype=torch.float16)
        Uc = torch.empty_like(Kc)
        quant = ({4: rsu.kda_lq4_quantize, 6: rsu.kda_lq6_quantize, 8: rsu.kda_lq_quantize} if kda else
                 {4: rsu.gdn_lq4_quantize, 6: rsu.gdn_lq6_quantize, 8: rsu.gdn_lq_quantize})[w.bits]
        quant(S0, 8, Z, Bc, Cs, Kc, Uc)
        del S0
        Kb = torch.zeros(B, H, W, 128, device=dev, dtype=x["q"].dtype)
        Ub = torch.zeros(B, H, W, 128, device=dev)
        Gb = torch.zeros((B, H, W, 128) if kda else (B, H, W), device=dev)
        win = ({4: rsu.kda_lq4_window, 6: rsu.kda_lq6_window, 8: rsu.kda_lq_window} if kda else
               {4: rsu.gdn_lq4_window, 6: rsu.gdn_lq6_window, 8: rsu.gdn_lq_window})[w.bits]

        def step():
            t = state["t"]
            i = t % n_inputs
            win(W, t % W, n_iter, Z, Bc, Cs, Kc, Uc, Kb, Ub, Gb, xv[i]["q"], xv[i]["k"], xv[i]["v"],
                xv[i]["gate"], xv[i]["beta"], y)
            state["t"] += 1
    else:
        C = w.M - 1
        Sb = S0
        lbar = torch.zeros((B, H, 128) if kda else (B, H), device=dev)
        cap = max(C, 1)
        Kl = torch.zeros(B, H, cap, 128, device=dev, dtype=x["q"].dtype)
        rwkv6 = w.variant == "rwkv6"
        Ul = torch.zeros(B, H, cap, 128, device=dev, dtype=x["q"].dtype if rwkv6 else torch.float32)
        Lm = torch.zeros((B, H, cap, 128) if kda else (B, H, cap), device=dev)
        if rwkv6:
            # RWKV6's calls take no beta; wrap them to the delta-rule calls' argument list
            def _nb(f):
                return lambda C_, L_, Sb_, lb_, K_, U_, Lm_, q_, k_, v_, g_, b_, y_: \
                    f(C_, L_, Sb_, lb_, K_, U_, Lm_, q_, k_, v_, g_, y_)
        if slots:
            # every request-head at its own point of the cycle: 1/M of them merge per step
            Ld = torch.from_numpy(slot_lengths(w)).to(dev).view(B, H)
            fs = rsu.kda_log_step_slots if kda else rsu.gdn_log_step_slots
            if rwkv6:
                fs = _nb(rsu.rwkv6_log_step_slots)

            def step():
                i = state["t"] % n_inputs
                fs(C, Ld, Sb, lbar, Kl, Ul, Lm, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["gate"],
                   xv[i]["beta"], y)
                state["t"] += 1
        else:
            app = rsu.kda_log_append if kda else rsu.gdn_log_append
            mrg = rsu.kda_log_merge if kda else rsu.gdn_log_merge
            if rwkv6:
                app, mrg = _nb(rsu.rwkv6_log_append), _nb(rsu.rwkv6_log_merge)
            state["L"] = 0

            def step():
                i = state["t"] % n_inputs
                L = state["L"]
                f = app if L < C else mrg
                f(C, L, Sb, lbar, Kl, Ul, Lm, xv[i]["q"], xv[i]["k"], xv[i]["v"], xv[i]["gate"], xv[i]["beta"], y)
                state["L"] = L + 1 if L < C else 0
                state["t"] += 1

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    phases = None
    if w.path not in ("dense", "stepq"):
        # one untimed pass over whole cycles with an event between consecutive launches:
        # average launch time per window position / per live log length
        cyc = w.W if w.path in ("q8_window", "lq_window") else w.M
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4 * cyc + 1)]
        evs[0].record(stream)
        for e in evs[1:]:
            step()
            e.record(stream)
        torch.cuda.synchronize()
        per = [0.0] * cyc
        for i in range(4 * cyc):
            per[i % cyc] += evs[i].elapsed_time(evs[i + 1]) * 1e3 / 4
        key = "pos" if w.path in ("q8_window", "lq_window") else ("step" if slots else "L")
        phases = {f"{key}{i}_us": round(t, 2) for i, t in enumerate(per)}
    # one untimed pass with an event between consecutive launches: the distribution of step
    # times (whole cycles for the window and log paths, so that every position is included)
    cyc = {"q8_window": w.W, "lq_window": w.W, "log": w.M}.get(w.path, 1)
    n_dist = max(cyc, min(steps, 64) // cyc * cyc)
    evd = [torch.cuda.Event(enable_timing=True) for _ in range(n_dist + 1)]
    evd[0].record(stream)
    for e in evd[1:]:
        step()
        e.record(stream)
    torch.cuda.synchronize()
    per_step = np.array([evd[i].elapsed_time(evd[i + 1]) * 1e3 for i in range(n_dist)])
    dist = {"n": n_dist, "median_us": round(float(np.median(per_step)), 2),
            "p10_us": round(float(np.percentile(per_step, 10)), 2),
            "p90_us": round(float(np.percentile(per_step, 90)), 2)}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        # the K steps' launches captured once (capturing runs nothing; the host-side step
        # counters advance with the capture and match what the replay leaves on the device),
        # then replayed once inside the timed region: no host launch gaps between kernels
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del g
    else:
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            step()
        if drain is not None:
            drain()  # the timed region ends after the last launch on every stream
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    gpu_sec = e0.elapsed_time(e1) / 1e3
    if split:
        phases = split_phases()
    ceiling = None
    if w.path == "dense" and measure_ceiling:
        rb, wb = dense_rw_bytes_per_head(w)
        ceiling = hbm_ceiling(torch, rsu, w.heads, rb * w.heads, wb * w.heads, gpu_sec / steps)
    return gpu_sec, wall, ceiling, phases, dist


# ----------------------------------------------------------------- the other workloads

# The other workloads of the default line, with their timed and warm-up steps (whole windows
# and whole merge cycles): the dense KDA step, the int8 window and the base + log cycle.
OTHER_CONFIGS = ((3, 32, 4), (4, 64, 16), (5, 64, 16))


def run_other_configs() -> dict:
    """GPU-only measurements of the other workloads, each over whole windows / cycles, in the
    same process as the headline line (no CPU baseline): time per step, head-updates/s and
    algorithmic GB/s against the HBM peak."""
    out = {}
    for cid, steps, warmup in OTHER_CONFIGS:
        w = wl.WORKLOADS[cid]
        gpu_sec, _, _, _, dist = run_gpu(w, steps, warmup, measure_ceiling=False)
        per_head = cycle_bytes_per_head(w)
        launch = gpu_sec / steps
        gbs = per_head * w.heads / launch / 1e9
        out[w.name] = {"ms_per_step": launch * 1e3, "value": w.heads / launch, "unit": "head-updates/s",
                       "steps": steps, "warmup": warmup, "algorithmic_bytes_per_head_update": per_head,
                       "achieved_GBps": gbs, "frac": gbs / PEAK_HBM_GBS,
                       "median_step_us": dist["median_us"]}
    return out


# ----------------------------------------------------------------- CPU baseline (oracle)

def _cpu_model() -> str | None:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_cpu_baseline(w: wl.Workload, budget_s: float = 10.0, max_steps: int = 4096, slots: bool = False,
                     n_iter: int = 1):
    """The fp64 oracle (as it stands) of the workload's own path on the host cores: consecutive
    steps (cycling the workload's distinct step inputs) until the time budget is spent, on all
    heads for the dense steps and on the first 512 heads where the oracle loops over heads in
    Python (LeapQuant's refit, the packed state) or keeps per-window records. Only the oracle
    calls are timed."""
    import oracle
    oracle.build(force=False)
    n = w.heads if w.path == "dense" else min(w.heads, 512)
    S = wl.initial_state(w)[:n].astype(np.float64)
    cache = {}

    def inputs(t):
        i = t % max(1, w.steps)
        if i not in cache:
            x = wl.step_inputs(w, i)
            cache[i] = {name: a[:n] for name, a in x.items()}
        return cache[i]

    step = None
    if w.path == "dense":
        if w.variant == "rwkv6":
            def step(x): oracle.rwkv6_step(S, x["q"], x["k"], x["v"], x["gate"])  # noqa: E704
        elif w.variant == "rwkv7":
            def step(x): oracle.rwkv7_step(S, x["q"], x["k"], x["v"], x["gate"], x["kappa"], x["a"])  # noqa: E704
        elif w.variant == "deltaproduct":
            def step(x): oracle.deltaproduct_step(S, x["q"], x["k"], x["v"], x["gate"], x["beta"])  # noqa: E704
        else:
            def step(x): oracle.dense_step(S, x["q"], x["k"], x["v"], x["gate"], x["beta"])  # noqa: E704
    elif w.path == "q8_window":
        Z, a = oracle.q8_quantize(S)
        if w.variant == "rwkv7":
            ws = oracle.Rwkv7WindowState(Z, a, w.W)

            def step(x): ws.step(x["q"], x["k"], x["v"], x["gate"], x["kappa"], x["a"])  # noqa: E704
        elif w.variant == "deltaproduct":
            ws = oracle.DeltaProductWindowState(Z, a, w.W, w.n)

            def step(x): ws.step(x["q"], x["k"], x["v"], x["gate"], x["beta"])  # noqa: E704
        else:
            ws = oracle.WindowState(Z, a, w.W, w.per_key_gate)

            def step(x): ws.step(x["q"], x["k"], x["v"], x["gate"], x["beta"])  # noqa: E704
    elif w.path == "log":
        ls = oracle.LogState(S, w.M - 1, w.per_key_gate, rwkv6=w.variant == "rwkv6")
        Ls = slot_lengths(w)[:n].copy() if slots else None

        def step(x):
            if slots:
                ls.step_slots(Ls, x["q"], x["k"], x["v"], x["gate"], x.get("beta"))
            else:
                ls.step(x["q"], x["k"], x["v"], x["gate"], x.get("beta"))
    elif w.path == "lq_window":
        from oracle import lq
        qmax = lq.qmax_of(w.bits)
        r = 8 if w.bits == 4 else LQ_TOKENS
        reps = [lq.boundary(S[i], lq.walsh_start(r=r), 8, qmax) for i in range(n)]
        st = {"pos": 0, "S": None}

        def step(x):
            if st["pos"] == 0:
                st["S"] = np.stack([lq.represent(p["Z"], p["B"], p["c"], p["K16"], p["U16"], qmax) for p in reps])
            oracle.dense_step(st["S"], x["q"], x["k"], x["v"], x["gate"], x["beta"])
            st["pos"] += 1
            if st["pos"] == w.W:
                for i in range(n):
                    reps[i] = lq.boundary(st["S"][i], reps[i]["U"], n_iter, qmax)
                st["pos"] = 0
    elif w.path == "stepq":
        from oracle import stepq
        om = wl.row_influence(w)[:n].astype(np.float64)
        wts = stepq.row_weights(om)
        packs = [stepq.pack(S[i], wts[i]) for i in range(n)]
        st = {"z": np.stack([p["z"] for p in packs]), "r": np.stack([p["r"] for p in packs]),
              "c": np.stack([p["c"] for p in packs])}

        def step(x):
            _, new, _ = stepq.step(st["z"], st["r"], st["c"], om, x["q"], x["k"], x["v"], x["gate"], x["beta"])
            st["z"] = np.stack([p["z"] for p in new])
            st["r"] = np.stack([p["r"] for p in new])
            st["c"] = np.stack([p["c"] for p in new])
    n_steps, t_total = 0, 0.0
    while n_steps < max_steps and t_total < budget_s:
        x = inputs(n_steps)
        t0 = time.perf_counter()
        step(x)
        t_total += time.perf_counter() - t0
        n_steps += 1
    sample = f"{'all' if n == w.heads else 'the first'} {n} of {w.heads} heads x {n_steps} consecutive steps " \
             f"of the same workload (fp64 oracle of this path, {t_total:.1f} s of compute)"
    return {"value": n * n_steps / t_total, "unit": "head-updates/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": _cpu_model(),
            "host_cpus": os.cpu_count(), "sample": sample}


def override_workload(w: wl.Workload, args) -> wl.Workload:
    """Apply the command-line overrides; the workload's name records them."""
    ch = {}
    if args.variant and args.variant != w.variant:
        if w.path not in ("dense", "log", "stepq") and args.variant != "kda":
            raise SystemExit(f"--variant {args.variant} does not apply to the {w.path} workload")
        per_key = args.variant in ("kda", "rwkv6")
        ch.update(variant=args.variant, gate_lo=0.8 if per_key else 0.9, gate_hi=1.0 if per_key else 0.999)
    if args.B:
        ch["B"] = args.B
    if args.H:
        ch["H"] = args.H
    if args.M is not None:
        if w.path != "log" or not 1 <= args.M <= 64:
            raise SystemExit("--M applies to the log workload, 1 <= M <= 64")
        ch["M"] = args.M
    if args.slots and w.path != "log":
        raise SystemExit("--slots applies to the log workload")
    if not ch and not args.slots:
        return w
    w2 = wl.custom(w, **ch)
    var = w2.variant
    tail = {"dense": "", "stepq": "", "q8_window": f"_w{w2.W}", "lq_window": f"_w{w2.W}",
            "log": f"_m{w2.M}"}[w2.path]
    path = w2.path
    name = f"{var}_{path}_b{w2.B}_h{w2.H}{tail}" + ("_slots" if args.slots else "")
    return wl.custom(w2, name=name)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: 256 for gdn)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", choices=sorted(WORKLOAD_BY_FLAG), default="gdn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed steps as one captured HIP graph instead of launching them one by one "
                         "(measured: no faster, and 3-6%% slower for the window workloads)")
    ap.add_argument("--variant", choices=["gdn", "kda", "rwkv6"], default=None,
                    help="override the update kind of the workload (dense and log paths; kda also int8)")
    ap.add_argument("--B", type=int, default=None, help="override the batch size")
    ap.add_argument("--H", type=int, default=None, help="override the heads per request")
    ap.add_argument("--M", type=int, default=None, help="log path: merge interval (1..64)")
    ap.add_argument("--n-iter", type=int, default=1,
                    help="lq path: subspace iterations per boundary refit (warm-started)")
    ap.add_argument("--split", action="store_true",
                    help="stepq path: the readout and the repack as two launches on two streams")
    ap.add_argument("--layers", type=int, default=1,
                    help="stepq path: independent packed states stepped in turn (a model's layers); with "
                         "--split a layer's repack can run beside the next layer's readout")
    ap.add_argument("--slots", action="store_true",
                    help="log path: per-slot live lengths, every head at its own cycle point")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="default workload: skip the GPU-only lines of the KDA, int8-window and base+log workloads")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    w = wl.WORKLOADS[WORKLOAD_BY_FLAG[args.workload]]
    w = override_workload(w, args)
    cycle = {"dense": 1, "stepq": 1, "q8_window": w.W, "lq_window": w.W, "log": w.M}[w.path]
    steps = args.steps if args.steps is not None else 256
    steps = max(cycle, (steps + cycle - 1) // cycle * cycle)   # whole windows / cycles
    warmup = args.warmup if args.warmup is not None else 2 * cycle
    warmup = (warmup + cycle - 1) // cycle * cycle

    if args.split and (w.path != "stepq" or args.graph):
        raise SystemExit("--split applies to the stepq workload, without --graph")
    if args.layers < 1 or (args.layers > 1 and (w.path != "stepq" or args.graph)):
        raise SystemExit("--layers N > 1 applies to the stepq workload, without --graph")
    gpu_sec, wall, ceiling, phases, dist = run_gpu(w, steps, warmup, args.slots, args.n_iter, args.graph, args.split,
                                                   layers=args.layers)
    heads = w.heads * args.layers   # head-updates of one step (every layer once)
    per_head = slots_bytes_per_head(w) if args.slots else cycle_bytes_per_head(w)
    launch_sec = gpu_sec / steps
    achieved = per_head * heads / launch_sec / 1e9
    traffic = counter_traffic(per_head * heads) if w is wl.WORKLOADS[2] else None
    others = None
    if w is wl.WORKLOADS[2] and not args.no_other_configs and not args.graph:
        others = run_other_configs()

    out = {
        "metric": METRIC,
        "value": heads * steps / gpu_sec,
        "unit": "head-updates/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": launch_sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "dk": 128, "dv": 128,
                   "qkv": w.qkv, "state": ("int4+fp16 row and column factors" if w.path == "stepq" else
                                           "int4+f32 scales+8 fp16 token pairs" if w.bits == 4 else
                                           "int6+f32 scales+4 fp16 token pairs" if w.bits == 6 else
                                            {"q8_window": "int8+f32 scales",
                                             "lq_window": "int8+f32 scales+4 fp16 token pairs"}.get(w.path, "f32")),
                   "W": w.W or None, "M": w.M or None, "gates": w.variant,
                   "log_phases": ("per-slot (mixed)" if args.slots else "batch-uniform") if w.path == "log" else None,
                   "refit_iterations": args.n_iter if w.path == "lq_window" else None,
                   "layers": args.layers if w.path == "stepq" else None},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "traffic_source": (f"{os.path.relpath(PROFILE_COUNTERS, ROOT)}: rocprofv3 FETCH_SIZE and "
                                        "WRITE_SIZE of this kernel source (hash-checked), scaled by the stream "
                                        "probes; not measured in this run" if traffic is not None else None),
                     "algorithmic_bytes_per_launch": per_head * heads},
        "hbm_ceiling": ceiling,
        "wall_s_timed_region": wall,
        "timing": ("the K steps captured as one HIP graph, replayed once" if args.graph else
                   "eager launches, readout and repack on two streams" if args.split else "eager launches")
                  + (f"; {args.layers} layers per step" if args.layers > 1 else ""),
    }
    out["step_time_distribution"] = dist
    if phases:
        out["phases"] = phases
    if others:
        out["other_configs"] = others
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = run_cpu_baseline(w, slots=args.slots, n_iter=args.n_iter)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
