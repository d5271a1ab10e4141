"""Seeded synthetic inputs for the delta-rule decode step.

This module is shared by the HIP path's tests and benchmark and by the fp64
oracle's tests. It holds random draws, the L2-normalisation of q and k that the
workloads prescribe, and dtype casts of inputs -- and none of the recurrence's
arithmetic.

Workload shapes follow the decode-kernel experiments of the three pages:
128x128 states per head (LeapQuant, sec. 4.3 "Kernel speedup"; DeltaLog, Table 3),
32-48 heads per layer and batches of 4-512 requests, a window of 16 tokens
(LeapQuant, sec. 4.1 "Implementation") and a merge interval of 8 for GDN
(DeltaLog, Table 3).

Every tensor of every step has its own substream:
``numpy.random.SeedSequence([1000 + config_id, tensor_tag, step])`` feeding an
SFC64 generator (float32 normals and uniforms), so any step can be regenerated
on its own. The initial state is drawn in chunks of 256 heads, each with its
own substream ``[1000 + config_id, 0, chunk]``, on a few threads.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os

import numpy as np

DK = 128
DV = 128

# tensor tags of the substreams
(_TAG_S0, _TAG_Q, _TAG_K, _TAG_V, _TAG_GATE, _TAG_BETA, _TAG_OUTLIER, _TAG_KAPPA, _TAG_A, _TAG_OMEGA,
 _TAG_SUB_K, _TAG_SUB_V, _TAG_SUB_BETA) = range(13)


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    variant: str          # "gdn" (scalar gate alpha), "kda" (per-key gate d), "rwkv6" (per-key decay w,
                          # no delta read), "rwkv7" (per-key decay w, erase along kappa read with a * kappa)
                          # or "deltaproduct" (n delta-rule sub-steps per token, scalar gate alpha)
    path: str             # "dense", "q8_window", "lq_window", "log" or "stepq"
    B: int
    H: int
    steps: int
    qkv: str              # "f32" or "bf16"
    gate_lo: float
    gate_hi: float
    state_std: float = 0.02
    W: int = 0            # window length of the int8 path
    M: int = 0            # merge interval of the base+log path (capacity C = M - 1)
    outliers: bool = False
    bits: int = 8         # code width of the LeapQuant window format (8, 6, or 4 with 8 tokens)
    n: int = 1            # DeltaProduct: delta-rule sub-steps per token
    tiny_row: int = -1    # >= 0: that key row of every S_0 is scaled by a power of two to a maximum
                          # in (2^-123, 2^-122], where 127 / max overflows fp32, and every key (k,
                          # kappa, the sub-step keys) is zero there, so no record writes to the row

    @property
    def heads(self) -> int:
        return self.B * self.H

    @property
    def seed(self) -> int:
        return 1000 + self.cid

    @property
    def per_key_gate(self) -> bool:
        return self.variant in ("kda", "rwkv6", "rwkv7")


WORKLOADS = {
    1: Workload(1, "gdn_dense_b4_h8_f32", "gdn", "dense", 4, 8, 64, "f32", 0.90, 0.999),
    2: Workload(2, "gdn_dense_b256_h48_bf16", "gdn", "dense", 256, 48, 16, "bf16", 0.90, 0.999),
    3: Workload(3, "kda_dense_b128_h32_bf16", "kda", "dense", 128, 32, 32, "bf16", 0.80, 1.0),
    4: Workload(4, "gdn_q8_window_b256_h48_w16", "gdn", "q8_window", 256, 48, 256, "bf16",
                0.90, 0.999, W=16, outliers=True),
    5: Workload(5, "gdn_log_b256_h48_m8", "gdn", "log", 256, 48, 128, "bf16", 0.90, 0.999, M=8),
    # LeapQuant's boundary format on the int8 workload's own inputs (same seed as 4)
    6: Workload(4, "gdn_lq_window_b256_h48_w16", "gdn", "lq_window", 256, 48, 256, "bf16",
                0.90, 0.999, W=16, outliers=True),
    # RWKV6 at the shape of DeltaLog's kernel study (Table 3: 32 heads of 128 x 128, M = 4),
    # batch 128 as in its interval sweep; per-key decays drawn like KDA's gates
    # LeapQuant's format at 4 bits with 8 tokens on the int8 workload's inputs (same seed as 4)
    12: Workload(4, "gdn_lq4_window_b256_h48_w16", "gdn", "lq_window", 256, 48, 256, "bf16", 0.90, 0.999,
                 W=16, outliers=True, bits=4),
    # LeapQuant's format at 6 bits (4 tokens) on the int8 workload's inputs (same seed as 4)
    16: Workload(4, "gdn_lq6_window_b256_h48_w16", "gdn", "lq_window", 256, 48, 256, "bf16", 0.90, 0.999,
                 W=16, outliers=True, bits=6),
    # LeapQuant's format at 4 and 6 bits with KDA gates on the KDA workload's shape (same seed as 9)
    17: Workload(9, "kda_lq4_window_b128_h32_w16", "kda", "lq_window", 128, 32, 256, "bf16", 0.80, 1.0,
                 W=16, outliers=True, bits=4),
    18: Workload(9, "kda_lq6_window_b128_h32_w16", "kda", "lq_window", 128, 32, 256, "bf16", 0.80, 1.0,
                 W=16, outliers=True, bits=6),
    # LeapQuant's format with KDA gates on the KDA workload's shape (same outliers as 4)
    9: Workload(9, "kda_lq_window_b128_h32_w16", "kda", "lq_window", 128, 32, 256, "bf16", 0.80, 1.0,
                W=16, outliers=True),
    10: Workload(10, "rwkv7_dense_b128_h32_bf16", "rwkv7", "dense", 128, 32, 32, "bf16", 0.80, 1.0),
    # RWKV7 on the int8 window, two records per token (with the int8 workload's outliers)
    11: Workload(11, "rwkv7_q8_window_b128_h32_w16", "rwkv7", "q8_window", 128, 32, 256, "bf16", 0.80, 1.0,
                 W=16, outliers=True),
    7: Workload(7, "rwkv6_dense_b128_h32_bf16", "rwkv6", "dense", 128, 32, 32, "bf16", 0.80, 1.0),
    8: Workload(8, "rwkv6_log_b128_h32_m4", "rwkv6", "log", 128, 32, 128, "bf16", 0.80, 1.0, M=4),
    # STEPQuant-style per-step packed state (4-bit codes, fp16 row and column factors) at the
    # dense GDN workload's serving shape, with the int8 workload's row and column outliers
    13: Workload(13, "gdn_stepq_b256_h48_bf16", "gdn", "stepq", 256, 48, 16, "bf16", 0.90, 0.999,
                 outliers=True, bits=4),
    # DeltaProduct with two sub-steps per token (LeapQuant App. A, Table 4) at the dense GDN
    # workload's serving shape, and on the int8 window (one record per sub-step, 32 per window)
    14: Workload(14, "deltaproduct_dense_b256_h48_n2_bf16", "deltaproduct", "dense", 256, 48, 16, "bf16",
                 0.90, 0.999, n=2),
    15: Workload(15, "deltaproduct_q8_window_b256_h48_n2_w16", "deltaproduct", "q8_window", 256, 48, 256,
                 "bf16", 0.90, 0.999, W=16, outliers=True, n=2),
}


def custom(base: Workload, **changes) -> Workload:
    """A workload with some fields replaced (smaller batches for fast parity runs)."""
    return dataclasses.replace(base, **changes)


def _rng(wl: Workload, tag: int, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence([wl.seed, tag, step])))


_CHUNK = 256
_THREADS = max(1, min(16, os.cpu_count() or 1))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bfloat16 (ties to even), returned as fp32.

    Every returned value is exactly representable in bfloat16, so casting it to
    bfloat16 on the device is exact and widening it to fp64 for the oracle is exact.
    """
    bits = np.array(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> 16) & np.uint32(1)
    bits += np.uint32(0x7FFF)
    bits += lsb
    bits &= np.uint32(0xFFFF0000)
    return bits.view(np.float32)


def _cast(wl: Workload, x64: np.ndarray) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return round_to_bf16(x32) if wl.qkv == "bf16" else x32


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def initial_state(wl: Workload) -> np.ndarray:
    """S_0 of every head: fp32 [B*H, 128, 128], entries N(0, std^2).

    For the int8 workload, 2 distinct key rows and 2 distinct value columns of
    every head are multiplied by 50 (union of the row and column masks, so the
    4 crossings are x50 too). Large rows and columns in real states are
    described by LeapQuant (sec. 1; Figure 6) and by the STEPQuant notes
    (row/column max-to-median ratios).
    """
    n = wl.heads
    S = np.empty((n, DK, DV), dtype=np.float32)
    std = np.float32(wl.state_std)

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        r = _rng(wl, _TAG_S0, c)
        r.standard_normal((hi - lo, DK, DV), dtype=np.float32, out=S[lo:hi])
        S[lo:hi] *= std
        if wl.outliers:
            ro = _rng(wl, _TAG_OUTLIER, c)
            rows = np.argsort(ro.random((hi - lo, DK)), axis=1)[:, :2]
            cols = np.argsort(ro.random((hi - lo, DV)), axis=1)[:, :2]
            rm = np.zeros((hi - lo, DK), dtype=bool)
            cm = np.zeros((hi - lo, DV), dtype=bool)
            np.put_along_axis(rm, rows, True, axis=1)
            np.put_along_axis(cm, cols, True, axis=1)
            blk = S[lo:hi]
            blk[rm[:, :, None] | cm[:, None, :]] *= np.float32(50.0)

    nchunks = (n + _CHUNK - 1) // _CHUNK
    with concurrent.futures.ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, range(nchunks)))
    if wl.tiny_row >= 0:
        row = S[:, wl.tiny_row, :]
        e = np.ceil(np.log2(np.abs(row).max(axis=1).astype(np.float64))).astype(np.int32)
        S[:, wl.tiny_row, :] = np.ldexp(row, (-122 - e)[:, None])
    return S


def _keys(wl: Workload, x: np.ndarray) -> np.ndarray:
    """Unit keys over d_k (fp64 normalisation, then the input dtype), zero at tiny_row."""
    x = x.astype(np.float64)
    if wl.tiny_row >= 0:
        x[..., wl.tiny_row] = 0.0
    return _cast(wl, _unit_rows(x))


def step_inputs(wl: Workload, t: int) -> dict:
    """Inputs of decode step t (0-based) for all heads.

    q, k: N(0,1) then L2-normalised over d_k in fp64, then cast to the
    workload's input dtype (fp32 values, bf16-representable when qkv == bf16).
    v: N(0,1) in the input dtype. gate: alpha ~ U(lo, hi) per head [B*H] for
    GDN, d ~ U(lo, hi) per key channel [B*H, 128] for KDA. beta ~ U(0, 1) [B*H].
    RWKV7 also draws its removal key kappa (N(0,1), L2-normalised, input dtype) and its
    per-key erase rate a ~ U(0, 1) [B*H, 128]. DeltaProduct draws a key, a value and a
    strength per sub-step the same way (k [B*H, n, 128], v [B*H, n, 128], beta [B*H, n]).
    All arrays are fp32.
    """
    n = wl.heads
    f32 = np.float32
    q = _cast(wl, _unit_rows(_rng(wl, _TAG_Q, t).standard_normal((n, DK), dtype=f32).astype(np.float64)))
    k = _keys(wl, _rng(wl, _TAG_K, t).standard_normal((n, DK), dtype=f32))
    v = _cast(wl, _rng(wl, _TAG_V, t).standard_normal((n, DV), dtype=f32))
    gshape = (n, DK) if wl.per_key_gate else (n,)
    lo, hi = wl.gate_lo, wl.gate_hi
    gate = (lo + (hi - lo) * _rng(wl, _TAG_GATE, t).random(gshape)).astype(f32)
    gate = np.clip(gate, f32(lo), f32(hi))
    beta = _rng(wl, _TAG_BETA, t).random((n,), dtype=f32)
    out = {"q": q, "k": k, "v": v, "gate": gate, "beta": beta}
    if wl.variant == "rwkv7":
        out["kappa"] = _keys(wl, _rng(wl, _TAG_KAPPA, t).standard_normal((n, DK), dtype=f32))
        out["a"] = _rng(wl, _TAG_A, t).random((n, DK), dtype=f32)
    if wl.variant == "deltaproduct":
        # sub-step 0 takes the draws above; sub-steps 1 .. n-1 draw their own key, value and
        # strength the same way: k [heads, n, d_k], v [heads, n, d_v], beta [heads, n]
        ks, vs, bs = [k], [v], [beta]
        for i in range(1, wl.n):
            ks.append(_keys(wl, _rng(wl, _TAG_SUB_K, wl.n * t + i).standard_normal((n, DK), dtype=f32)))
            vs.append(_cast(wl, _rng(wl, _TAG_SUB_V, wl.n * t + i).standard_normal((n, DV), dtype=f32)))
            bs.append(_rng(wl, _TAG_SUB_BETA, wl.n * t + i).random((n,), dtype=f32))
        out["k"] = np.ascontiguousarray(np.stack(ks, axis=1))
        out["v"] = np.ascontiguousarray(np.stack(vs, axis=1))
        out["beta"] = np.ascontiguousarray(np.stack(bs, axis=1))
    return out


def row_influence(wl: Workload) -> np.ndarray:
    """Row influence scores omega [B*H, 128] fp32 of the packed-state workload: log-normal,
    exp(1.08 N(0, 1)), whose 90th/10th percentile ratio, exp(2 * 1.2816 * 1.08) = 15.9, is the
    per-head median ratio the STEPQuant notes report (15.95). They stand in for calibration."""
    n = wl.heads
    z = _rng(wl, _TAG_OMEGA, 0).standard_normal((n, DK), dtype=np.float32).astype(np.float64)
    return np.exp(1.08 * z).astype(np.float32)


def sample_heads(wl: Workload, count: int, seed: int = 7) -> np.ndarray:
    """Sorted distinct head indices for sampled full-size comparisons (always
    includes the first and the last head)."""
    n = wl.heads
    if count >= n:
        return np.arange(n)
    r = np.random.default_rng(seed)
    pick = set(r.choice(n, size=count - 2, replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(pick))
