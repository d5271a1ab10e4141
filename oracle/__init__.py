"""fp64 CPU oracle of the delta-rule decode step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library
and never imports it. The arithmetic lives in ``rsu_oracle.c`` (plain C,
fp64, built with gcc without fast-math); this module only marshals numpy
arrays into it and keeps the per-head state of the three representations.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against properties fixed by the pages and by the mathematics (identities,
special cases, closed forms, bounds); see the header of that file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rsu_oracle.c")
_LIB = os.path.join(_HERE, "librsu_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, -O2, OpenMP over heads, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64, I = ctypes.c_int64, ctypes.c_int
        lib.oracle_dense_step.argtypes = [I64, I, I, I, P, P, P, P, P, P, P]
        lib.oracle_q8_quantize.argtypes = [I64, I, P, P, P, P]
        lib.oracle_q8_window_step.argtypes = [I64, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P,
                                              P, P, P]
        lib.oracle_log_step.argtypes = [I64, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_log_step_slots.argtypes = [I64, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_rwkv6_step.argtypes = [I64, I, I, P, P, P, P, P, P]
        lib.oracle_rwkv7_step.argtypes = [I64, I, I, P, P, P, P, P, P, P, P]
        lib.oracle_rwkv7_q8_window_step.argtypes = [I64, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                                    P]
        lib.oracle_deltaproduct_step.argtypes = [I64, I, I, I, P, P, P, P, P, P, P]
        lib.oracle_deltaproduct_q8_window_step.argtypes = [I64, I, I, I, I, I, P, P, P, P, P, P, P, P,
                                                           P, P, P, P, P]
        lib.oracle_rwkv6_log_step.argtypes = [I64, I, I, I, I, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_rwkv6_log_step_slots.argtypes = [I64, I, I, I, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        for f in (lib.oracle_dense_step, lib.oracle_q8_quantize, lib.oracle_q8_window_step,
                  lib.oracle_log_step, lib.oracle_log_step_slots, lib.oracle_rwkv6_step,
                  lib.oracle_rwkv6_log_step, lib.oracle_rwkv6_log_step_slots, lib.oracle_rwkv7_step,
                  lib.oracle_rwkv7_q8_window_step, lib.oracle_deltaproduct_step,
                  lib.oracle_deltaproduct_q8_window_step):
            f.restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle uses (one head per thread at a time)."""
    return _load().oracle_num_threads()


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_step_inputs(nh, dk, dv, per_key, q, k, v, gate, beta):
    assert q.shape == (nh, dk) and k.shape == (nh, dk) and v.shape == (nh, dv)
    assert gate.shape == ((nh, dk) if per_key else (nh,))
    assert beta.shape == (nh,)


def dense_step(S: np.ndarray, q, k, v, gate, beta) -> np.ndarray:
    """One eager decode step on fp64 states S[nh, dk, dv] (updated in place).
    Returns y[nh, dv]. gate is alpha [nh] (GDN) or d [nh, dk] (KDA)."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    nh, dk, dv = S.shape
    q, k, v, gate, beta = map(_f64, (q, k, v, gate, beta))
    per_key = int(gate.ndim == 2)
    _check_step_inputs(nh, dk, dv, per_key, q, k, v, gate, beta)
    y = np.empty((nh, dv))
    _load().oracle_dense_step(nh, dk, dv, per_key, _ptr(S), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(gate), _ptr(beta), _ptr(y))
    return y


def rwkv6_step(S: np.ndarray, q, k, v, w) -> np.ndarray:
    """One RWKV6 decode step in the pages' common form, S <- Diag(w) S + k v^T and
    y = S^T q, on fp64 states S[nh, dk, dv] (updated in place); w is [nh, dk]."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    nh, dk, dv = S.shape
    q, k, v, w = map(_f64, (q, k, v, w))
    assert q.shape == (nh, dk) and k.shape == (nh, dk) and v.shape == (nh, dv) and w.shape == (nh, dk)
    y = np.empty((nh, dv))
    _load().oracle_rwkv6_step(nh, dk, dv, _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(y))
    return y


def rwkv7_step(S: np.ndarray, q, k, v, w, kappa, a) -> np.ndarray:
    """One RWKV7 decode step as its two sub-steps (erase along kappa read with a * kappa,
    then write k v^T), y = S^T q, on fp64 states S[nh, dk, dv] (updated in place)."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    nh, dk, dv = S.shape
    q, k, v, w, kappa, a = map(_f64, (q, k, v, w, kappa, a))
    for x, n in ((q, dk), (k, dk), (v, dv), (w, dk), (kappa, dk), (a, dk)):
        assert x.shape == (nh, n)
    y = np.empty((nh, dv))
    _load().oracle_rwkv7_step(nh, dk, dv, _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(kappa), _ptr(a),
                              _ptr(y))
    return y


def _check_dp_inputs(nh, dk, dv, q, k, v, alpha, beta):
    n = k.shape[1] if k.ndim == 3 else 0
    assert n >= 1 and q.shape == (nh, dk) and k.shape == (nh, n, dk) and v.shape == (nh, n, dv)
    assert alpha.shape == (nh,) and beta.shape == (nh, n)
    return n


def deltaproduct_step(S: np.ndarray, q, k, v, alpha, beta) -> np.ndarray:
    """One DeltaProduct token (n delta-rule sub-steps, the scalar gate in the first) on fp64
    states S[nh, dk, dv] (updated in place): k [nh, n, dk], v [nh, n, dv], alpha [nh],
    beta [nh, n]. Returns y[nh, dv] read after the last sub-step."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    nh, dk, dv = S.shape
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    n = _check_dp_inputs(nh, dk, dv, q, k, v, alpha, beta)
    y = np.empty((nh, dv))
    _load().oracle_deltaproduct_step(nh, dk, dv, n, _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                     _ptr(beta), _ptr(y))
    return y


def q8_quantize(X: np.ndarray, with_w: bool = False):
    """Per-row symmetric int8 quantization of X[..., ncols] (fp32 decision).
    Returns (Z int8, a fp32[...]) and, if asked, the exact pre-rounding codes."""
    X = _f64(X)
    shape = X.shape
    nrows, ncols = int(np.prod(shape[:-1])), shape[-1]
    Z = np.empty(shape, dtype=np.int8)
    a = np.empty(shape[:-1], dtype=np.float32)
    w = np.empty(shape) if with_w else None
    _load().oracle_q8_quantize(nrows, ncols, _ptr(X), _ptr(Z), _ptr(a),
                               _ptr(w) if with_w else None)
    return (Z, a, w) if with_w else (Z, a)


def dequant(Z: np.ndarray, a: np.ndarray) -> np.ndarray:
    """z * a / 127 per row, in fp64 (LeapQuant App. B.3 with per-row scales)."""
    return Z.astype(np.float64) * (a.astype(np.float64)[..., None] / 127.0)


class WindowState:
    """The int8 window representation of nh heads: window-start codes Z and row
    scales a, plus the window's records (LeapQuant sec. 3.2)."""

    def __init__(self, Z: np.ndarray, a: np.ndarray, W: int, per_key: bool):
        nh, dk, dv = Z.shape
        self.Z = np.ascontiguousarray(Z, dtype=np.int8).copy()
        self.a = np.ascontiguousarray(a, dtype=np.float32).copy()
        self.W, self.per_key = W, per_key
        self.G = np.zeros((nh, W, dk) if per_key else (nh, W))
        self.K = np.zeros((nh, W, dk))
        self.U = np.zeros((nh, W, dv))
        self.pos = 0

    def step(self, q, k, v, gate, beta, want_boundary: bool = False):
        """Run step self.pos; returns y (and (S_W, w) at a boundary if asked)."""
        nh, dk, dv = self.Z.shape
        q, k, v, gate, beta = map(_f64, (q, k, v, gate, beta))
        _check_step_inputs(nh, dk, dv, self.per_key, q, k, v, gate, beta)
        y = np.empty((nh, dv))
        boundary = self.pos == self.W - 1
        Sw = np.empty((nh, dk, dv)) if (boundary and want_boundary) else None
        w = np.empty((nh, dk, dv)) if (boundary and want_boundary) else None
        _load().oracle_q8_window_step(
            nh, dk, dv, int(self.per_key), self.W, self.pos, _ptr(self.Z), _ptr(self.a),
            _ptr(self.G), _ptr(self.K), _ptr(self.U), _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
            _ptr(beta), _ptr(y), _ptr(Sw) if Sw is not None else None,
            _ptr(w) if w is not None else None)
        self.pos = 0 if boundary else self.pos + 1
        if boundary:
            self.G[:] = 0.0
            self.K[:] = 0.0
            self.U[:] = 0.0
        if want_boundary:
            return y, Sw, w
        return y


class Rwkv7WindowState:
    """RWKV7 on the int8 window representation: window-start (Z, a) plus two records per
    token (erase along kappa, then write k v^T; LeapQuant App. A), 2W records per window."""

    def __init__(self, Z: np.ndarray, a: np.ndarray, W: int):
        nh, dk, dv = Z.shape
        self.Z = np.ascontiguousarray(Z, dtype=np.int8).copy()
        self.a = np.ascontiguousarray(a, dtype=np.float32).copy()
        self.W = W
        self.G = np.zeros((nh, 2 * W, dk))
        self.K = np.zeros((nh, 2 * W, dk))
        self.U = np.zeros((nh, 2 * W, dv))
        self.pos = 0

    def step(self, q, k, v, w, kappa, erase, want_boundary: bool = False):
        nh, dk, dv = self.Z.shape
        q, k, v, w, kappa, erase = map(_f64, (q, k, v, w, kappa, erase))
        for x, n in ((q, dk), (k, dk), (v, dv), (w, dk), (kappa, dk), (erase, dk)):
            assert x.shape == (nh, n)
        y = np.empty((nh, dv))
        boundary = self.pos == self.W - 1
        Sw = np.empty((nh, dk, dv)) if (boundary and want_boundary) else None
        wq = np.empty((nh, dk, dv)) if (boundary and want_boundary) else None
        _load().oracle_rwkv7_q8_window_step(
            nh, dk, dv, self.W, self.pos, _ptr(self.Z), _ptr(self.a), _ptr(self.G), _ptr(self.K),
            _ptr(self.U), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(kappa), _ptr(erase), _ptr(y),
            _ptr(Sw) if Sw is not None else None, _ptr(wq) if wq is not None else None)
        self.pos = 0 if boundary else self.pos + 1
        if boundary:
            self.G[:] = 0
            self.K[:] = 0
            self.U[:] = 0
        return (y, Sw, wq) if (boundary and want_boundary) else y


class DeltaProductWindowState:
    """DeltaProduct on the int8 window representation: window-start (Z, a) plus n records per
    token (one per delta-rule sub-step; LeapQuant App. A), nW records per window."""

    def __init__(self, Z: np.ndarray, a: np.ndarray, W: int, n: int):
        nh, dk, dv = Z.shape
        self.Z = np.ascontiguousarray(Z, dtype=np.int8).copy()
        self.a = np.ascontiguousarray(a, dtype=np.float32).copy()
        self.W, self.n = W, n
        self.G = np.zeros((nh, n * W))
        self.K = np.zeros((nh, n * W, dk))
        self.U = np.zeros((nh, n * W, dv))
        self.pos = 0

    def step(self, q, k, v, alpha, beta, want_boundary: bool = False):
        nh, dk, dv = self.Z.shape
        q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
        assert _check_dp_inputs(nh, dk, dv, q, k, v, alpha, beta) == self.n
        y = np.empty((nh, dv))
        boundary = self.pos == self.W - 1
        Sw = np.empty((nh, dk, dv)) if (boundary and want_boundary) else None
        wq = np.empty((nh, dk, dv)) if (boundary and want_boundary) else None
        _load().oracle_deltaproduct_q8_window_step(
            nh, dk, dv, self.n, self.W, self.pos, _ptr(self.Z), _ptr(self.a), _ptr(self.G), _ptr(self.K),
            _ptr(self.U), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(y),
            _ptr(Sw) if Sw is not None else None, _ptr(wq) if wq is not None else None)
        self.pos = 0 if boundary else self.pos + 1
        if boundary:
            self.G[:] = 0
            self.K[:] = 0
            self.U[:] = 0
        return (y, Sw, wq) if (boundary and want_boundary) else y


class LogState:
    """The base + log representation of nh heads (DeltaLog sec. 3.1): dense base
    Sbar, cumulative log-decay lbar, and a log of capacity C = M - 1. ``rwkv6``
    selects the update without the delta read (per-key decay, pair (k, v))."""

    def __init__(self, Sbar: np.ndarray, C: int, per_key: bool, rwkv6: bool = False):
        nh, dk, dv = Sbar.shape
        self.Sbar = _f64(Sbar).copy()
        self.C, self.per_key, self.rwkv6 = C, per_key or rwkv6, rwkv6
        per_key = self.per_key
        gd = (dk,) if per_key else ()
        self.lbar = np.zeros((nh,) + gd)
        cap = max(C, 1)
        self.K = np.zeros((nh, cap, dk))
        self.U = np.zeros((nh, cap, dv))
        self.Lam = np.zeros((nh, cap) + gd)
        self.L = 0

    def step(self, q, k, v, gate, beta=None):
        nh, dk, dv = self.Sbar.shape
        if self.rwkv6:
            q, k, v, w = map(_f64, (q, k, v, gate))
            assert w.shape == (nh, dk)
            y = np.empty((nh, dv))
            _load().oracle_rwkv6_log_step(nh, dk, dv, self.C, self.L, _ptr(self.Sbar), _ptr(self.lbar),
                                          _ptr(self.K), _ptr(self.U), _ptr(self.Lam), _ptr(q), _ptr(k),
                                          _ptr(v), _ptr(w), _ptr(y))
            self.L = self.L + 1 if self.L < self.C else 0
            return y
        q, k, v, gate, beta = map(_f64, (q, k, v, gate, beta))
        _check_step_inputs(nh, dk, dv, self.per_key, q, k, v, gate, beta)
        y = np.empty((nh, dv))
        _load().oracle_log_step(nh, dk, dv, int(self.per_key), self.C, self.L, _ptr(self.Sbar),
                                _ptr(self.lbar), _ptr(self.K), _ptr(self.U), _ptr(self.Lam),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(y))
        self.L = self.L + 1 if self.L < self.C else 0
        return y

    def step_slots(self, Ls, q, k, v, gate, beta=None):
        """One step with a live length per head (Ls: int array [nh], each in [0, C],
        advanced in place): heads with Ls < C append, heads with Ls == C merge."""
        nh, dk, dv = self.Sbar.shape
        if Ls.dtype != np.int32 or Ls.shape != (nh,) or not Ls.flags.c_contiguous:
            raise ValueError("Ls must be a contiguous int32 array of one live length per head")
        if (Ls < 0).any() or (Ls > self.C).any():
            raise ValueError("live lengths must lie in [0, C]")
        y = np.empty((nh, dv))
        if self.rwkv6:
            q, k, v, w = map(_f64, (q, k, v, gate))
            assert w.shape == (nh, dk)
            _load().oracle_rwkv6_log_step_slots(nh, dk, dv, self.C, Ls.ctypes.data_as(ctypes.c_void_p),
                                                _ptr(self.Sbar), _ptr(self.lbar), _ptr(self.K), _ptr(self.U),
                                                _ptr(self.Lam), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(y))
            return y
        q, k, v, gate, beta = map(_f64, (q, k, v, gate, beta))
        _check_step_inputs(nh, dk, dv, self.per_key, q, k, v, gate, beta)
        _load().oracle_log_step_slots(nh, dk, dv, int(self.per_key), self.C,
                                      Ls.ctypes.data_as(ctypes.c_void_p), _ptr(self.Sbar),
                                      _ptr(self.lbar), _ptr(self.K), _ptr(self.U), _ptr(self.Lam),
                                      _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(y))
        return y

    def logical_state(self) -> np.ndarray:
        """Eq. 7 of DeltaLog, evaluated with numpy (for inspection in tests)."""
        S = np.exp(self.lbar)[..., None] * self.Sbar if self.per_key else \
            np.exp(self.lbar)[:, None, None] * self.Sbar
        for m in range(self.L):
            dec = np.exp(self.lbar - self.Lam[:, m])
            Km = (dec * self.K[:, m]) if self.per_key else dec[:, None] * self.K[:, m]
            S = S + Km[:, :, None] * self.U[:, m][:, None, :]
        return S
