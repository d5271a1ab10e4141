"""fp64 oracle of STEPQuant's per-step packed state -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this module. It shares no code with the HIP library. Plain numpy in fp64; the
decode-step update itself is the (separately pinned) dense oracle step.

The format (STEPQuant notes, the section on the key-row-aware dual-axis fit): element
(i, j) of a head's state X -- key row i, value column j -- is stored as r_i c_j z_ij, a
per-key-row factor r_i and a per-value-column factor c_j (both fp16) and a low-bit integer
code z_ij. It is refitted after every decode step from the new state X_t: the page's fused
kernel decodes the packed state, applies the delta update, reads y_t = X_t^T q_t out, and
packs X_t again.

Readings taken where the notes are silent or their text is lost (stated once here):
  * row influence weights: the notes compress omega with the exponent gamma = 0.25 and say
    that this makes w_i proportional to omega_i^(1/8); read as the power gamma of the RMS read
    weight sqrt(omega_i): w_i = omega_i^(gamma / 2), divided by their geometric mean over the
    head's 128 rows; omega (the calibrated row influence scores) is an input;
  * row factor: r_i = sqrt(m_i / w_i) with m_i = mean_j |X_ij| (the notes' formula did not
    survive extraction; they describe it as SmoothQuant's fractional-power balance of the
    row's magnitude against its influence, read here as SmoothQuant's square root), rounded
    to fp16; a row with m_i = 0 gets r_i = 0 and zero codes. Parity unpinned: the pins fix
    what follows from any row factor, not this exponent;
  * codes of one uniform width (qmax = 7, i.e. 4 bits: the calibrated per-unit width tables
    and the fp16 pivot rows come from data and are not built): with the column range
    a_j = max_i |X_ij| / r_i over the rows with r_i > 0, z_ij = clamp(rne(X_ij / r_i * qmax /
    a_j), -qmax, qmax); a column with a_j = 0 gets zero codes;
  * column factor: for these codes, c_j minimizes sum_i w_i^2 (X_ij - r_i c_j z_ij)^2, the
    closed-form weighted least squares c_j = sum_i w_i^2 r_i z_ij X_ij / sum_i w_i^2 r_i^2 z_ij^2
    (0 when the column has no nonzero code), rounded to fp16.
Decisions are taken on the exact fp64 values; ``pack`` also returns the pre-rounding values
so that parity checks can tell rounding ties apart.
"""
from __future__ import annotations

import numpy as np

GAMMA = 0.25
QMAX4 = 7


def to_fp16(x) -> np.ndarray:
    """Round to the nearest fp16 (ties to even), returned widened to fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def row_weights(omega: np.ndarray) -> np.ndarray:
    """w_i = sqrt(omega_i)^gamma = omega_i^(1/8) over its geometric mean along the last axis
    (the head's rows)."""
    p = np.sqrt(np.asarray(omega, dtype=np.float64)) ** GAMMA
    return p / np.exp(np.mean(np.log(p), axis=-1, keepdims=True))


def column_factors(X: np.ndarray, r: np.ndarray, z: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Weighted least squares per value column, codes fixed: argmin_c sum_i w_i^2 (X_ij -
    r_i c z_ij)^2 = sum_i w_i^2 r_i z_ij X_ij / sum_i w_i^2 r_i^2 z_ij^2 (0 for no nonzero code)."""
    wr = (w ** 2 * r)[:, None]
    num = np.sum(wr * z * X, axis=0)
    den = np.sum(wr * r[:, None] * z * z, axis=0)
    c = np.zeros(X.shape[1])
    nz = den > 0
    c[nz] = num[nz] / den[nz]
    return c


def pack(X: np.ndarray, w: np.ndarray, qmax: int = QMAX4) -> dict:
    """One head's state X [128, 128] in the dual-axis format. Returns z (int8 up to qmax = 127), r and c
    (fp16 values widened to fp64), and the pre-rounding values r_pre, code_pre, c_pre."""
    X = np.asarray(X, dtype=np.float64)
    m = np.mean(np.abs(X), axis=1)
    r_pre = np.sqrt(m / w)
    r = to_fp16(r_pre)
    live = r > 0
    U = np.zeros_like(X)
    U[live] = X[live] / r[live][:, None]
    a = np.max(np.abs(U), axis=0)
    code_pre = np.zeros_like(X)
    cols = a > 0
    code_pre[:, cols] = U[:, cols] * (qmax / a[cols])[None, :]
    z = np.clip(np.rint(code_pre), -qmax, qmax).astype(np.int8 if qmax <= 127 else np.int64)
    c_pre = column_factors(X, r, z.astype(np.float64), w)
    return {"z": z, "r": r, "c": to_fp16(c_pre), "r_pre": r_pre, "code_pre": code_pre, "c_pre": c_pre, "a": a}


def decode(z, r, c) -> np.ndarray:
    """X = r_i c_j z_ij."""
    return np.asarray(r, np.float64)[..., :, None] * np.asarray(c, np.float64)[..., None, :] * \
        np.asarray(z, np.float64)


def objective(X, r, c, z, w) -> float:
    """sum_ij w_i^2 (X_ij - r_i c_j z_ij)^2, the fit's weighted reconstruction error."""
    return float(np.sum((np.asarray(w, np.float64) ** 2)[:, None] * (X - decode(z, r, c)) ** 2))


def step(z, r, c, omega, q, k, v, gate, beta, qmax: int = QMAX4):
    """One decode step of nh heads on the packed state (arrays with a leading head axis):
    decode X_{t-1}, the dense step (LeapQuant App. A's expansion, the pinned dense oracle),
    y_t = X_t^T q_t, then pack X_t. Returns (y, packs, X_t)."""
    import oracle
    X = decode(z, r, c)
    y = oracle.dense_step(X, q, k, v, gate, beta)
    w = row_weights(omega)
    packs = [pack(X[h], w[h], qmax) for h in range(X.shape[0])]
    return y, packs, X
