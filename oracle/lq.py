"""fp64 oracle of LeapQuant's window-boundary format -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this module. It shares no code with the HIP library. Plain numpy in fp64.

The format (LeapQuant sec. 3.3 eqs. 5-6, sec. 3.4 eq. 7, App. B.3 eq. 10): at a window
boundary the reconstructed state S is split into r compensator tokens and a residual,

    S = C * dequant(Z, B) + Kt Ut^T,   C = Diag(c),   dequant(Z, B)_ij = Z_ij B_j / 127,

where (Kt, Ut) are r key/value vector pairs stored in fp16 that approximate S's
dominant low-rank part (the argmin of ||S - K U^T||_F), c is a per-key-row smoothing
scale (the square root of the row's mean absolute residual, floored), and Z / B are
the int8 payload and fp32 per-value-channel absmax of the smoothed residual C^{-1} R.
Inside a window the state is that representation plus the buffered real-token
records; eq. 10 reads it without materializing it.

Readings taken where the pages are silent (stated once here, used everywhere):
  * the fit is subspace (block power) iteration for the top-r right singular
    subspace: V <- MGS(S^T S V), repeated n_iter times, then Kt = S V, Ut = V;
    MGS is modified Gram-Schmidt over the columns in order, a zero column stays zero;
  * the start is the previous window's Ut (orthonormalized); the first fit, from a
    plain state, starts from the first r Walsh (Sylvester-Hadamard) columns;
  * parity unpinned: the page gives the objective and names power iteration, not the
    solver; the pins fix the limit of the iteration (the truncated SVD), not the tokens
    that one warm-started iteration per boundary leaves;
  * Kt and Ut are rounded to fp16 (round to nearest even) and the residual is taken
    against the rounded tokens, so the stored pieces add up to the reconstruction;
  * the smoothing floor is 1e-6 on c; c and B are stored in fp32;
  * codes round half to even and are clamped to [-127, 127]; B_j = 0 gives Z = 0.
  * at 4 bits (the page uses r = 8 tokens there) the same recipe with codes in [-7, 7]
    and dequant(Z, B)_ij = Z_ij B_j / 7 (the /127 convention at 4 bits); on the device two
    codes share a byte, the even column in the low nibble.
  * at 6 bits (sec. 4.1 evaluates a 6-bit group but gives a token count only for 4 bits,
    so the default r = 4 holds) codes in [-31, 31] and dequant Z B / 31. The page prints
    no packing; the device stores a row of 128 codes in 96 bytes: bytes 0..63 hold the
    high parts z >> 2 (floor division by 4, a 4-bit two's complement in [-8, 7]) in the
    4-bit layout, bytes 64..95 the low parts z & 3, four per byte, column 4b + i in bits
    2i .. 2i+1 of byte 64 + b (pack6 / unpack6 below).
"""
from __future__ import annotations

import numpy as np

R_TOKENS = 4
C_FLOOR = 1e-6
QMAX8, QMAX6, QMAX4 = 127, 31, 7


def qmax_of(bits: int) -> int:
    """Largest code of the symmetric format: 127 at 8 bits, 31 at 6 bits, 7 at 4 bits."""
    return (1 << (bits - 1)) - 1


def walsh_start(d: int = 128, r: int = R_TOKENS) -> np.ndarray:
    """The first r Walsh columns of the d x d Sylvester-Hadamard matrix, orthonormal:
    entry (i, h) is (-1)^popcount(i & h) / sqrt(d)."""
    i = np.arange(d)[:, None]
    h = np.arange(r)[None, :]
    bits = np.vectorize(lambda x: bin(int(x)).count("1"))(i & h)
    return np.where(bits % 2 == 0, 1.0, -1.0) / np.sqrt(d)


def mgs(W: np.ndarray) -> np.ndarray:
    """Modified Gram-Schmidt over the columns of W, in order; a column with zero norm
    after the projections stays zero."""
    Q = np.array(W, dtype=np.float64, copy=True)
    r = Q.shape[1]
    for h in range(r):
        v = Q[:, h]
        for g in range(h):
            v = v - (Q[:, g] @ v) * Q[:, g]
        n = np.sqrt(v @ v)
        Q[:, h] = v / n if n > 0 else 0.0
    return Q


def fit(S: np.ndarray, V0: np.ndarray, n_iter: int):
    """Compensator tokens of S: n_iter steps of V <- MGS(S^T (S V)) from MGS(V0);
    returns (Kt, Ut) = (S V, V), unrounded (LeapQuant sec. 3.3, eqs. 5-6)."""
    V = mgs(V0)
    for _ in range(n_iter):
        V = mgs(S.T @ (S @ V))
    return S @ V, V


def to_fp16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest fp16 (ties to even), returned widened to fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def smooth_quantize(S: np.ndarray, K16: np.ndarray, U16: np.ndarray, qmax: int = QMAX8):
    """Residual, smoothing and per-value-channel int8 (LeapQuant sec. 3.4, eq. 7); qmax = 7
    gives the 4-bit codes.

    Returns Z (int8), B (fp32 values in fp64), c (fp32 values in fp64) and w, the
    exact pre-rounding code values (for the tie band of parity checks)."""
    R = S - K16 @ U16.T
    m = np.mean(np.abs(R), axis=1)
    c = np.float32(np.maximum(np.sqrt(m), C_FLOOR)).astype(np.float64)
    X = R / c[:, None]
    B = np.max(np.abs(X), axis=0).astype(np.float32).astype(np.float64)
    w = np.zeros_like(X)
    nz = B > 0
    w[:, nz] = X[:, nz] * float(qmax) / B[nz][None, :]
    Z = np.clip(np.rint(w), -qmax, qmax).astype(np.int8)
    return Z, B, c, w


def boundary(S: np.ndarray, V0: np.ndarray, n_iter: int, qmax: int = QMAX8) -> dict:
    """The whole boundary: fit (r = the columns of V0), fp16 tokens, residual, smoothing,
    payload."""
    K, U = fit(S, V0, n_iter)
    K16, U16 = to_fp16(K), to_fp16(U)
    Z, B, c, w = smooth_quantize(S, K16, U16, qmax)
    return {"K": K, "U": U, "K16": K16, "U16": U16, "Z": Z, "B": B, "c": c, "w": w}


def represent(Z, B, c, K16, U16, qmax: int = QMAX8) -> np.ndarray:
    """The state a window starts from: C dequant(Z, B) + Kt Ut^T (eq. 7 at l = 0)."""
    Zf = np.asarray(Z, dtype=np.float64)
    return np.asarray(c, np.float64)[:, None] * (Zf * (np.asarray(B, np.float64) / float(qmax))[None, :]) + \
        np.asarray(K16, np.float64) @ np.asarray(U16, np.float64).T


def bytes_per_element(d: int = 128, r: int = R_TOKENS, bits: int = 8) -> float:
    """Stored bytes per state element at a boundary: the payload, fp32 B and c, fp16
    token pairs (LeapQuant sec. 4.3)."""
    return (d * d * bits / 8 + d * 4 + d * 4 + 2 * r * d * 2) / (d * d)


def pack_nibbles(Z: np.ndarray) -> np.ndarray:
    """4-bit codes [..., d] in [-7, 7] -> bytes [..., d / 2]: column 2m in the low nibble,
    2m + 1 in the high nibble, each a 4-bit two's complement."""
    z = np.asarray(Z, dtype=np.int64) & 0xF
    return (z[..., 0::2] | (z[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(P: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles."""
    p = np.asarray(P, dtype=np.int64)
    lo, hi = p & 0xF, (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return out


def pack6(Z: np.ndarray) -> np.ndarray:
    """6-bit codes [..., d] in [-31, 31] -> bytes [..., 3 d / 4]: the high parts z >> 2 as
    nibbles (pack_nibbles), then the low parts z & 3, four per byte, column 4b + i in bits
    2i .. 2i+1 of byte b of the second part."""
    z = np.asarray(Z, dtype=np.int64)
    hi = pack_nibbles(z >> 2)
    lo = z & 3
    lo_bytes = lo[..., 0::4] | (lo[..., 1::4] << 2) | (lo[..., 2::4] << 4) | (lo[..., 3::4] << 6)
    return np.concatenate([hi, lo_bytes.astype(np.uint8)], axis=-1)


def unpack6(P: np.ndarray) -> np.ndarray:
    """Inverse of pack6."""
    p = np.asarray(P, dtype=np.int64)
    d = p.shape[-1] * 4 // 3
    hi = unpack_nibbles(p[..., :d // 2]).astype(np.int64)
    lb = p[..., d // 2:]
    lo = np.empty(p.shape[:-1] + (d,), dtype=np.int64)
    for i in range(4):
        lo[..., i::4] = (lb >> (2 * i)) & 3
    return (4 * hi + lo).astype(np.int8)
