"""Python binding of librsu.so, the gfx950 decode-step library for delta-rule
recurrent states (Gated DeltaNet / Kimi Delta Attention).

Argument marshalling only: every function checks torch tensors (device,
dtype, contiguity, shape), derives the ``rsu_dims`` and calls the C entry point
of the same name (include/rsu.h) on torch's current HIP stream. All the work
runs in the HIP kernels; there is no fallback. Importing this package raises
if the library has not been built (``python -m recurrent_state_update_head_amd._build``).

Shapes (B requests, H heads, d = 128):
  S, Sbase [B,H,d,d] fp32          q, k, v [B,H,d] fp32 or bf16 (all the same dtype)
  alpha, beta [B,H] fp32           d (KDA gate) [B,H,d] fp32           y [B,H,d] fp32
  Z [B,H,d,d] int8, row_absmax [B,H,d] fp32
  Kbuf [B,H,W,d] (q dtype), Ubuf [B,H,W,d] fp32, Gbuf [B,H,W] or [B,H,W,d] fp32
  Klog [B,H,C,d] (q dtype), Ulog [B,H,C,d] fp32, Lam [B,H,C] or [B,H,C,d] fp32,
  lbar [B,H] or [B,H,d] fp32, per-slot live lengths L [B,H] int32
  LeapQuant format: Z [B,H,d,d] int8, col_absmax [B,H,d] fp32, row_smooth [B,H,d] fp32,
  Kc, Uc [B,H,4,d] fp16 (4 bits: Z [B,H,d,d/2] uint8 nibbles, Kc, Uc [B,H,8,d] fp16;
  6 bits: Z [B,H,d,3d/4] uint8, high-part nibbles then low 2-bit parts, Kc, Uc [B,H,4,d])
  STEPQuant packed state: Z [B,H,d,d/2] uint8 nibbles, R, C [B,H,d] fp16, omega [B,H,d] fp32,
  u [B,H,d] fp32 (the readout's correction, consumed by the repack)
  DeltaProduct (n sub-steps per token): k, v [B,H,n,d], alpha [B,H], beta [B,H,n] fp32;
  on the int8 window Kbuf [B,H,nW,d] (q dtype), Ubuf [B,H,nW,d] fp32, Gbuf [B,H,nW] fp32
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._build import LIB as LIB_PATH

D = 128
RSU_F32, RSU_BF16 = 0, 1


class RsuError(RuntimeError):
    pass


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m recurrent_state_update_head_amd._build`")



class _Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("qkv_dtype", ctypes.c_int32)]


_P, _I = ctypes.c_void_p, ctypes.c_int
_DP = ctypes.POINTER(_Dims)
_SIGS = {
    "gdn_decode_step": [_DP, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_decode_step": [_DP, _P, _P, _P, _P, _P, _P, _P, _P],
    "q8_quantize": [_DP, _P, _P, _P, _P],
    "gdn_q8_window": [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_q8_window": [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "gdn_log_append": [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_log_append": [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "gdn_log_merge": [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_log_merge": [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "gdn_lq_quantize": [_DP, _P, _I, _P, _P, _P, _P, _P, _P],
    "gdn_lq_window": [_DP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_lq_quantize": [_DP, _P, _I, _P, _P, _P, _P, _P, _P],
    "gdn_lq4_quantize": [_DP, _P, _I, _P, _P, _P, _P, _P, _P],
    "gdn_lq4_window": [_DP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "gdn_lq6_quantize": [_DP, _P, _I, _P, _P, _P, _P, _P, _P],
    "kda_lq4_quantize": [_DP, _P, _I, _P, _P, _P, _P, _P, _P],
    "kda_lq6_quantize": [_DP, _P, _I, _P, _P, _P, _P, _P, _P],
    "kda_lq4_window": [_DP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_lq6_window": [_DP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "gdn_lq6_window": [_DP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_lq_window": [_DP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "gdn_log_step_slots": [_DP, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_log_step_slots": [_DP, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "rwkv6_decode_step": [_DP, _P, _P, _P, _P, _P, _P, _P],
    "rwkv7_decode_step": [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "rwkv7_q8_window": [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "rwkv6_log_append": [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "rwkv6_log_merge": [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "rwkv6_log_step_slots": [_DP, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "stepq_pack": [_DP, _P, _P, _P, _P, _P, _P],
    "gdn_stepq_step": [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_stepq_step": [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "gdn_stepq_readout": [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_stepq_readout": [_DP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "gdn_stepq_repack": [_DP, _P, _P, _P, _P, _P, _P, _P, _P],
    "kda_stepq_repack": [_DP, _P, _P, _P, _P, _P, _P, _P, _P],
    "deltaproduct_decode_step": [_DP, _I, _P, _P, _P, _P, _P, _P, _P, _P],
    "deltaproduct_q8_window": [_DP, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "rsu_copy_f32": [_P, _P, ctypes.c_int64, _P],
    "rsu_read_f32": [_P, _P, ctypes.c_int64, _P],
    "rsu_fill_f32": [_P, ctypes.c_float, ctypes.c_int64, _P],
    "rsu_debug_metadata_counts": [_P, ctypes.c_int64, _P],
}


def _open(path: str) -> ctypes.CDLL:
    """Load one build of the library and declare its entry points' signatures."""
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = ctypes.c_int
    lib.rsu_abi_version.restype = ctypes.c_int
    lib.rsu_last_error.restype = ctypes.c_char_p
    return lib


_lib = _open(LIB_PATH)
_fns = {name: getattr(_lib, name) for name in _SIGS}

# torch's current HIP stream as a raw handle; the private accessor skips building a Stream
# object on every call (a few microseconds, which matter beside launches of 20-30 us)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def abi_version() -> int:
    return _lib.rsu_abi_version()


def _stream():
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None):
    return t.data_ptr() if t is not None else None


def _call(name: str, *args):
    rc = _fns[name](*args)
    if rc != 0:
        raise RsuError(f"{name} returned {rc}: {_lib.rsu_last_error().decode()}")


def _need(t: torch.Tensor, name: str, dtype, shape):
    # the common case in one expression; the checks below name what is wrong
    if (isinstance(t, torch.Tensor) and t.is_cuda and (dtype is None or t.dtype == dtype) and t.shape == shape
            and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dims(q: torch.Tensor, k, v) -> _Dims:
    if q.dim() != 3 or q.shape[-1] != D:
        raise ValueError(f"q must be [B, H, {D}], got {tuple(q.shape)}")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"q, k, v must be float32 or bfloat16, got {q.dtype}")
    B, H = int(q.shape[0]), int(q.shape[1])
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, (B, H, D))
    return _Dims(B, H, D, D, RSU_BF16 if q.dtype == torch.bfloat16 else RSU_F32)


def _gate_shape(B, H, per_key):
    return (B, H, D) if per_key else (B, H)


def _step_common(dims, gate, beta, y, per_key, gname):
    B, H = dims.B, dims.H
    _need(gate, gname, torch.float32, _gate_shape(B, H, per_key))
    _need(beta, "beta", torch.float32, (B, H))
    _need(y, "y", torch.float32, (B, H, D))


def _dense(name, per_key, S, q, k, v, gate, beta, y):
    dims = _dims(q, k, v)
    _need(S, "S", torch.float32, (dims.B, dims.H, D, D))
    _step_common(dims, gate, beta, y, per_key, "d" if per_key else "alpha")
    _call(name, ctypes.byref(dims), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
          _ptr(y), _stream())
    return y


def gdn_decode_step(S, q, k, v, alpha, beta, y):
    """One GDN decode step: S updated in place, y written. Returns y."""
    return _dense("gdn_decode_step", False, S, q, k, v, alpha, beta, y)


def kda_decode_step(S, q, k, v, d, beta, y):
    """One KDA decode step (per-key gate d): S updated in place, y written. Returns y."""
    return _dense("kda_decode_step", True, S, q, k, v, d, beta, y)


def q8_quantize(S, Z, row_absmax):
    """Per-key-row int8 quantization of S into (Z, row_absmax)."""
    if S.dim() != 4:
        raise ValueError("S must be [B, H, 128, 128]")
    B, H = int(S.shape[0]), int(S.shape[1])
    _need(S, "S", torch.float32, (B, H, D, D))
    _need(Z, "Z", torch.int8, (B, H, D, D))
    _need(row_absmax, "row_absmax", torch.float32, (B, H, D))
    dims = _Dims(B, H, D, D, RSU_F32)
    _call("q8_quantize", ctypes.byref(dims), _ptr(S), _ptr(Z), _ptr(row_absmax), _stream())


def _window(name, per_key, W, pos, Z, row_absmax, Kbuf, Ubuf, Gbuf, q, k, v, gate, beta, y):
    dims = _dims(q, k, v)
    B, H = dims.B, dims.H
    _need(Z, "Z", torch.int8, (B, H, D, D))
    _need(row_absmax, "row_absmax", torch.float32, (B, H, D))
    _need(Kbuf, "Kbuf", q.dtype, (B, H, W, D))
    _need(Ubuf, "Ubuf", torch.float32, (B, H, W, D))
    _need(Gbuf, "Gbuf", torch.float32, (B, H, W, D) if per_key else (B, H, W))
    _step_common(dims, gate, beta, y, per_key, "d" if per_key else "alpha")
    _call(name, ctypes.byref(dims), int(W), int(pos), _ptr(Z), _ptr(row_absmax), _ptr(Kbuf),
          _ptr(Ubuf), _ptr(Gbuf), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(y),
          _stream())
    return y


def gdn_q8_window(W, pos, Z, row_absmax, Kbuf, Ubuf, Gbuf, q, k, v, alpha, beta, y):
    """Step pos of a window of W on the int8 state (requantizes at pos == W - 1)."""
    return _window("gdn_q8_window", False, W, pos, Z, row_absmax, Kbuf, Ubuf, Gbuf, q, k, v,
                   alpha, beta, y)


def kda_q8_window(W, pos, Z, row_absmax, Kbuf, Ubuf, Gbuf, q, k, v, d, beta, y):
    return _window("kda_q8_window", True, W, pos, Z, row_absmax, Kbuf, Ubuf, Gbuf, q, k, v, d,
                   beta, y)


def _log(name, per_key, C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, gate, beta, y):
    dims = _dims(q, k, v)
    B, H = dims.B, dims.H
    _need(Sbase, "Sbase", torch.float32, (B, H, D, D))
    _need(lbar, "lbar", torch.float32, _gate_shape(B, H, per_key))
    if C > 0:
        _need(Klog, "Klog", q.dtype, (B, H, C, D))
        _need(Ulog, "Ulog", torch.float32, (B, H, C, D))
        _need(Lam, "Lam", torch.float32, (B, H, C, D) if per_key else (B, H, C))
    _step_common(dims, gate, beta, y, per_key, "d" if per_key else "alpha")
    _call(name, ctypes.byref(dims), int(C), int(L), _ptr(Sbase), _ptr(lbar),
          _ptr(Klog if C > 0 else None), _ptr(Ulog if C > 0 else None),
          _ptr(Lam if C > 0 else None), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(y),
          _stream())
    return y


def gdn_log_append(C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, alpha, beta, y):
    """Decode step that appends entry L (requires L < C); the caller then sets L += 1."""
    return _log("gdn_log_append", False, C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, alpha, beta, y)


def kda_log_append(C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, d, beta, y):
    return _log("kda_log_append", True, C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, d, beta, y)


def gdn_log_merge(C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, alpha, beta, y):
    """Decode step that folds the log into Sbase (requires L == C); the caller then sets L = 0."""
    return _log("gdn_log_merge", False, C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, alpha, beta, y)


def kda_log_merge(C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, d, beta, y):
    return _log("kda_log_merge", True, C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, d, beta, y)


def _log_slots(name, per_key, C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, gate, beta, y):
    dims = _dims(q, k, v)
    _need(L, "L", torch.int32, (dims.B, dims.H))
    _need(Sbase, "Sbase", torch.float32, (dims.B, dims.H, D, D))
    _need(lbar, "lbar", torch.float32, _gate_shape(dims.B, dims.H, per_key))
    if C > 0:
        _need(Klog, "Klog", q.dtype, (dims.B, dims.H, C, D))
        _need(Ulog, "Ulog", torch.float32, (dims.B, dims.H, C, D))
        _need(Lam, "Lam", torch.float32, (dims.B, dims.H, C, D) if per_key else (dims.B, dims.H, C))
    _step_common(dims, gate, beta, y, per_key, "d" if per_key else "alpha")
    _call(name, ctypes.byref(dims), int(C), _ptr(L), _ptr(Sbase), _ptr(lbar),
          _ptr(Klog if C > 0 else None), _ptr(Ulog if C > 0 else None),
          _ptr(Lam if C > 0 else None), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(y),
          _stream())
    return y


def gdn_log_step_slots(C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, alpha, beta, y):
    """Decode step with a live length per head (L: int32 [B,H] on the device): heads with
    L < C append, heads with L == C merge; L is advanced in place."""
    return _log_slots("gdn_log_step_slots", False, C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, alpha,
                      beta, y)


def kda_log_step_slots(C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, d, beta, y):
    return _log_slots("kda_log_step_slots", True, C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, d, beta, y)


def rwkv6_decode_step(S, q, k, v, w, y):
    """One RWKV6 step in the common form (S <- Diag(w) S + k v^T, y = S^T q; no beta):
    S updated in place, y written. Returns y."""
    dims = _dims(q, k, v)
    _need(S, "S", torch.float32, (dims.B, dims.H, D, D))
    _need(w, "w", torch.float32, (dims.B, dims.H, D))
    _need(y, "y", torch.float32, (dims.B, dims.H, D))
    _call("rwkv6_decode_step", ctypes.byref(dims), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(y),
          _stream())
    return y


def rwkv7_decode_step(S, q, k, v, kappa, w, a, y):
    """One RWKV7 step (erase along kappa read with a * kappa, then write k v^T; y = S^T q):
    S updated in place, y written. kappa in q's dtype; w and a fp32 [B, H, 128]."""
    dims = _dims(q, k, v)
    _need(S, "S", torch.float32, (dims.B, dims.H, D, D))
    _need(kappa, "kappa", q.dtype, (dims.B, dims.H, D))
    _need(w, "w", torch.float32, (dims.B, dims.H, D))
    _need(a, "a", torch.float32, (dims.B, dims.H, D))
    _need(y, "y", torch.float32, (dims.B, dims.H, D))
    _call("rwkv7_decode_step", ctypes.byref(dims), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(kappa), _ptr(w),
          _ptr(a), _ptr(y), _stream())
    return y


def rwkv7_q8_window(W, pos, Z, row_absmax, Kbuf, Ubuf, Gbuf, q, k, v, kappa, w, a, y):
    """Token pos of a window of W on the int8 state with two records per token (records
    2 pos and 2 pos + 1; at pos == W - 1 the state is requantized from all 2W records)."""
    dims = _dims(q, k, v)
    B, H = dims.B, dims.H
    _need(Z, "Z", torch.int8, (B, H, D, D))
    _need(row_absmax, "row_absmax", torch.float32, (B, H, D))
    _need(Kbuf, "Kbuf", q.dtype, (B, H, 2 * W, D))
    _need(Ubuf, "Ubuf", torch.float32, (B, H, 2 * W, D))
    _need(Gbuf, "Gbuf", torch.float32, (B, H, 2 * W, D))
    _need(kappa, "kappa", q.dtype, (B, H, D))
    _need(w, "w", torch.float32, (B, H, D))
    _need(a, "a", torch.float32, (B, H, D))
    _need(y, "y", torch.float32, (B, H, D))
    _call("rwkv7_q8_window", ctypes.byref(dims), int(W), int(pos), _ptr(Z), _ptr(row_absmax), _ptr(Kbuf),
          _ptr(Ubuf), _ptr(Gbuf), _ptr(q), _ptr(k), _ptr(v), _ptr(kappa), _ptr(w), _ptr(a), _ptr(y), _stream())
    return y


def _dp_dims(q, k, v, alpha, beta):
    """rsu_dims and n of a DeltaProduct call: q [B,H,d], k, v [B,H,n,d] in q's dtype,
    alpha [B,H], beta [B,H,n] fp32."""
    if q.dim() != 3 or q.shape[-1] != D:
        raise ValueError(f"q must be [B, H, {D}], got {tuple(q.shape)}")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"q, k, v must be float32 or bfloat16, got {q.dtype}")
    B, H = int(q.shape[0]), int(q.shape[1])
    if k.dim() != 4:
        raise ValueError(f"k must be [B, H, n, {D}], got {tuple(k.shape)}")
    n = int(k.shape[2])
    _need(q, "q", q.dtype, (B, H, D))
    _need(k, "k", q.dtype, (B, H, n, D))
    _need(v, "v", q.dtype, (B, H, n, D))
    _need(alpha, "alpha", torch.float32, (B, H))
    _need(beta, "beta", torch.float32, (B, H, n))
    return _Dims(B, H, D, D, RSU_BF16 if q.dtype == torch.bfloat16 else RSU_F32), n


def deltaproduct_decode_step(S, q, k, v, alpha, beta, y):
    """One DeltaProduct token of n = k.shape[2] delta-rule sub-steps on the dense state S
    [B,H,d,d] (in place); y [B,H,d] is read after the last sub-step."""
    dims, n = _dp_dims(q, k, v, alpha, beta)
    _need(S, "S", torch.float32, (dims.B, dims.H, D, D))
    _need(y, "y", torch.float32, (dims.B, dims.H, D))
    _call("deltaproduct_decode_step", ctypes.byref(dims), n, _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
          _ptr(beta), _ptr(y), _stream())
    return y


def deltaproduct_q8_window(W, pos, Z, row_absmax, Kbuf, Ubuf, Gbuf, q, k, v, alpha, beta, y):
    """Token pos of a window of W on the int8 state with one record per sub-step (records
    n pos .. n pos + n - 1; at pos == W - 1 the state is requantized from all n W records).
    Kbuf [B,H,nW,d] in q's dtype, Ubuf [B,H,nW,d] fp32, Gbuf [B,H,nW] fp32."""
    dims, n = _dp_dims(q, k, v, alpha, beta)
    B, H = dims.B, dims.H
    _need(Z, "Z", torch.int8, (B, H, D, D))
    _need(row_absmax, "row_absmax", torch.float32, (B, H, D))
    _need(Kbuf, "Kbuf", q.dtype, (B, H, n * W, D))
    _need(Ubuf, "Ubuf", torch.float32, (B, H, n * W, D))
    _need(Gbuf, "Gbuf", torch.float32, (B, H, n * W))
    _need(y, "y", torch.float32, (B, H, D))
    _call("deltaproduct_q8_window", ctypes.byref(dims), n, int(W), int(pos), _ptr(Z), _ptr(row_absmax), _ptr(Kbuf),
          _ptr(Ubuf), _ptr(Gbuf), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(y), _stream())
    return y


def _rwkv6_log(name, C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, w, y):
    """L: an int for the batch-uniform calls, an int32 [B,H] device tensor per slot."""
    dims = _dims(q, k, v)
    B, H = dims.B, dims.H
    slots = isinstance(L, torch.Tensor)
    if slots:
        _need(L, "L", torch.int32, (B, H))
    _need(Sbase, "Sbase", torch.float32, (B, H, D, D))
    _need(lbar, "lbar", torch.float32, (B, H, D))
    if C > 0:
        _need(Klog, "Klog", q.dtype, (B, H, C, D))
        _need(Ulog, "Ulog", q.dtype, (B, H, C, D))
        _need(Lam, "Lam", torch.float32, (B, H, C, D))
    _need(w, "w", torch.float32, (B, H, D))
    _need(y, "y", torch.float32, (B, H, D))
    _call(name, ctypes.byref(dims), int(C), _ptr(L) if slots else int(L), _ptr(Sbase), _ptr(lbar),
          _ptr(Klog if C > 0 else None), _ptr(Ulog if C > 0 else None), _ptr(Lam if C > 0 else None),
          _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(y), _stream())
    return y


def rwkv6_log_append(C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, w, y):
    """RWKV6 base + log step that appends (k, v) as entry L (requires L < C); Ulog holds
    the raw values in q's dtype. The caller then sets L += 1."""
    return _rwkv6_log("rwkv6_log_append", C, int(L), Sbase, lbar, Klog, Ulog, Lam, q, k, v, w, y)


def rwkv6_log_merge(C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, w, y):
    """RWKV6 base + log step that folds the log into Sbase (requires L == C)."""
    return _rwkv6_log("rwkv6_log_merge", C, int(L), Sbase, lbar, Klog, Ulog, Lam, q, k, v, w, y)


def rwkv6_log_step_slots(C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, w, y):
    """RWKV6 base + log step with a live length per head (L: int32 [B,H] on the device)."""
    if not isinstance(L, torch.Tensor):
        raise ValueError("L must be an int32 [B, H] device tensor")
    return _rwkv6_log("rwkv6_log_step_slots", C, L, Sbase, lbar, Klog, Ulog, Lam, q, k, v, w, y)


def _lq_state(B, H, Z, col_absmax, row_smooth, Kc, Uc, bits=8):
    if bits == 8:
        _need(Z, "Z", torch.int8, (B, H, D, D))
    else:
        _need(Z, "Z", torch.uint8, (B, H, D, D * bits // 8))
    _need(col_absmax, "col_absmax", torch.float32, (B, H, D))
    _need(row_smooth, "row_smooth", torch.float32, (B, H, D))
    r = 8 if bits == 4 else 4
    _need(Kc, "Kc", torch.float16, (B, H, r, D))
    _need(Uc, "Uc", torch.float16, (B, H, r, D))


def _lq_quantize(name, S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, bits=8):
    if S.dim() != 4:
        raise ValueError("S must be [B, H, 128, 128]")
    B, H = S.shape[0], S.shape[1]
    _need(S, "S", torch.float32, (B, H, D, D))
    _lq_state(B, H, Z, col_absmax, row_smooth, Kc, Uc, bits)
    dims = _Dims(B, H, D, D, RSU_F32)
    _call(name, ctypes.byref(dims), _ptr(S), int(n_iter), _ptr(Z), _ptr(col_absmax),
          _ptr(row_smooth), _ptr(Kc), _ptr(Uc), _stream())


def gdn_lq_quantize(S, n_iter, Z, col_absmax, row_smooth, Kc, Uc):
    """Convert fp32 states into LeapQuant's boundary format (tokens fitted with n_iter
    subspace iterations from the Walsh start)."""
    _lq_quantize("gdn_lq_quantize", S, n_iter, Z, col_absmax, row_smooth, Kc, Uc)


def kda_lq_quantize(S, n_iter, Z, col_absmax, row_smooth, Kc, Uc):
    """The same conversion for KDA states (the format does not depend on the gates)."""
    _lq_quantize("kda_lq_quantize", S, n_iter, Z, col_absmax, row_smooth, Kc, Uc)


def _lq_window(name, per_key, W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v,
               gate, beta, y, bits=8):
    dims = _dims(q, k, v)
    B, H = dims.B, dims.H
    _lq_state(B, H, Z, col_absmax, row_smooth, Kc, Uc, bits)
    _need(Kbuf, "Kbuf", q.dtype, (B, H, W, D))
    _need(Ubuf, "Ubuf", torch.float32, (B, H, W, D))
    _need(Gbuf, "Gbuf", torch.float32, (B, H, W, D) if per_key else (B, H, W))
    _step_common(dims, gate, beta, y, per_key, "d" if per_key else "alpha")
    _call(name, ctypes.byref(dims), int(W), int(pos), int(n_iter), _ptr(Z), _ptr(col_absmax),
          _ptr(row_smooth), _ptr(Kc), _ptr(Uc), _ptr(Kbuf), _ptr(Ubuf), _ptr(Gbuf), _ptr(q), _ptr(k), _ptr(v),
          _ptr(gate), _ptr(beta), _ptr(y), _stream())
    return y


def gdn_lq_window(W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v, alpha,
                  beta, y):
    """One decode step in LeapQuant's format (eq. 10 readout; at pos = W - 1 the refit)."""
    return _lq_window("gdn_lq_window", False, W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf,
                      Gbuf, q, k, v, alpha, beta, y)


def gdn_lq4_quantize(S, n_iter, Z, col_absmax, row_smooth, Kc, Uc):
    """Convert fp32 states into LeapQuant's format at 4 bits with 8 tokens (Z: uint8
    [B, H, 128, 64] packed nibbles; Kc, Uc: fp16 [B, H, 8, 128])."""
    _lq_quantize("gdn_lq4_quantize", S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, bits=4)


def gdn_lq4_window(W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v, alpha, beta, y):
    """One decode step in the 4-bit, 8-token format (eq. 10; at pos = W - 1 the refit)."""
    return _lq_window("gdn_lq4_window", False, W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf,
                      Gbuf, q, k, v, alpha, beta, y, bits=4)


def gdn_lq6_quantize(S, n_iter, Z, col_absmax, row_smooth, Kc, Uc):
    """Convert fp32 states into LeapQuant's format at 6 bits with 4 tokens (Z: uint8
    [B, H, 128, 96], per row the high parts as nibbles then the low 2-bit parts; Kc, Uc:
    fp16 [B, H, 4, 128])."""
    _lq_quantize("gdn_lq6_quantize", S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, bits=6)


def gdn_lq6_window(W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v, alpha, beta, y):
    """One decode step in the 6-bit, 4-token format (eq. 10; at pos = W - 1 the refit)."""
    return _lq_window("gdn_lq6_window", False, W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf,
                      Gbuf, q, k, v, alpha, beta, y, bits=6)


def kda_lq4_quantize(S, n_iter, Z, col_absmax, row_smooth, Kc, Uc):
    """The 4-bit conversion for KDA states (the format does not depend on the gates)."""
    _lq_quantize("kda_lq4_quantize", S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, bits=4)


def kda_lq6_quantize(S, n_iter, Z, col_absmax, row_smooth, Kc, Uc):
    """The 6-bit conversion for KDA states (the format does not depend on the gates)."""
    _lq_quantize("kda_lq6_quantize", S, n_iter, Z, col_absmax, row_smooth, Kc, Uc, bits=6)


def kda_lq4_window(W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v, d, beta, y):
    """The 4-bit, 8-token step with KDA's per-key gate d (Gbuf holds [B, H, W, 128] gates)."""
    return _lq_window("kda_lq4_window", True, W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf,
                      Gbuf, q, k, v, d, beta, y, bits=4)


def kda_lq6_window(W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v, d, beta, y):
    """The 6-bit, 4-token step with KDA's per-key gate d (Gbuf holds [B, H, W, 128] gates)."""
    return _lq_window("kda_lq6_window", True, W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf,
                      Gbuf, q, k, v, d, beta, y, bits=6)


def kda_lq_window(W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf, Gbuf, q, k, v, d, beta, y):
    """The same step with KDA's per-key gate d (Gbuf holds [B, H, W, 128] gates)."""
    return _lq_window("kda_lq_window", True, W, pos, n_iter, Z, col_absmax, row_smooth, Kc, Uc, Kbuf, Ubuf,
                      Gbuf, q, k, v, d, beta, y)


def _stepq_state(B, H, Z, R, C, omega):
    _need(Z, "Z", torch.uint8, (B, H, D, D // 2))
    _need(R, "R", torch.float16, (B, H, D))
    _need(C, "C", torch.float16, (B, H, D))
    _need(omega, "omega", torch.float32, (B, H, D))


def stepq_pack(S, omega, Z, R, C):
    """Pack fp32 states into STEPQuant's dual-axis format: element (i, j) = R_i C_j z_ij
    (Z: uint8 [B, H, 128, 64], two signed 4-bit codes per byte, the even value column in
    the low nibble; R, C: fp16 [B, H, 128]; omega: the row influence scores)."""
    if S.dim() != 4:
        raise ValueError("S must be [B, H, 128, 128]")
    B, H = S.shape[0], S.shape[1]
    _need(S, "S", torch.float32, (B, H, D, D))
    _stepq_state(B, H, Z, R, C, omega)
    dims = _Dims(B, H, D, D, RSU_F32)
    _call("stepq_pack", ctypes.byref(dims), _ptr(S), _ptr(omega), _ptr(Z), _ptr(R), _ptr(C), _stream())


def _stepq_step(name, per_key, Z, R, C, omega, q, k, v, gate, beta, y):
    dims = _dims(q, k, v)
    _stepq_state(dims.B, dims.H, Z, R, C, omega)
    _step_common(dims, gate, beta, y, per_key, "d" if per_key else "alpha")
    _call(name, ctypes.byref(dims), _ptr(Z), _ptr(R), _ptr(C), _ptr(omega), _ptr(q), _ptr(k), _ptr(v),
          _ptr(gate), _ptr(beta), _ptr(y), _stream())
    return y


def gdn_stepq_step(Z, R, C, omega, q, k, v, alpha, beta, y):
    """One GDN decode step on the packed state: decode, update, read out y, pack again."""
    return _stepq_step("gdn_stepq_step", False, Z, R, C, omega, q, k, v, alpha, beta, y)


def kda_stepq_step(Z, R, C, omega, q, k, v, d, beta, y):
    """The same step with KDA's per-key gate d."""
    return _stepq_step("kda_stepq_step", True, Z, R, C, omega, q, k, v, d, beta, y)


def _stepq_readout(name, per_key, Z, R, C, q, k, v, gate, beta, u, y):
    dims = _dims(q, k, v)
    B, H = dims.B, dims.H
    _need(Z, "Z", torch.uint8, (B, H, D, D // 2))
    _need(R, "R", torch.float16, (B, H, D))
    _need(C, "C", torch.float16, (B, H, D))
    _need(u, "u", torch.float32, (B, H, D))
    _step_common(dims, gate, beta, y, per_key, "d" if per_key else "alpha")
    _call(name, ctypes.byref(dims), _ptr(Z), _ptr(R), _ptr(C), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
          _ptr(u), _ptr(y), _stream())
    return y


def gdn_stepq_readout(Z, R, C, q, k, v, alpha, beta, u, y):
    """The readout half of a packed-state step: writes the correction u and y; the packed
    state is only read. gdn_stepq_repack with the same u completes the step."""
    return _stepq_readout("gdn_stepq_readout", False, Z, R, C, q, k, v, alpha, beta, u, y)


def kda_stepq_readout(Z, R, C, q, k, v, d, beta, u, y):
    return _stepq_readout("kda_stepq_readout", True, Z, R, C, q, k, v, d, beta, u, y)


def _stepq_repack(name, per_key, Z, R, C, omega, k, gate, u):
    if k.dim() != 3 or k.shape[-1] != D or k.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"k must be a float32 or bfloat16 [B, H, {D}] tensor")
    B, H = int(k.shape[0]), int(k.shape[1])
    _need(k, "k", k.dtype, (B, H, D))
    _stepq_state(B, H, Z, R, C, omega)
    _need(gate, "d" if per_key else "alpha", torch.float32, _gate_shape(B, H, per_key))
    _need(u, "u", torch.float32, (B, H, D))
    dims = _Dims(B, H, D, D, RSU_BF16 if k.dtype == torch.bfloat16 else RSU_F32)
    _call(name, ctypes.byref(dims), _ptr(Z), _ptr(R), _ptr(C), _ptr(omega), _ptr(k), _ptr(gate), _ptr(u), _stream())


def gdn_stepq_repack(Z, R, C, omega, k, alpha, u):
    """The repack half: X_t = alpha X + k u^T from the packed state and the readout's u, packed
    in place (may run on another stream, ordered after its readout and before the next)."""
    _stepq_repack("gdn_stepq_repack", False, Z, R, C, omega, k, alpha, u)


def kda_stepq_repack(Z, R, C, omega, k, d, u):
    _stepq_repack("kda_stepq_repack", True, Z, R, C, omega, k, d, u)


def copy_f32(src: torch.Tensor, dst: torch.Tensor):
    """dst <- src with the dense step's access pattern (HBM ceiling probe)."""
    _need(src, "src", torch.float32, src.shape)
    _need(dst, "dst", torch.float32, src.shape)
    _call("rsu_copy_f32", _ptr(src), _ptr(dst), src.numel(), _stream())


def read_f32(src: torch.Tensor, col_sums: torch.Tensor):
    """Read-only stream over whole 128 x 128 fp32 tiles with the dense step's access pattern:
    src [..., 128, 128], col_sums [..., 128] <- the column sums of every tile."""
    if src.dim() < 2 or tuple(src.shape[-2:]) != (D, D):
        raise ValueError(f"src must be [..., {D}, {D}], got {tuple(src.shape)}")
    _need(src, "src", torch.float32, src.shape)
    _need(col_sums, "col_sums", torch.float32, tuple(src.shape[:-1]))
    _call("rsu_read_f32", _ptr(src), _ptr(col_sums), src.numel() // (D * D), _stream())


def fill_f32(dst: torch.Tensor, value: float):
    """Write-only stream over whole 128 x 128 fp32 tiles with the dense step's access
    pattern: every element of dst [..., 128, 128] <- value."""
    if dst.dim() < 2 or tuple(dst.shape[-2:]) != (D, D):
        raise ValueError(f"dst must be [..., {D}, {D}], got {tuple(dst.shape)}")
    _need(dst, "dst", torch.float32, dst.shape)
    _call("rsu_fill_f32", _ptr(dst), ctypes.c_float(value), dst.numel() // (D * D), _stream())


def debug_metadata_counts(heads: int):
    """Per-head metadata write counts of the log kernels since the last read (the checking
    build only; the ordinary build raises RsuError): a numpy uint32 array [heads, 8] with
    columns K_log elements, Lam elements, lbar elements, L, U_log elements. Waits for
    torch's current stream and clears the counters."""
    import numpy as np
    out = np.zeros((heads, 8), dtype=np.uint32)
    _call("rsu_debug_metadata_counts", out.ctypes.data_as(ctypes.c_void_p), heads, _stream())
    return out


def raw_library() -> ctypes.CDLL:
    """The loaded librsu.so (for ABI-level tests)."""
    return _lib


def select_library(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Route every later call to lib, a build opened with _open (the checking build, for
    tests); returns the library used until now."""
    global _lib, _fns
    prev = _lib
    _lib, _fns = lib, {name: getattr(lib, name) for name in _SIGS}
    return prev
