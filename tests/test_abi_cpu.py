"""The C ABI without a GPU: librsu.so loads, exports every function include/rsu.h
declares, and rejects invalid arguments before any launch (those paths make no
HIP call, so they run on a host without a device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rsu.h")
LIB = os.path.join(ROOT, "recurrent_state_update_head_amd", "librsu.so")

RSU_OK, E_NULL, E_DIMS, E_DTYPE, E_ALIGN, E_RANGE, E_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -7
CHECK_LIB = os.path.join(ROOT, "recurrent_state_update_head_amd", "librsu_check.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    return ctypes.CDLL(LIB)


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("qkv_dtype", ctypes.c_int32)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("gdn_decode_step", "kda_decode_step", "q8_quantize", "gdn_q8_window",
              "kda_q8_window", "gdn_log_append", "kda_log_append", "gdn_log_merge",
              "kda_log_merge", "rsu_last_error", "rsu_abi_version", "rsu_copy_f32"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    lib.rsu_abi_version.restype = ctypes.c_int
    assert lib.rsu_abi_version() == 1


P = ctypes.c_void_p
GOOD = P(0x1000)        # aligned, never dereferenced (every call below fails validation)
ODD = P(0x1004)


def _dense(lib, dims, S=GOOD, q=GOOD, k=GOOD, v=GOOD, g=GOOD, b=GOOD, y=GOOD):
    f = lib.gdn_decode_step
    f.restype = ctypes.c_int
    return f(ctypes.byref(dims) if dims is not None else None, S, q, k, v, g, b, y, None)


def _last(lib):
    lib.rsu_last_error.restype = ctypes.c_char_p
    return lib.rsu_last_error().decode()


def test_dense_validation(lib):
    assert _dense(lib, None) == E_NULL
    assert _dense(lib, Dims(2, 3, 64, 128, 0)) == E_DIMS
    assert "128" in _last(lib)
    assert _dense(lib, Dims(-1, 3, 128, 128, 0)) == E_DIMS
    assert _dense(lib, Dims(2, 3, 128, 128, 7)) == E_DTYPE
    assert _dense(lib, Dims(2, 3, 128, 128, 0), S=None) == E_NULL
    assert "S is NULL" in _last(lib)
    assert _dense(lib, Dims(2, 3, 128, 128, 1), y=ODD) == E_ALIGN
    assert _dense(lib, Dims(70000, 70000, 128, 128, 0)) == E_DIMS


def test_empty_batch_is_a_no_op(lib):
    assert _dense(lib, Dims(0, 48, 128, 128, 1), S=None, q=None, k=None, v=None) == RSU_OK
    assert _last(lib) == ""


def test_window_and_log_ranges(lib):
    w = lib.gdn_q8_window
    w.restype = ctypes.c_int
    d = Dims(2, 3, 128, 128, 1)
    args = [GOOD] * 11
    assert w(ctypes.byref(d), 16, 16, *args, None) == E_RANGE
    assert w(ctypes.byref(d), 0, 0, *args, None) == E_RANGE
    assert w(ctypes.byref(d), 33, 0, *args, None) == E_RANGE
    assert w(ctypes.byref(d), 16, -1, *args, None) == E_RANGE
    a = lib.gdn_log_append
    a.restype = ctypes.c_int
    m = lib.gdn_log_merge
    m.restype = ctypes.c_int
    largs = [GOOD] * 12
    assert a(ctypes.byref(d), 7, 7, *largs, None) == E_RANGE   # append needs L < C
    assert m(ctypes.byref(d), 7, 6, *largs, None) == E_RANGE   # merge needs L == C
    assert a(ctypes.byref(d), 64, 0, *largs, None) == E_RANGE  # C above the limit (M <= 64)
    assert a(ctypes.byref(d), -1, 0, *largs, None) == E_RANGE
    assert a(ctypes.byref(d), 0, 0, *largs, None) == E_RANGE   # no append with C == 0
    # C == 0 merge may pass NULL log buffers; the NULL base is still caught
    assert m(ctypes.byref(d), 0, 0, None, GOOD, None, None, None, *([GOOD] * 6), None) == E_NULL
    assert "Sbase" in _last(lib)
    sl = lib.gdn_log_step_slots
    sl.restype = ctypes.c_int
    assert sl(ctypes.byref(d), 64, *largs, None) == E_RANGE      # C above the limit
    assert sl(ctypes.byref(d), 7, None, *([GOOD] * 11), None) == E_NULL  # the live-length array
    assert "L is NULL" in _last(lib)
    assert sl(ctypes.byref(d), 7, ODD, *([GOOD] * 11), None) == E_ALIGN


def test_lq_validation(lib):
    w = lib.gdn_lq_window
    w.restype = ctypes.c_int
    d16 = Dims(2, 3, 128, 128, 1)
    args = [GOOD] * 14
    assert w(ctypes.byref(Dims(2, 3, 128, 128, 0)), 16, 0, 1, *args, None) == E_DTYPE  # bf16 only
    assert "bf16" in _last(lib)
    assert w(ctypes.byref(d16), 17, 0, 1, *args, None) == E_RANGE
    assert w(ctypes.byref(d16), 16, 16, 1, *args, None) == E_RANGE
    assert w(ctypes.byref(d16), 16, 3, -1, *args, None) == E_RANGE
    assert w(ctypes.byref(d16), 16, 3, 65, *args, None) == E_RANGE
    assert w(ctypes.byref(d16), 16, 3, 1, None, *([GOOD] * 13), None) == E_NULL
    assert w(ctypes.byref(Dims(0, 3, 128, 128, 1)), 16, 3, 1, *([None] * 14), None) == RSU_OK
    qz = lib.gdn_lq_quantize
    qz.restype = ctypes.c_int
    assert qz(ctypes.byref(d16), GOOD, 99, *([GOOD] * 5), None) == E_RANGE
    assert qz(ctypes.byref(d16), GOOD, 2, GOOD, GOOD, ODD, GOOD, GOOD, None) == E_ALIGN


def test_lq4_validation(lib):
    w = lib.gdn_lq4_window
    w.restype = ctypes.c_int
    d16 = Dims(2, 3, 128, 128, 1)
    args = [GOOD] * 14
    assert w(ctypes.byref(Dims(2, 3, 128, 128, 0)), 16, 0, 1, *args, None) == E_DTYPE  # bf16 only
    assert w(ctypes.byref(d16), 17, 0, 1, *args, None) == E_RANGE
    assert w(ctypes.byref(d16), 16, 16, 1, *args, None) == E_RANGE
    assert w(ctypes.byref(d16), 16, 3, -1, *args, None) == E_RANGE
    assert w(ctypes.byref(d16), 16, 3, 1, None, *([GOOD] * 13), None) == E_NULL
    assert w(ctypes.byref(d16), 16, 3, 1, ODD, *([GOOD] * 13), None) == E_ALIGN
    assert w(ctypes.byref(Dims(0, 3, 128, 128, 1)), 16, 3, 1, *([None] * 14), None) == RSU_OK
    qz = lib.gdn_lq4_quantize
    qz.restype = ctypes.c_int
    assert qz(ctypes.byref(d16), GOOD, 99, *([GOOD] * 5), None) == E_RANGE
    assert qz(ctypes.byref(d16), GOOD, 2, GOOD, GOOD, ODD, GOOD, GOOD, None) == E_ALIGN
    assert qz(ctypes.byref(Dims(2, 3, 128, 64, 1)), GOOD, 2, *([GOOD] * 5), None) == E_DIMS


def test_stepq_validation(lib):
    d32 = Dims(2, 3, 128, 128, 0)
    pk = lib.stepq_pack
    pk.restype = ctypes.c_int
    assert pk(ctypes.byref(d32), GOOD, None, GOOD, GOOD, GOOD, None) == E_NULL
    assert "omega is NULL" in _last(lib)
    assert pk(ctypes.byref(d32), GOOD, GOOD, GOOD, ODD, GOOD, None) == E_ALIGN
    assert pk(ctypes.byref(Dims(2, 3, 64, 128, 0)), *([GOOD] * 5), None) == E_DIMS
    assert pk(ctypes.byref(Dims(0, 3, 128, 128, 0)), *([None] * 5), None) == RSU_OK
    for name, gname in (("gdn_stepq_step", "alpha"), ("kda_stepq_step", "d")):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        args = [GOOD] * 10
        assert f(ctypes.byref(Dims(2, 3, 128, 128, 7)), *args, None) == E_DTYPE
        bad = list(args)
        bad[7] = None
        assert f(ctypes.byref(d32), *bad, None) == E_NULL
        assert f"{gname} is NULL" in _last(lib)
        bad[7] = ODD
        assert f(ctypes.byref(d32), *bad, None) == E_ALIGN
        assert f(ctypes.byref(Dims(-1, 3, 128, 128, 1)), *args, None) == E_DIMS
        assert f(ctypes.byref(Dims(2, 0, 128, 128, 1)), *([None] * 10), None) == RSU_OK


def test_stepq_split_validation(lib):
    d32 = Dims(2, 3, 128, 128, 0)
    for name, gname in (("gdn_stepq_readout", "alpha"), ("kda_stepq_readout", "d")):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        args = [GOOD] * 10
        bad = list(args)
        bad[8] = None
        assert f(ctypes.byref(d32), *bad, None) == E_NULL
        assert "u is NULL" in _last(lib)
        bad[8] = ODD
        assert f(ctypes.byref(d32), *bad, None) == E_ALIGN
        bad = list(args)
        bad[6] = None
        assert f(ctypes.byref(d32), *bad, None) == E_NULL
        assert f"{gname} is NULL" in _last(lib)
        assert f(ctypes.byref(Dims(2, 3, 128, 128, 9)), *args, None) == E_DTYPE
        assert f(ctypes.byref(Dims(0, 3, 128, 128, 1)), *([None] * 10), None) == RSU_OK
    for name, gname in (("gdn_stepq_repack", "alpha"), ("kda_stepq_repack", "d")):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        args = [GOOD] * 7
        for i, n in enumerate(("Z", "R", "C", "omega", "k", gname, "u")):
            bad = list(args)
            bad[i] = None
            assert f(ctypes.byref(d32), *bad, None) == E_NULL
            assert f"{n} is NULL" in _last(lib)
        bad = list(args)
        bad[6] = ODD
        assert f(ctypes.byref(d32), *bad, None) == E_ALIGN
        assert f(ctypes.byref(Dims(2, 3, 128, 96, 0)), *args, None) == E_DIMS
        assert f(ctypes.byref(Dims(2, 0, 128, 128, 0)), *([None] * 7), None) == RSU_OK


def test_copy_validation(lib):
    c = lib.rsu_copy_f32
    c.restype = ctypes.c_int
    c.argtypes = [P, P, ctypes.c_int64, P]
    assert c(GOOD, GOOD, 6, None) == E_DIMS
    assert c(GOOD, ODD, 8, None) == E_ALIGN
    assert c(None, None, 0, None) == RSU_OK


def test_stream_probe_validation(lib):
    r = lib.rsu_read_f32
    r.restype = ctypes.c_int
    r.argtypes = [P, P, ctypes.c_int64, P]
    w = lib.rsu_fill_f32
    w.restype = ctypes.c_int
    w.argtypes = [P, ctypes.c_float, ctypes.c_int64, P]
    assert r(GOOD, GOOD, -1, None) == E_DIMS
    assert r(GOOD, GOOD, 1 << 31, None) == E_DIMS
    assert r(GOOD, None, 4, None) == E_NULL
    assert "col_sums is NULL" in _last(lib)
    assert r(ODD, GOOD, 4, None) == E_ALIGN
    assert r(None, None, 0, None) == RSU_OK
    assert w(None, 1.0, 4, None) == E_NULL
    assert w(ODD, 1.0, 4, None) == E_ALIGN
    assert w(GOOD, 1.0, -2, None) == E_DIMS
    assert w(None, 1.0, 0, None) == RSU_OK


def test_deltaproduct_validation(lib):
    f = lib.deltaproduct_decode_step
    f.restype = ctypes.c_int
    d = Dims(2, 3, 128, 128, 1)
    args = [GOOD] * 7                                          # S, q, k, v, alpha, beta, y
    assert f(ctypes.byref(d), 0, *args, None) == E_RANGE
    assert f(ctypes.byref(d), 5, *args, None) == E_RANGE
    assert f(ctypes.byref(d), 2, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, None) == E_NULL
    assert "beta is NULL" in _last(lib)
    assert f(ctypes.byref(d), 2, GOOD, GOOD, ODD, GOOD, GOOD, GOOD, GOOD, None) == E_ALIGN
    assert f(ctypes.byref(Dims(0, 3, 128, 128, 1)), 2, *([None] * 7), None) == RSU_OK
    w = lib.deltaproduct_q8_window
    w.restype = ctypes.c_int
    wargs = [GOOD] * 11                                        # Z .. y
    assert w(ctypes.byref(d), 2, 17, 0, *wargs, None) == E_RANGE   # n W > 32
    assert w(ctypes.byref(d), 4, 9, 0, *wargs, None) == E_RANGE
    assert w(ctypes.byref(d), 2, 16, 16, *wargs, None) == E_RANGE  # pos >= W
    assert w(ctypes.byref(d), 2, 0, 0, *wargs, None) == E_RANGE
    assert w(ctypes.byref(d), 0, 8, 0, *wargs, None) == E_RANGE
    assert w(ctypes.byref(d), 2, 16, 3, *([GOOD] * 4), None, *([GOOD] * 6), None) == E_NULL
    assert "Gbuf is NULL" in _last(lib)
    assert w(ctypes.byref(Dims(2, 0, 128, 128, 1)), 2, 16, 3, *([None] * 11), None) == RSU_OK


def test_rwkv6_validation(lib):
    f = lib.rwkv6_decode_step
    f.restype = ctypes.c_int
    d = Dims(2, 3, 128, 128, 1)
    # no beta: six arrays; a NULL decay is named as w
    assert f(ctypes.byref(d), GOOD, GOOD, GOOD, GOOD, None, GOOD, None) == E_NULL
    assert "w is NULL" in _last(lib)
    assert f(ctypes.byref(Dims(2, 3, 128, 64, 1)), *([GOOD] * 6), None) == E_DIMS
    assert f(ctypes.byref(d), GOOD, GOOD, GOOD, GOOD, GOOD, ODD, None) == E_ALIGN
    assert f(ctypes.byref(Dims(0, 3, 128, 128, 1)), *([None] * 6), None) == RSU_OK
    a = lib.rwkv6_log_append
    a.restype = ctypes.c_int
    m = lib.rwkv6_log_merge
    m.restype = ctypes.c_int
    sl = lib.rwkv6_log_step_slots
    sl.restype = ctypes.c_int
    largs = [GOOD] * 10                                        # Sbase .. y
    assert a(ctypes.byref(d), 3, 3, *largs, None) == E_RANGE    # append needs L < C
    assert m(ctypes.byref(d), 3, 2, *largs, None) == E_RANGE    # merge needs L == C
    assert a(ctypes.byref(d), 64, 0, *largs, None) == E_RANGE
    assert a(ctypes.byref(d), 3, 0, *([GOOD] * 8), None, GOOD, None) == E_NULL  # w
    assert "w is NULL" in _last(lib)
    assert sl(ctypes.byref(d), 3, None, *([GOOD] * 10), None) == E_NULL       # live lengths
    assert sl(ctypes.byref(d), 3, GOOD, GOOD, GOOD, GOOD, ODD, *([GOOD] * 6), None) == E_ALIGN


def test_rwkv7_validation(lib):
    f = lib.rwkv7_decode_step
    f.restype = ctypes.c_int
    d = Dims(2, 3, 128, 128, 1)
    # S, q, k, v, kappa, w, a, y
    assert f(ctypes.byref(d), GOOD, GOOD, GOOD, GOOD, None, GOOD, GOOD, GOOD, None) == E_NULL
    assert "kappa is NULL" in _last(lib)
    assert f(ctypes.byref(d), GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, None) == E_NULL
    assert "a is NULL" in _last(lib)
    assert f(ctypes.byref(d), GOOD, GOOD, GOOD, GOOD, GOOD, ODD, GOOD, GOOD, None) == E_ALIGN
    assert f(ctypes.byref(Dims(2, 3, 128, 128, 5)), *([GOOD] * 8), None) == E_DTYPE
    assert f(ctypes.byref(Dims(0, 3, 128, 128, 1)), *([None] * 8), None) == RSU_OK


def test_checking_build_exports_the_same_symbols(lib):
    if not os.path.exists(CHECK_LIB):
        import __graft_entry__
        __graft_entry__.build()
    chk = ctypes.CDLL(CHECK_LIB)
    for n in declared_functions():
        assert hasattr(chk, n), n


def test_metadata_counts_need_the_checking_build(lib):
    f = lib.rsu_debug_metadata_counts
    f.restype = ctypes.c_int
    f.argtypes = [P, ctypes.c_int64, P]
    buf = (ctypes.c_uint32 * 32)()
    assert f(None, 4, None) == E_NULL
    assert f(ctypes.cast(buf, P), -1, None) == E_RANGE
    assert f(ctypes.cast(buf, P), 65537, None) == E_RANGE
    assert f(ctypes.cast(buf, P), 4, None) == E_UNSUPPORTED
    assert "RSU_CHECK_METADATA" in _last(lib)
