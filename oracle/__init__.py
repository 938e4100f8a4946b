"""CPU oracle of the DLRMv1 forward hot path (numpy front end over oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__.py
and the cpu_baseline leg of bench.py may import this package.  It never imports
the HIP library package and the HIP library never imports it.

Every function takes and returns host numpy arrays; the arithmetic happens in
oracle.c (fp64 sums, one rounding to float32 per output element).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)

ACT_NONE, ACT_RELU, ACT_SIGMOID = 0, 1, 2
_ACTS = {"none": ACT_NONE, "relu": ACT_RELU, "sigmoid": ACT_SIGMOID}


class OracleError(RuntimeError):
    """An argument the oracle rejects (bad size, index or offset)."""


class _Layer(ctypes.Structure):
    _fields_ = [("in_features", ctypes.c_int32),
                ("out_features", ctypes.c_int32),
                ("weight", _f32p),
                ("bias", _f32p),
                ("act", ctypes.c_int32)]


def load(path: str = None):
    """Load liboracle.so, compiling it first if it is not there."""
    global _LIB
    if path is None and _LIB is not None:
        return _LIB
    lib_path = path or _build.LIB
    if not os.path.exists(lib_path):
        _build.build()
    lib = ctypes.CDLL(lib_path)
    lib.oracle_pair_count.restype = ctypes.c_int64
    lib.oracle_pair_count.argtypes = [ctypes.c_int64]
    lib.oracle_pair_enumerate.argtypes = [ctypes.c_int64, _i32p, _i32p]
    lib.oracle_pair_closed_form.argtypes = [ctypes.c_int64, _i64p, _i64p]
    lib.oracle_pair_closed_form_range.argtypes = [ctypes.c_int64, ctypes.c_int64,
                                                  _i32p, _i32p]
    lib.oracle_emb_bag_sum.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.POINTER(_f32p), _i64p, ctypes.POINTER(_i32p),
        ctypes.POINTER(_i32p), _i64p, _f32p]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_fp8_e4m3_to_f64.restype = ctypes.c_double
    lib.oracle_fp8_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_emb_bag.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.POINTER(ctypes.c_void_p), _i64p, ctypes.POINTER(_i32p),
        ctypes.POINTER(_i32p), ctypes.POINTER(_f32p), _i64p, ctypes.c_int32, _f32p, _f32p]
    lib.oracle_interact.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    _f32p, _f32p, _f32p]
    lib.oracle_linear.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  _f32p, ctypes.c_int64, _f32p, _f32p,
                                  ctypes.c_int32, _f32p, ctypes.c_int64]
    lib.oracle_forward.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_Layer), ctypes.c_int32,
        ctypes.POINTER(_Layer), ctypes.c_int32, ctypes.c_int32,
        ctypes.POINTER(_f32p), _i64p, _f32p, ctypes.POINTER(_i32p),
        ctypes.POINTER(_i32p), _i64p, _f32p, _f32p, _f32p]
    if path is None:
        _LIB = lib
    return lib


def _p(a, ptype):
    return a.ctypes.data_as(ptype)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} rejected its arguments (code {rc})")


def pair_count(F: int) -> int:
    return int(load().oracle_pair_count(F))


def pair_enumerate(F: int, lib=None):
    """(i, j) arrays of the strict lower triangle, row by row."""
    lib = lib or load()
    n = pair_count(F)
    pi = np.empty(max(n, 1), np.int32)
    pj = np.empty(max(n, 1), np.int32)
    _check(lib.oracle_pair_enumerate(F, _p(pi, _i32p), _p(pj, _i32p)), "pair_enumerate")
    return pi[:n], pj[:n]


def pair_closed_form(p: int, lib=None):
    lib = lib or load()
    i = ctypes.c_int64()
    j = ctypes.c_int64()
    _check(lib.oracle_pair_closed_form(p, ctypes.byref(i), ctypes.byref(j)),
           "pair_closed_form")
    return i.value, j.value


def pair_closed_form_range(p0: int, n: int, lib=None):
    lib = lib or load()
    pi = np.empty(max(n, 1), np.int32)
    pj = np.empty(max(n, 1), np.int32)
    _check(lib.oracle_pair_closed_form_range(p0, n, _p(pi, _i32p), _p(pj, _i32p)),
           "pair_closed_form_range")
    return pi[:n], pj[:n]


def _ptr_array(arrays, ptype):
    arr = (ptype * len(arrays))()
    for k, a in enumerate(arrays):
        arr[k] = ctypes.cast(a.ctypes.data, ptype)
    return arr


def emb_bag_sum(tables, indices, offsets=None, batch=None, lib=None):
    """Pooled (B, K, D) float32.

    tables  : list of K (rows_k, D) float32 arrays
    indices : list of K (n_idx_k,) int32 arrays
    offsets : None (uniform stride, L_k = n_idx_k / B) or list of K (B,) int32
    batch   : B (required when offsets is None)
    """
    lib = lib or load()
    K = len(tables)
    tables = [_f32(t) for t in tables]
    indices = [_i32(i) for i in indices]
    D = tables[0].shape[1]
    if offsets is not None:
        offsets = [_i32(o) for o in offsets]
        B = offsets[0].shape[0]
    else:
        B = batch
    rows = np.array([t.shape[0] for t in tables], np.int64)
    n_idx = np.array([i.shape[0] for i in indices], np.int64)
    # keep a non-empty buffer alive for empty index arrays
    idx_bufs = [i if i.size else np.zeros(1, np.int32) for i in indices]
    out = np.empty((B, K, D), np.float32)
    rc = lib.oracle_emb_bag_sum(
        K, B, D, _ptr_array(tables, _f32p), _p(rows, _i64p),
        _ptr_array(idx_bufs, _i32p),
        _ptr_array(offsets, _i32p) if offsets is not None else None,
        _p(n_idx, _i64p), _p(out, _f32p))
    _check(rc, "emb_bag_sum")
    return out


POOLS = {"sum": 0, "mean": 1}


def bf16_to_f32(bits, lib=None):
    """float32 value of each uint16 bfloat16 bit pattern (elementwise)."""
    lib = lib or load()
    bits = np.asarray(bits, np.uint16)
    return np.array([lib.oracle_bf16_to_f32(int(b)) for b in bits.ravel()],
                    np.float32).reshape(bits.shape)


def fp8_e4m3_to_f64(codes, lib=None):
    """float64 value of each uint8 FP8 E4M3 code (elementwise)."""
    lib = lib or load()
    codes = np.asarray(codes, np.uint8)
    return np.array([lib.oracle_fp8_e4m3_to_f64(int(c)) for c in codes.ravel()],
                    np.float64).reshape(codes.shape)


_DTYPES = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.uint8): 2}


def emb_bag(tables, indices, offsets=None, batch=None, weights=None, pool="sum", scales=None,
            lib=None):
    """Pooled (B, K, D) float32 with mean pooling, per-sample weights and
    narrow table storage: uint16 tables hold bfloat16 bit patterns, uint8
    tables FP8 E4M3 codes; scales (K,) multiplies each table's pooled value."""
    lib = lib or load()
    K = len(tables)
    dt = np.asarray(tables[0]).dtype
    code = _DTYPES.get(dt, 0)
    store = {0: np.float32, 1: np.uint16, 2: np.uint8}[code]
    tables = [np.ascontiguousarray(t, store) for t in tables]
    indices = [_i32(i) for i in indices]
    D = tables[0].shape[1]
    if offsets is not None:
        offsets = [_i32(o) for o in offsets]
        B = offsets[0].shape[0]
    else:
        B = batch
    rows = np.array([t.shape[0] for t in tables], np.int64)
    n_idx = np.array([i.shape[0] for i in indices], np.int64)
    idx_bufs = [i if i.size else np.zeros(1, np.int32) for i in indices]
    tab_ptrs = (ctypes.c_void_p * K)(*[t.ctypes.data for t in tables])
    w_ptrs = None
    if weights is not None:
        weights = [_f32(w) if np.asarray(w).size else np.zeros(1, np.float32) for w in weights]
        w_ptrs = _ptr_array(weights, _f32p)
    out = np.empty((B, K, D), np.float32)
    sc = _f32(scales) if scales is not None else None
    rc = lib.oracle_emb_bag(
        K, B, D, code, tab_ptrs, _p(rows, _i64p), _ptr_array(idx_bufs, _i32p),
        _ptr_array(offsets, _i32p) if offsets is not None else None, w_ptrs,
        _p(n_idx, _i64p), POOLS[pool], _p(sc, _f32p) if sc is not None else None,
        _p(out, _f32p))
    _check(rc, "emb_bag")
    return out


def interact(dense, emb, lib=None):
    """[dense | strict-lower-triangle dots] as (B, D + F(F-1)/2) float32."""
    lib = lib or load()
    dense = _f32(dense)
    emb = _f32(emb)
    B, K, D = emb.shape
    assert dense.shape == (B, D)
    P = (K + 1) * K // 2
    out = np.empty((B, D + P), np.float32)
    _check(lib.oracle_interact(B, K, D, _p(dense, _f32p), _p(emb, _f32p),
                               _p(out, _f32p)), "interact")
    return out


def linear(a, w, bias=None, act="none", lib=None):
    """act(a @ w.T + bias) as float32; a (M, K), w (N, K), bias (N,)."""
    lib = lib or load()
    a = _f32(a)
    w = _f32(w)
    M, Kd = a.shape
    N = w.shape[0]
    assert w.shape[1] == Kd
    b = _f32(bias) if bias is not None else None
    out = np.empty((M, N), np.float32)
    rc = lib.oracle_linear(M, N, Kd, _p(a, _f32p), Kd, _p(w, _f32p),
                           _p(b, _f32p) if b is not None else None,
                           _ACTS[act] if isinstance(act, str) else act,
                           _p(out, _f32p), N)
    _check(rc, "linear")
    return out


def forward(dense_in, bottom, top, tables, indices, offsets=None, lib=None):
    """DLRMv1 forward.

    bottom / top : lists of (weight (out, in), bias (out,) or None, act str)
    Returns (out, R, E).
    """
    lib = lib or load()
    dense_in = _f32(dense_in)
    B = dense_in.shape[0]
    tables = [_f32(t) for t in tables]
    indices = [_i32(i) for i in indices]
    K = len(tables)
    D = tables[0].shape[1]
    keep = []

    def layers(spec):
        arr = (_Layer * len(spec))()
        for n, (w, b, act) in enumerate(spec):
            w = _f32(w)
            b = _f32(b) if b is not None else None
            keep.extend([w, b])
            arr[n].in_features = w.shape[1]
            arr[n].out_features = w.shape[0]
            arr[n].weight = _p(w, _f32p)
            arr[n].bias = _p(b, _f32p) if b is not None else None
            arr[n].act = _ACTS[act]
        return arr

    bl = layers(bottom)
    tl = layers(top)
    rows = np.array([t.shape[0] for t in tables], np.int64)
    n_idx = np.array([i.shape[0] for i in indices], np.int64)
    if offsets is not None:
        offsets = [_i32(o) for o in offsets]
    P = (K + 1) * K // 2
    out = np.empty((B, top[-1][0].shape[0]), np.float32)
    R = np.empty((B, D + P), np.float32)
    E = np.empty((B, K, D), np.float32)
    rc = lib.oracle_forward(
        B, len(bottom), bl, len(top), tl, K, D, _ptr_array(tables, _f32p),
        _p(rows, _i64p), _p(dense_in, _f32p), _ptr_array(indices, _i32p),
        _ptr_array(offsets, _i32p) if offsets is not None else None,
        _p(n_idx, _i64p), _p(out, _f32p), _p(R, _f32p), _p(E, _f32p))
    _check(rc, "forward")
    return out, R, E
