"""ctypes binding of libdlrm_mi355x.so -- argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it checks that tensors are device tensors of the
documented types (float32 or bfloat16 tables, int32 indices), passes their device pointers and the current HIP stream, and turns a
non-zero dlrm_status into a DlrmError.  There is no CPU fallback: without the
built library, or with tensors off the GPU, calls raise.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdlrm_mi355x.so")

DLRM_OK = 0
STATUS_NAMES = {0: "DLRM_OK", 1: "DLRM_ERR_NULL", 2: "DLRM_ERR_SHAPE",
                3: "DLRM_ERR_UNSUPPORTED", 4: "DLRM_ERR_WORKSPACE", 5: "DLRM_ERR_HIP"}
ACTS = {"none": 0, "relu": 1, "sigmoid": 2}
MAX_TABLES = 64
NOALLOC_SCRATCH_BYTES = 64 << 20
MAX_DIM = 1024
DTYPES = {"f32": 0, "bf16": 1, "fp8": 2}
POOLS = {"sum": 0, "mean": 1}
PLAN_MODES = {"direct": 0, "graph": 1}
FORWARD_OPTIONS = {"layered": 1, "unfused_head": 2, "unfused_bottom": 4, "unsplit_k": 8}
EXPORTS = ("dlrm_status_string", "dlrm_abi_version", "dlrm_set_kernel_timing_events",
           "dlrm_stream_read", "emb_bag_sum_multi",
           "dlrm_interact_lower_tri", "dlrm_emb_interact", "emb_bag_pool",
           "dlrm_emb_interact_pool", "dlrm_emb_interact_dots", "linear_bias_act",
           "linear_bias_act_split", "linear_bias_act_head", "mlp_forward",
           "dlrm_forward_workspace_bytes", "dlrm_forward", "dlrm_forward_noalloc",
           "dlrm_plan_create",
           "dlrm_plan_update", "dlrm_plan_run", "dlrm_plan_destroy")

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class DlrmError(RuntimeError):
    def __init__(self, status: int, call: str, message: str):
        super().__init__(f"{call}: {message}")
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


class Layer(ctypes.Structure):
    _fields_ = [("in_features", _i32), ("out_features", _i32),
                ("weight", _vp), ("bias", _vp), ("act", _i32)]


class Bags(ctypes.Structure):
    _fields_ = [("num_tables", _i32), ("batch", _i32), ("dim", _i32),
                ("table_dtype", _i32), ("pool", _i32),
                ("tables", ctypes.POINTER(_vp)), ("rows", ctypes.POINTER(_i64)),
                ("indices", ctypes.POINTER(_vp)), ("offsets", ctypes.POINTER(_vp)),
                ("n_idx", ctypes.POINTER(_i64)), ("weights", ctypes.POINTER(_vp)),
                ("scales", ctypes.POINTER(ctypes.c_float))]


class Model(ctypes.Structure):
    _fields_ = [("num_bottom", _i32), ("bottom", ctypes.POINTER(Layer)),
                ("num_top", _i32), ("top", ctypes.POINTER(Layer)),
                ("num_tables", _i32), ("dim", _i32),
                ("tables", ctypes.POINTER(_vp)), ("rows", ctypes.POINTER(_i64)),
                ("options", ctypes.c_uint32)]


_LIB = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    lib.dlrm_status_string.restype = ctypes.c_char_p
    lib.dlrm_status_string.argtypes = [ctypes.c_int]
    lib.dlrm_abi_version.restype = ctypes.c_int
    lib.dlrm_abi_version.argtypes = []
    lib.dlrm_set_kernel_timing_events.restype = ctypes.c_int
    lib.dlrm_set_kernel_timing_events.argtypes = [_vp, _vp]
    lib.dlrm_stream_read.restype = ctypes.c_int
    lib.dlrm_stream_read.argtypes = [_vp, ctypes.c_size_t, _vp, _vp]
    ptrs = ctypes.POINTER(_vp)
    lib.emb_bag_sum_multi.restype = ctypes.c_int
    lib.emb_bag_sum_multi.argtypes = [_i32, _i32, _i32, ptrs, ctypes.POINTER(_i64), ptrs,
                                      ptrs, ctypes.POINTER(_i64), _vp, _vp]
    lib.dlrm_interact_lower_tri.restype = ctypes.c_int
    lib.dlrm_interact_lower_tri.argtypes = [_i32, _i32, _i32, _vp, _vp, _vp, _vp]
    lib.dlrm_emb_interact.restype = ctypes.c_int
    lib.dlrm_emb_interact.argtypes = [_i32, _i32, _i32, ptrs, ctypes.POINTER(_i64), ptrs,
                                      ptrs, ctypes.POINTER(_i64), _vp, _vp, _vp, _vp]
    lib.emb_bag_pool.restype = ctypes.c_int
    lib.emb_bag_pool.argtypes = [ctypes.POINTER(Bags), _vp, _vp]
    lib.dlrm_emb_interact_pool.restype = ctypes.c_int
    lib.dlrm_emb_interact_pool.argtypes = [ctypes.POINTER(Bags), _vp, _vp, _vp, _vp]
    lib.dlrm_emb_interact_dots.restype = ctypes.c_int
    lib.dlrm_emb_interact_dots.argtypes = [ctypes.POINTER(Bags), _vp, _vp, _i64, _vp, _vp]
    lib.linear_bias_act_split.restype = ctypes.c_int
    lib.linear_bias_act_split.argtypes = [_i32, _i32, _i32, _vp, _i64, _i32, _vp, _i64, _vp, _vp,
                                          _i32, _vp, _i64, _vp]
    lib.linear_bias_act.restype = ctypes.c_int
    lib.linear_bias_act.argtypes = [_i32, _i32, _i32, _vp, _i64, _vp, _vp, _i32, _vp, _i64,
                                    _vp]
    lib.linear_bias_act_head.restype = ctypes.c_int
    lib.linear_bias_act_head.argtypes = [_i32, _i32, _i32, _vp, _i64, _vp, _vp, _i32, _vp, _vp,
                                         _i32, _vp, _i64, _vp]
    lib.mlp_forward.restype = ctypes.c_int
    lib.mlp_forward.argtypes = [_i32, _i32, ctypes.POINTER(Layer), _vp, _i64, _vp, _i64, _vp]
    lib.dlrm_forward_workspace_bytes.restype = ctypes.c_size_t
    lib.dlrm_forward_workspace_bytes.argtypes = [ctypes.POINTER(Model), _i32]
    lib.dlrm_forward.restype = ctypes.c_int
    lib.dlrm_forward.argtypes = [ctypes.POINTER(Model), _i32, _vp, ptrs, ptrs,
                                 ctypes.POINTER(_i64), _vp, _vp, ctypes.c_size_t, _vp]
    lib.dlrm_forward_noalloc.restype = ctypes.c_int
    lib.dlrm_forward_noalloc.argtypes = [ctypes.POINTER(Model), _i32, _vp, ptrs, ptrs,
                                         ctypes.POINTER(_i64), _vp, _vp]
    lib.dlrm_plan_create.restype = ctypes.c_int
    lib.dlrm_plan_create.argtypes = [ctypes.POINTER(Model), _i32, _vp, ptrs, ptrs,
                                     ctypes.POINTER(_i64), _vp, _vp, ctypes.c_size_t, _i32,
                                     ctypes.POINTER(_vp)]
    lib.dlrm_plan_update.restype = ctypes.c_int
    lib.dlrm_plan_update.argtypes = [_vp, _vp, ptrs, ptrs, ctypes.POINTER(_i64), _vp]
    lib.dlrm_plan_run.restype = ctypes.c_int
    lib.dlrm_plan_run.argtypes = [_vp, _vp]
    lib.dlrm_plan_destroy.restype = ctypes.c_int
    lib.dlrm_plan_destroy.argtypes = [_vp]
    if path == LIB_PATH:
        _LIB = lib
    return lib


def _check(status: int, call: str):
    if status != DLRM_OK:
        msg = load().dlrm_status_string(status).decode()
        raise DlrmError(status, call, msg)


# ------------------------------------------------------------ marshalling --
def _torch():
    import torch
    return torch


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _stream_obj(stream):
    """A torch stream object for `stream` (None: the current stream; an int:
    an external hipStream_t handle)."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def _empty(shape, device, stream, dtype=None):
    """An uninitialised float32 (or `dtype`) tensor allocated on the stream the
    call will run on, so that the caching allocator orders its reuse after
    the call's kernels."""
    torch = _torch()
    with torch.cuda.stream(_stream_obj(stream)):
        return torch.empty(shape, dtype=dtype or torch.float32, device=device)


def _dev(t, dtype, what):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a GPU tensor (got {t.device}); there is no CPU path")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _ptr_array(tensors):
    arr = (_vp * len(tensors))()
    for k, t in enumerate(tensors):
        arr[k] = t.data_ptr() if t is not None else None
    return arr


def _i64_array(values):
    arr = (_i64 * len(values))()
    for k, v in enumerate(values):
        arr[k] = int(v)
    return arr


def _tables_args(tables, indices, offsets):
    torch = _torch()
    tables = [_dev(t, torch.float32, f"tables[{k}]") for k, t in enumerate(tables)]
    indices = [_dev(i, torch.int32, f"indices[{k}]") for k, i in enumerate(indices)]
    if len(tables) != len(indices):
        raise ValueError("tables and indices must have the same length")
    if offsets is not None:
        offsets = [_dev(o, torch.int32, f"offsets[{k}]") for k, o in enumerate(offsets)]
        if len(offsets) != len(tables):
            raise ValueError("offsets must have one entry per table")
    rows = [t.shape[0] for t in tables]
    n_idx = [i.numel() for i in indices]
    return (tables, indices, offsets, _ptr_array(tables), _i64_array(rows),
            _ptr_array(indices), _ptr_array(offsets) if offsets is not None else None,
            _i64_array(n_idx))


# ---------------------------------------------------------------- entries --
def dlrm_set_kernel_timing_events(start, stop):
    """Raw hipEvent_t handles (ints) that this thread's kernel launches record
    at their start and end, or (None, None) to stop."""
    _check(load().dlrm_set_kernel_timing_events(start, stop), "dlrm_set_kernel_timing_events")


def dlrm_stream_read(buf, sink, stream=None):
    """One streaming read of the device tensor `buf` (measurement support);
    `sink` is a float32 device tensor of at least one element."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    _dev(sink, torch.float32, "sink")
    _check(load().dlrm_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                   sink.data_ptr(), _stream(stream)), "dlrm_stream_read")


def emb_bag_sum_multi(tables, indices, offsets=None, batch=None, out=None, stream=None):
    """(B, K, D) float32 pooled sums; see include/dlrm_embedding_bag.h."""
    torch = _torch()
    lib = load()
    (tables, indices, offsets, tp, rows, ip, op, nidx) = _tables_args(tables, indices, offsets)
    K = len(tables)
    D = tables[0].shape[1]
    B = offsets[0].shape[0] if offsets is not None else batch
    if B is None:
        raise ValueError("batch is required with uniform-stride (offsets=None) bags")
    if out is None:
        out = _empty((B, K, D), tables[0].device, stream)
    _dev(out, torch.float32, "out")
    _check(lib.emb_bag_sum_multi(K, B, D, tp, rows, ip, op, nidx, out.data_ptr(),
                                 _stream(stream)), "emb_bag_sum_multi")
    return out


def dlrm_interact_lower_tri(dense, emb, out=None, stream=None):
    """(B, D + F(F-1)/2) float32 = [dense | strict-lower-triangle dots]."""
    torch = _torch()
    lib = load()
    _dev(dense, torch.float32, "dense")
    _dev(emb, torch.float32, "emb")
    B, N, D = emb.shape
    P = (N + 1) * N // 2
    if out is None:
        out = _empty((B, D + P), emb.device, stream)
    _dev(out, torch.float32, "out")
    if dense.shape != (B, D) or out.shape != (B, D + P):
        raise ValueError("dense must be (B, D) and out (B, D + F(F-1)/2)")
    _check(lib.dlrm_interact_lower_tri(B, N, D, dense.data_ptr(), emb.data_ptr(),
                                       out.data_ptr(), _stream(stream)),
           "dlrm_interact_lower_tri")
    return out


def dlrm_emb_interact(tables, indices, dense, offsets=None, out=None, emb_out=None,
                      stream=None):
    """Fused gather + interaction: (B, D + F(F-1)/2) float32."""
    torch = _torch()
    lib = load()
    (tables, indices, offsets, tp, rows, ip, op, nidx) = _tables_args(tables, indices, offsets)
    _dev(dense, torch.float32, "dense")
    K = len(tables)
    B, D = dense.shape
    P = (K + 1) * K // 2
    if out is None:
        out = _empty((B, D + P), dense.device, stream)
    _dev(out, torch.float32, "out")
    if out.shape != (B, D + P):
        raise ValueError("out must be (B, D + F(F-1)/2)")
    eo = None
    if emb_out is not None:
        _dev(emb_out, torch.float32, "emb_out")
        if emb_out.shape != (B, K, D):
            raise ValueError("emb_out must be (B, K, D)")
        eo = emb_out.data_ptr()
    _check(lib.dlrm_emb_interact(K, B, D, tp, rows, ip, op, nidx, dense.data_ptr(),
                                 out.data_ptr(), eo, _stream(stream)), "dlrm_emb_interact")
    return out


class _BagsArg:
    """A dlrm_bags struct and the host arrays it points to (kept alive)."""

    def __init__(self, tables, indices, offsets, weights, pool, batch, scales=None):
        torch = _torch()
        if len(tables) == 0:
            raise ValueError("at least one table is required")
        dt = tables[0].dtype
        codes = {torch.float32: 0, torch.bfloat16: 1, torch.float8_e4m3fn: 2}
        if dt not in codes:
            raise TypeError("tables must be float32, bfloat16 or float8_e4m3fn")
        self.tables = [_dev(t, dt, f"tables[{k}]") for k, t in enumerate(tables)]
        self.indices = [_dev(i, torch.int32, f"indices[{k}]") for k, i in enumerate(indices)]
        if len(self.tables) != len(self.indices):
            raise ValueError("tables and indices must have the same length")
        self.offsets = None
        if offsets is not None:
            self.offsets = [_dev(o, torch.int32, f"offsets[{k}]") for k, o in enumerate(offsets)]
            if len(self.offsets) != len(self.tables):
                raise ValueError("offsets must have one entry per table")
            batch = self.offsets[0].shape[0]
        if batch is None:
            raise ValueError("batch is required with uniform-stride (offsets=None) bags")
        self.weights = None
        if weights is not None:
            self.weights = [_dev(w, torch.float32, f"weights[{k}]") for k, w in enumerate(weights)]
            if len(self.weights) != len(self.tables):
                raise ValueError("weights must have one entry per table")
        self.K = len(self.tables)
        self.B = int(batch)
        self.D = self.tables[0].shape[1]
        self._arrays = (_ptr_array(self.tables), _i64_array([t.shape[0] for t in self.tables]),
                        _ptr_array(self.indices),
                        _ptr_array(self.offsets) if self.offsets is not None else None,
                        _i64_array([i.numel() for i in self.indices]),
                        _ptr_array(self.weights) if self.weights is not None else None)
        tp, rows, ip, op, nidx, wp = self._arrays
        self._scales = None
        if scales is not None:
            if len(scales) != self.K:
                raise ValueError("scales must have one entry per table")
            self._scales = (ctypes.c_float * self.K)(*[float(x) for x in scales])
        self.struct = Bags(self.K, self.B, self.D, codes[dt], POOLS[pool], tp, rows, ip, op, nidx,
                           wp, self._scales)


def emb_bag_pool(tables, indices, offsets=None, weights=None, pool="sum", batch=None, out=None,
                 stream=None, scales=None):
    """(B, K, D) float32 pooled bags of float32, bfloat16 or float8_e4m3fn
    tables, sum or mean pooling, optional per-sample weights and per-table
    scales; see include/dlrm_embedding_bag.h."""
    torch = _torch()
    lib = load()
    g = _BagsArg(tables, indices, offsets, weights, pool, batch, scales)
    if out is None:
        out = _empty((g.B, g.K, g.D), g.tables[0].device, stream)
    _dev(out, torch.float32, "out")
    if out.shape != (g.B, g.K, g.D):
        raise ValueError("out must be (B, K, D)")
    _check(lib.emb_bag_pool(ctypes.byref(g.struct), out.data_ptr(), _stream(stream)),
           "emb_bag_pool")
    return out


def dlrm_emb_interact_pool(tables, indices, dense, offsets=None, weights=None, pool="sum",
                           out=None, emb_out=None, stream=None, scales=None):
    """Fused gather + interaction over any dlrm_bags form: (B, D + F(F-1)/2)."""
    torch = _torch()
    lib = load()
    _dev(dense, torch.float32, "dense")
    g = _BagsArg(tables, indices, offsets, weights, pool, dense.shape[0], scales)
    B, D = dense.shape
    if D != g.D:
        raise ValueError("dense must be (B, D)")
    P = (g.K + 1) * g.K // 2
    if out is None:
        out = _empty((B, D + P), dense.device, stream)
    _dev(out, torch.float32, "out")
    if out.shape != (B, D + P):
        raise ValueError("out must be (B, D + F(F-1)/2)")
    eo = None
    if emb_out is not None:
        _dev(emb_out, torch.float32, "emb_out")
        if emb_out.shape != (B, g.K, D):
            raise ValueError("emb_out must be (B, K, D)")
        eo = emb_out.data_ptr()
    _check(lib.dlrm_emb_interact_pool(ctypes.byref(g.struct), dense.data_ptr(), out.data_ptr(),
                                      eo, _stream(stream)), "dlrm_emb_interact_pool")
    return out


def dlrm_emb_interact_dots(tables, indices, dense, offsets=None, weights=None, pool="sum",
                           out=None, emb_out=None, stream=None, scales=None):
    """Fused gather + interaction writing only the dots: (B, F(F-1)/2) float32
    (out may be a row-strided view with unit column stride)."""
    torch = _torch()
    lib = load()
    _dev(dense, torch.float32, "dense")
    g = _BagsArg(tables, indices, offsets, weights, pool, dense.shape[0], scales)
    B, D = dense.shape
    if D != g.D:
        raise ValueError("dense must be (B, D)")
    P = (g.K + 1) * g.K // 2
    if out is None:
        out = _empty((B, P), dense.device, stream)
    if (not isinstance(out, torch.Tensor) or out.device.type != "cuda"
            or out.dtype != torch.float32 or out.shape != (B, P) or out.stride(1) != 1):
        raise ValueError("out must be a (B, F(F-1)/2) float32 GPU tensor with unit column stride")
    eo = None
    if emb_out is not None:
        _dev(emb_out, torch.float32, "emb_out")
        if emb_out.shape != (B, g.K, D):
            raise ValueError("emb_out must be (B, K, D)")
        eo = emb_out.data_ptr()
    _check(lib.dlrm_emb_interact_dots(ctypes.byref(g.struct), dense.data_ptr(), out.data_ptr(),
                                      out.stride(0), eo, _stream(stream)),
           "dlrm_emb_interact_dots")
    return out


def _matrix(t, what):
    torch = _torch()
    if (not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.float32
            or t.dim() != 2 or t.stride(1) != 1):
        raise ValueError(f"{what} must be a 2-D float32 GPU tensor with unit column stride")
    return t


def linear_bias_act_split(a_lo, a_hi, w, bias=None, act="none", out=None, stream=None):
    """act([a_lo | a_hi] @ w.T + bias) as (M, N) float32, the concat read in place."""
    torch = _torch()
    lib = load()
    _matrix(a_lo, "a_lo")
    _matrix(a_hi, "a_hi")
    _dev(w, torch.float32, "w")
    M, K_lo = a_lo.shape
    K_hi = a_hi.shape[1]
    if a_hi.shape[0] != M or w.shape[1] != K_lo + K_hi:
        raise ValueError("a_lo (M, K_lo), a_hi (M, K_hi) and w (N, K_lo + K_hi) disagree")
    N = w.shape[0]
    bp = None
    if bias is not None:
        _dev(bias, torch.float32, "bias")
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
        bp = bias.data_ptr()
    if out is None:
        out = _empty((M, N), a_lo.device, stream)
    _matrix(out, "out")
    if out.shape != (M, N):
        raise ValueError("out must be (M, N)")
    _check(lib.linear_bias_act_split(M, N, K_lo, a_lo.data_ptr(), a_lo.stride(0), K_hi,
                                     a_hi.data_ptr(), a_hi.stride(0), w.data_ptr(), bp,
                                     ACTS[act] if isinstance(act, str) else int(act),
                                     out.data_ptr(), out.stride(0), _stream(stream)),
           "linear_bias_act_split")
    return out


def linear_bias_act(a, w, bias=None, act="none", out=None, stream=None):
    """act(a @ w.T + bias) as (M, N) float32."""
    torch = _torch()
    lib = load()
    if not isinstance(a, torch.Tensor) or a.device.type != "cuda" or a.dtype != torch.float32:
        raise ValueError("a must be a float32 GPU tensor")
    if a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("a must be 2-D with unit column stride")
    _dev(w, torch.float32, "w")
    M, Kd = a.shape
    N = w.shape[0]
    if w.shape[1] != Kd:
        raise ValueError("w must be (N, K)")
    bp = None
    if bias is not None:
        _dev(bias, torch.float32, "bias")
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
        bp = bias.data_ptr()
    if out is None:
        out = _empty((M, N), a.device, stream)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape != (M, N):
        raise ValueError("out must be (M, N) with unit column stride")
    _check(lib.linear_bias_act(M, N, Kd, a.data_ptr(), a.stride(0), w.data_ptr(), bp,
                               ACTS[act] if isinstance(act, str) else int(act),
                               out.data_ptr(), out.stride(0), _stream(stream)),
           "linear_bias_act")
    return out


def linear_bias_act_head(a, w, bias, act, head_w, head_bias=None, head_act="sigmoid", out=None,
                         stream=None):
    """head_act(act(a @ w.T + bias) @ head_w + head_bias) as (M, 1) float32:
    a layer and a one-output head in one launch (n <= 256)."""
    torch = _torch()
    lib = load()
    _matrix(a, "a")
    _dev(w, torch.float32, "w")
    M, Kd = a.shape
    N = w.shape[0]
    if w.shape[1] != Kd:
        raise ValueError("w must be (N, K)")
    bp = None
    if bias is not None:
        _dev(bias, torch.float32, "bias")
        if bias.numel() != N:
            raise ValueError("bias must have N elements")
        bp = bias.data_ptr()
    _dev(head_w, torch.float32, "head_w")
    if head_w.numel() != N:
        raise ValueError("head_w must have N elements")
    hb = None
    if head_bias is not None:
        _dev(head_bias, torch.float32, "head_bias")
        if head_bias.numel() != 1:
            raise ValueError("head_bias must have one element")
        hb = head_bias.data_ptr()
    if out is None:
        out = _empty((M, 1), a.device, stream)
    if (not isinstance(out, torch.Tensor) or out.device.type != "cuda"
            or out.dtype != torch.float32 or out.dim() != 2 or out.shape != (M, 1)):
        raise ValueError("out must be an (M, 1) float32 GPU tensor")
    _check(lib.linear_bias_act_head(M, N, Kd, a.data_ptr(), a.stride(0), w.data_ptr(), bp,
                                    ACTS[act] if isinstance(act, str) else int(act),
                                    head_w.data_ptr(), hb,
                                    ACTS[head_act] if isinstance(head_act, str) else int(head_act),
                                    out.data_ptr(), max(out.stride(0), 1), _stream(stream)),
           "linear_bias_act_head")
    return out


def _layer_array(spec, what, keep):
    torch = _torch()
    arr = (Layer * len(spec))()
    for n, (wt, b, act) in enumerate(spec):
        _dev(wt, torch.float32, f"{what}[{n}].weight")
        if b is not None:
            _dev(b, torch.float32, f"{what}[{n}].bias")
        keep.extend([wt, b])
        arr[n].in_features = wt.shape[1]
        arr[n].out_features = wt.shape[0]
        arr[n].weight = wt.data_ptr()
        arr[n].bias = b.data_ptr() if b is not None else None
        arr[n].act = ACTS[act] if isinstance(act, str) else int(act)
    return arr


def mlp_forward(a, layers, out=None, stream=None):
    """A stack of (weight (out, in), bias or None, act) layers in one launch."""
    torch = _torch()
    lib = load()
    if not isinstance(a, torch.Tensor) or a.device.type != "cuda" or a.dtype != torch.float32:
        raise ValueError("a must be a float32 GPU tensor")
    if a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("a must be 2-D with unit column stride")
    keep = []
    arr = _layer_array(layers, "layers", keep)
    M = a.shape[0]
    N = layers[-1][0].shape[0]
    if out is None:
        out = _empty((M, N), a.device, stream)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape != (M, N):
        raise ValueError("out must be (M, N) with unit column stride")
    _check(lib.mlp_forward(M, len(layers), arr, a.data_ptr(), a.stride(0), out.data_ptr(),
                           out.stride(0), _stream(stream)), "mlp_forward")
    return out


def forward_options(options=()):
    """The dlrm_model.options bits of an iterable of FORWARD_OPTIONS names
    (or an int, passed through)."""
    if isinstance(options, int):
        return options
    bits = 0
    for name in options:
        if name not in FORWARD_OPTIONS:
            raise ValueError(f"unknown forward option {name!r} (known: {sorted(FORWARD_OPTIONS)})")
        bits |= FORWARD_OPTIONS[name]
    return bits


class DlrmModel:
    """Host description of a DLRMv1 model over caller-owned device tensors.

    bottom / top: lists of (weight (out, in), bias (out,) or None, act) with
    GPU float32 tensors; tables: list of (rows_k, D) GPU float32 tensors;
    options: names from FORWARD_OPTIONS ("layered": never the one-launch
    small-model kernel; "unfused_head": the last top layer as its own
    launch; "unfused_bottom": each bottom layer as its own launch), or the
    raw bits.
    """

    def __init__(self, bottom, top, tables, options=()):
        torch = _torch()
        self._keep = []
        self.tables = [_dev(t, torch.float32, f"tables[{k}]") for k, t in enumerate(tables)]
        self.dim = self.tables[0].shape[1]

        self._bottom = _layer_array(bottom, "bottom", self._keep)
        self._top = _layer_array(top, "top", self._keep)
        self._tables = _ptr_array(self.tables)
        self._rows = _i64_array([t.shape[0] for t in self.tables])
        self.out_features = top[-1][0].shape[0]
        self.options = forward_options(options)
        self.struct = Model(len(bottom), self._bottom, len(top), self._top,
                            len(self.tables), self.dim, self._tables, self._rows, self.options)

    def workspace_bytes(self, batch: int) -> int:
        return dlrm_forward_workspace_bytes(self, batch)


def dlrm_forward_workspace_bytes(model: DlrmModel, batch: int) -> int:
    return int(load().dlrm_forward_workspace_bytes(ctypes.byref(model.struct), batch))


def dlrm_forward(model: DlrmModel, dense_in, indices, offsets=None, out=None, workspace=None,
                 stream=None):
    """DLRMv1 forward: (B, top[last].out_features) float32."""
    torch = _torch()
    lib = load()
    _dev(dense_in, torch.float32, "dense_in")
    B = dense_in.shape[0]
    indices = [_dev(i, torch.int32, f"indices[{k}]") for k, i in enumerate(indices)]
    if offsets is not None:
        offsets = [_dev(o, torch.int32, f"offsets[{k}]") for k, o in enumerate(offsets)]
    need = model.workspace_bytes(B)
    # Temporaries are allocated on the stream the forward runs on, so the
    # caching allocator does not hand their blocks to other work before the
    # forward's kernels are done with them.
    s = _stream_obj(stream)
    if out is None:
        out = _empty((B, model.out_features), dense_in.device, s)
    if workspace is None:
        workspace = _empty(max(need, 1), dense_in.device, s, torch.uint8)
    _dev(out, torch.float32, "out")
    ws = workspace.data_ptr()
    _check(lib.dlrm_forward(ctypes.byref(model.struct), B, dense_in.data_ptr(),
                            _ptr_array(indices),
                            _ptr_array(offsets) if offsets is not None else None,
                            _i64_array([i.numel() for i in indices]), out.data_ptr(), ws,
                            workspace.numel() * workspace.element_size(), s.cuda_stream),
           "dlrm_forward")
    return out


def dlrm_forward_noalloc(model: DlrmModel, dense_in, indices, out, offsets=None, stream=None):
    """DLRMv1 forward into the caller's `out` (B, top[last].out_features)
    with the library's fixed scratch array as workspace: the C call
    allocates nothing (see include/dlrm_embedding_bag.h for its limit)."""
    torch = _torch()
    lib = load()
    _dev(dense_in, torch.float32, "dense_in")
    _dev(out, torch.float32, "out")
    B = dense_in.shape[0]
    indices = [_dev(i, torch.int32, f"indices[{k}]") for k, i in enumerate(indices)]
    if offsets is not None:
        offsets = [_dev(o, torch.int32, f"offsets[{k}]") for k, o in enumerate(offsets)]
    _check(lib.dlrm_forward_noalloc(ctypes.byref(model.struct), B, dense_in.data_ptr(),
                                    _ptr_array(indices),
                                    _ptr_array(offsets) if offsets is not None else None,
                                    _i64_array([i.numel() for i in indices]), out.data_ptr(),
                                    _stream(stream)),
           "dlrm_forward_noalloc")
    return out


class DlrmPlan:
    """A dlrm_forward recorded once for fixed buffers (dlrm_plan_create), as
    its packed launches (mode "direct") or as a HIP graph (mode "graph");
    run() replays it (dlrm_plan_run).  The caller writes each batch into the
    bound dense_in / indices tensors and reads `out`."""

    def __init__(self, model: DlrmModel, dense_in, indices, offsets=None, out=None,
                 workspace=None, mode="direct"):
        torch = _torch()
        self._lib = load()
        self.model = model
        self.dense_in = _dev(dense_in, torch.float32, "dense_in")
        self.batch = dense_in.shape[0]
        if out is None:
            out = torch.empty((self.batch, model.out_features), dtype=torch.float32,
                              device=dense_in.device)
        self.out = _dev(out, torch.float32, "out")
        need = model.workspace_bytes(self.batch)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dense_in.device)
        self.workspace = workspace
        self._handle = _vp()
        self._bind(indices, offsets)
        _check(self._lib.dlrm_plan_create(
            ctypes.byref(model.struct), self.batch, self.dense_in.data_ptr(), self._ip,
            self._op, self._nidx, self.out.data_ptr(), self.workspace.data_ptr(),
            self.workspace.numel() * self.workspace.element_size(), PLAN_MODES[mode],
            ctypes.byref(self._handle)),
            "dlrm_plan_create")

    def _bind(self, indices, offsets):
        torch = _torch()
        self.indices = [_dev(i, torch.int32, f"indices[{k}]") for k, i in enumerate(indices)]
        self.offsets = None
        if offsets is not None:
            self.offsets = [_dev(o, torch.int32, f"offsets[{k}]") for k, o in enumerate(offsets)]
        self._ip = _ptr_array(self.indices)
        self._op = _ptr_array(self.offsets) if self.offsets is not None else None
        self._nidx = _i64_array([i.numel() for i in self.indices])

    _KEEP = object()

    def update(self, dense_in=None, indices=None, offsets=_KEEP, out=None):
        """Rebind the per-batch buffers (dlrm_plan_update).  An argument left
        out keeps its current binding; offsets=None explicitly switches the
        plan to uniform-stride bags, and a list of tensors to CSR bags."""
        torch = _torch()
        dense = self.dense_in if dense_in is None else _dev(dense_in, torch.float32, "dense_in")
        o = self.out if out is None else _dev(out, torch.float32, "out")
        new_idx = self.indices if indices is None else indices
        new_off = self.offsets if offsets is DlrmPlan._KEEP else offsets
        saved = (self.indices, self.offsets, self._ip, self._op, self._nidx)
        self._bind(new_idx, new_off)
        rc = self._lib.dlrm_plan_update(self._handle, dense.data_ptr(), self._ip, self._op,
                                        self._nidx, o.data_ptr())
        if rc != DLRM_OK:
            (self.indices, self.offsets, self._ip, self._op, self._nidx) = saved
            _check(rc, "dlrm_plan_update")
        self.dense_in = dense
        self.out = o

    def run(self, stream=None):
        _check(self._lib.dlrm_plan_run(self._handle, _stream(stream)), "dlrm_plan_run")
        return self.out

    def close(self):
        if self._handle:
            _check(self._lib.dlrm_plan_destroy(self._handle), "dlrm_plan_destroy")
            self._handle = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
