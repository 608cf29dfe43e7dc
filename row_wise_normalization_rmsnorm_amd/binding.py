"""Python binding of librmsnorm.so (C ABI in include/rmsnorm.h).

Argument marshalling only: torch tensors become device pointers, the current
HIP stream becomes the stream argument, and every step of the computation runs
in the library's HIP kernels.  There is no fallback: if the library is not
built, or a call fails, a ``RmsnormError`` is raised.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librmsnorm.so")

DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
DTYPE_NAME = {"f32": 0, "f16": 1, "bf16": 2}
KMAX = 16
EXPORTS = ("rmsnorm_fwd", "add_rmsnorm_fwd", "rmsnorm_strerror", "rmsnorm_last_error",
           "rmsnorm_plan", "rmsnorm_variants", "rmsnorm_fwd_ex", "add_rmsnorm_fwd_ex",
           "rmsnorm_plan_ex", "rmsnorm_variants_ex", "rmsnorm_plan_call", "add_rmsnorm_ag_fwd",
           "rmsnorm_plan_ag", "rmsnorm_variants_ag", "rmsnorm_tune")
GATHER_MAX = 16
BLOCK_SUM_EXPORTS = ("block_all_reduce_sum", "block_all_reduce_sum_noalloc", "block_sum_tune")
GEMM_SCATTER_EXPORTS = ("gemm_scatter_fwd", "gemm_scatter_tile_n", "gemm_scatter_tile_m",
                        "gemm_scatter_tiles", "gemm_scatter_schedule", "gemm_scatter_tune")

# GEMM with a reduce-scatter epilogue (include/gemm_scatter.h)
GEMM_SCATTER_WORLD_MAX = 16
GEMM_SCATTER_TILE_M = 256
GEMM_SCATTER_TILE_N = 256
GEMM_SCATTER_TILE_N_NARROW = 128
GEMM_SCATTER_CUS = 256

# block all-reduce sum (include/block_sum.h)
BRS_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2,
                  torch.float8_e4m3fn: 3, torch.float8_e5m2: 4, torch.int8: 5}
BRS_MAX_GROUPS = 2048
BRS_WORKSPACE_HEADER = 4608
BRS_WORKSPACE_BYTES = BRS_WORKSPACE_HEADER + 4 * BRS_MAX_GROUPS

_lib = None
_fast = None   # the CPython marshalling module for the per-step calls, when built
_lock = threading.Lock()


class RmsnormError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RmsnormError(-7, f"{LIB_PATH} is not built; run "
                                       "`python -m row_wise_normalization_rmsnorm_amd.build`")
            l = ctypes.CDLL(LIB_PATH)
            vp, i64, c_int, c_float = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
            l.rmsnorm_fwd.argtypes = [vp, vp, vp, i64, i64, c_float, c_int, vp]
            l.rmsnorm_fwd.restype = c_int
            l.add_rmsnorm_fwd.argtypes = [vp, vp, ctypes.POINTER(vp), c_int, vp, i64, i64,
                                          c_float, c_int, vp]
            l.add_rmsnorm_fwd.restype = c_int
            l.rmsnorm_strerror.argtypes = [c_int]
            l.rmsnorm_strerror.restype = ctypes.c_char_p
            l.rmsnorm_last_error.argtypes = []
            l.rmsnorm_last_error.restype = ctypes.c_char_p
            l.rmsnorm_plan.argtypes = [i64, i64, c_int, c_int, c_int, ctypes.c_char_p, c_int]
            l.rmsnorm_plan.restype = c_int
            l.rmsnorm_variants.argtypes = [c_int, ctypes.c_char_p, c_int]
            l.rmsnorm_variants.restype = c_int
            l.rmsnorm_fwd_ex.argtypes = [vp, i64, c_int, vp, i64, c_int, vp, c_int, i64, i64,
                                         c_float, vp]
            l.rmsnorm_fwd_ex.restype = c_int
            l.add_rmsnorm_fwd_ex.argtypes = [vp, i64, c_int, vp, i64, ctypes.POINTER(vp),
                                             ctypes.POINTER(i64), c_int, c_int, vp, c_int, i64, i64,
                                             c_float, vp]
            l.add_rmsnorm_fwd_ex.restype = c_int
            l.rmsnorm_plan_ex.argtypes = [i64, i64, c_int, c_int, c_int, c_int, c_int,
                                          ctypes.c_char_p, c_int]
            l.rmsnorm_plan_ex.restype = c_int
            l.rmsnorm_variants_ex.argtypes = [c_int, c_int, c_int, ctypes.c_char_p, c_int]
            l.rmsnorm_variants_ex.restype = c_int
            l.rmsnorm_plan_call.argtypes = [vp, i64, c_int, vp, i64, ctypes.POINTER(vp),
                                            ctypes.POINTER(i64), c_int, c_int, vp, c_int, i64, i64,
                                            c_float, ctypes.c_char_p, c_int]
            l.rmsnorm_plan_call.restype = c_int
            l.add_rmsnorm_ag_fwd.argtypes = [ctypes.POINTER(vp), c_int, vp, ctypes.POINTER(vp),
                                             c_int, vp, i64, i64, c_float, c_int, vp]
            l.add_rmsnorm_ag_fwd.restype = c_int
            l.rmsnorm_plan_ag.argtypes = [i64, i64, c_int, c_int, c_int, ctypes.c_char_p, c_int]
            l.rmsnorm_plan_ag.restype = c_int
            l.rmsnorm_variants_ag.argtypes = [c_int, ctypes.c_char_p, c_int]
            l.rmsnorm_variants_ag.restype = c_int
            l.rmsnorm_tune.argtypes = [ctypes.c_char_p, i64]
            l.rmsnorm_tune.restype = c_int
            l.block_all_reduce_sum.argtypes = [vp, vp, i64, c_int, vp, i64, vp]
            l.block_all_reduce_sum.restype = c_int
            l.block_all_reduce_sum_noalloc.argtypes = [vp, vp, i64, c_int, vp]
            l.block_all_reduce_sum_noalloc.restype = c_int
            l.block_sum_tune.argtypes = [c_int]
            l.block_sum_tune.restype = c_int
            l.gemm_scatter_fwd.argtypes = [ctypes.POINTER(vp), i64, c_int, c_int, vp, i64, vp,
                                           i64, vp, i64, c_float, c_float, i64, i64, i64, c_int,
                                           vp, ctypes.c_uint32, c_int, vp]
            l.gemm_scatter_fwd.restype = c_int
            l.gemm_scatter_tile_n.argtypes = [i64, i64]
            l.gemm_scatter_tile_n.restype = c_int
            l.gemm_scatter_tile_m.argtypes = [i64, i64, c_int]
            l.gemm_scatter_tile_m.restype = c_int
            l.gemm_scatter_tune.argtypes = [c_int]
            l.gemm_scatter_tune.restype = c_int
            l.gemm_scatter_tiles.argtypes = [i64, i64, c_int]
            l.gemm_scatter_tiles.restype = i64
            l.gemm_scatter_schedule.argtypes = [i64, i64, c_int, c_int, c_int,
                                                ctypes.POINTER(ctypes.c_int32),
                                                ctypes.POINTER(ctypes.c_int32), i64]
            l.gemm_scatter_schedule.restype = c_int
            _lib = l
            global _fast
            try:
                from . import _fastcall
                _fastcall.open(LIB_PATH)
                _fast = _fastcall
            except ImportError:
                _fast = None
        return _lib


def _check(rc: int) -> None:
    if rc != 0:
        l = lib()
        raise RmsnormError(rc, f"{l.rmsnorm_strerror(rc).decode()} ({rc}): "
                               f"{l.rmsnorm_last_error().decode()}")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor, stream) -> Optional[int]:
    """The HIP stream to launch on: the given one, else torch's current
    stream on the tensor's device."""
    return _stream_on(t.get_device(), stream)


def _stream_on(dev: int, stream) -> Optional[int]:
    """The given stream, else torch's current stream on GPU ``dev``."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(dev)
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _device(t: torch.Tensor, what: str, dev: Optional[int] = None) -> int:
    """The GPU index of a device tensor.  With ``dev`` given, the tensor must
    be on that GPU: the kernels run on one GPU and address every tensor of
    the call directly, so a tensor on another GPU is refused here."""
    d = t.get_device()
    if d < 0:
        raise RmsnormError(-1, f"{what} must be a device tensor")
    if dev is not None and d != dev:
        raise RmsnormError(-1, f"{what} is on cuda:{d}, the call's other tensors on cuda:{dev}")
    return d


def _dev_ptr(t: torch.Tensor, what: str, dev: Optional[int] = None) -> int:
    _device(t, what, dev)
    if not t.is_contiguous():
        raise RmsnormError(-2, f"{what} must be contiguous")
    return t.data_ptr()


def _rows_hidden(t: torch.Tensor):
    hidden = t.shape[-1] if t.dim() > 0 else 1
    rows = t.numel() // hidden if hidden else 0
    return rows, hidden


def rmsnorm_fwd(out: torch.Tensor, x: torch.Tensor, gamma: torch.Tensor, eps: float,
                stream=None) -> None:
    """out[..., H] = RMSNorm(x[..., H]) * gamma[H] (all one dtype, contiguous)."""
    rows, hidden = _rows_hidden(x)
    if out.shape != x.shape or gamma.numel() != hidden:
        raise RmsnormError(-2, f"shape mismatch: out {tuple(out.shape)} x {tuple(x.shape)} "
                               f"gamma {tuple(gamma.shape)}")
    code = DTYPE_CODE.get(x.dtype)
    if code is None or out.dtype != x.dtype or gamma.dtype != x.dtype:
        raise RmsnormError(-3, f"dtypes must match and be f32/f16/bf16")
    dev = _device(x, "x")
    args = (_dev_ptr(out, "out", dev), _dev_ptr(x, "x"), _dev_ptr(gamma, "gamma", dev), rows,
            hidden, float(eps), code, _stream_on(dev, stream))
    l = _lib or lib()
    _check(_fast.rmsnorm_fwd(*args) if _fast else l.rmsnorm_fwd(*args))


def add_rmsnorm_fwd(out: torch.Tensor, residual: torch.Tensor, partials: Sequence[torch.Tensor],
                    gamma: torch.Tensor, eps: float, stream=None) -> None:
    """residual <- round(p0 + ... + p(K-1) + residual) in place;
    out = RMSNorm(residual) * gamma."""
    rows, hidden = _rows_hidden(residual)
    k = len(partials)
    shape, dt = residual.shape, residual.dtype
    if out.shape != shape or gamma.numel() != hidden or any(p.shape != shape for p in partials):
        raise RmsnormError(-2, "shape mismatch between out, residual, partials and gamma")
    code = DTYPE_CODE.get(dt)
    if code is None or out.dtype != dt or gamma.dtype != dt or any(p.dtype != dt for p in partials):
        raise RmsnormError(-3, "dtypes must match and be f32/f16/bf16")
    dev = _device(residual, "residual")
    ptrs = [_dev_ptr(p, f"partials[{i}]", dev) for i, p in enumerate(partials)]
    o, r = _dev_ptr(out, "out", dev), _dev_ptr(residual, "residual")
    g = _dev_ptr(gamma, "gamma", dev)
    st = _stream_on(dev, stream)
    l = _lib or lib()
    if _fast:
        _check(_fast.add_rmsnorm_fwd(o, r, ptrs, g, rows, hidden, float(eps), code, st))
    else:
        arr = (ctypes.c_void_p * max(k, 1))(*ptrs)
        _check(l.add_rmsnorm_fwd(o, r, arr, k, g, rows, hidden, float(eps), code, st))


def add_rmsnorm_ag_fwd(outs: Sequence[torch.Tensor], residual: torch.Tensor,
                       partials: Sequence[torch.Tensor], gamma: torch.Tensor, eps: float,
                       stream=None) -> None:
    """add_rmsnorm_fwd whose normalised rows go to every tensor of ``outs``
    (the all-gather epilogue): residual <- round(p0 + ... + residual) in
    place; outs[j] = RMSNorm(residual) * gamma for every j."""
    rows, hidden = _rows_hidden(residual)
    k, nout = len(partials), len(outs)
    if gamma.numel() != hidden or any(p.shape != residual.shape for p in partials) or \
            any(o.shape != residual.shape for o in outs):
        raise RmsnormError(-2, "shape mismatch between outs, residual, partials and gamma")
    if any(t.dtype != residual.dtype for t in [gamma, *outs, *partials]) or \
            residual.dtype not in DTYPE_CODE:
        raise RmsnormError(-3, "dtypes must match and be f32/f16/bf16")
    dev = _device(residual, "residual")
    arr = (ctypes.c_void_p * max(k, 1))(*[_dev_ptr(p, f"partials[{i}]", dev)
                                          for i, p in enumerate(partials)])
    oarr = (ctypes.c_void_p * max(nout, 1))(*[_dev_ptr(o, f"outs[{i}]", dev)
                                              for i, o in enumerate(outs)])
    _check(lib().add_rmsnorm_ag_fwd(oarr, nout, _dev_ptr(residual, "residual"), arr, k,
                                    _dev_ptr(gamma, "gamma", dev), rows, hidden, float(eps),
                                    DTYPE_CODE[residual.dtype], _stream_on(dev, stream)))


def rmsnorm_plan_ag(rows: int, hidden: int, k: int, dtype: str, align: int = 16) -> str:
    """Name of the variant add_rmsnorm_ag_fwd would launch (k >= 1)."""
    buf = ctypes.create_string_buffer(128)
    _check(lib().rmsnorm_plan_ag(rows, hidden, k, DTYPE_NAME[dtype], int(align), buf, 128))
    return buf.value.decode()


def rmsnorm_variants_ag(dtype: str) -> list:
    """Names of every compiled all-gather variant for dtype."""
    buf = ctypes.create_string_buffer(1 << 16)
    n = lib().rmsnorm_variants_ag(DTYPE_NAME[dtype], buf, 1 << 16)
    if n < 0:
        _check(n)
    return [s for s in buf.value.decode().split("\n") if s]


def collapse_rows(shape, strides, what: str = "tensor"):
    """(rows, hidden, row stride in elements) of a [..., hidden] layout given
    by its shape and element strides: the last dimension must be contiguous
    and the leading dimensions must collapse into one row stride (page
    "RMSNorm kernel", section 2: inputs are [..., hidden_dim]).  Raises
    otherwise: the binding never copies."""
    if len(shape) == 0:
        return 1, 1, 1
    hidden = shape[-1]
    if hidden > 1 and strides[-1] != 1:
        raise RmsnormError(-2, f"{what}: the last dimension must be contiguous")
    rows = 1
    for n in shape[:-1]:
        rows *= n
    lead = [(n, st) for n, st in zip(shape[:-1], strides[:-1]) if n != 1]
    if not lead or rows == 0:
        return rows, hidden, max(hidden, 1)
    for (n0, s0), (n1, s1) in zip(lead[:-1], lead[1:]):
        if s0 != s1 * n1:
            raise RmsnormError(-2, f"{what}: leading dimensions {tuple(shape[:-1])} with strides "
                                   f"{tuple(strides[:-1])} do not form one row stride")
    return rows, hidden, lead[-1][1]


def row_view(t: torch.Tensor, what: str, dev: Optional[int] = None):
    """collapse_rows of a device tensor (on GPU ``dev`` when given)."""
    _device(t, what, dev)
    return collapse_rows(tuple(t.shape), t.stride(), what)


def rmsnorm_fwd_ex(out: torch.Tensor, x: torch.Tensor, gamma: torch.Tensor, eps: float,
                   stream=None) -> None:
    """out[..., H] = RMSNorm(x[..., H]) * gamma[H], general form: x and out
    are any [..., H] views with a contiguous last dimension (each with its
    own row stride), gamma is float32 or x's dtype, out any of the three
    dtypes."""
    dev = _device(x, "x")
    rows, hidden, xs = row_view(x, "x")
    orows, ohidden, os_ = row_view(out, "out", dev)
    if (orows, ohidden) != (rows, hidden) or gamma.numel() != hidden:
        raise RmsnormError(-2, f"shape mismatch: out {tuple(out.shape)} x {tuple(x.shape)} "
                               f"gamma {tuple(gamma.shape)}")
    for t, n in ((x, "x"), (out, "out"), (gamma, "gamma")):
        if t.dtype not in DTYPE_CODE:
            raise RmsnormError(-3, f"{n}: dtype {t.dtype} is not f32/f16/bf16")
    _check(lib().rmsnorm_fwd_ex(out.data_ptr(), os_, DTYPE_CODE[out.dtype], x.data_ptr(), xs,
                                DTYPE_CODE[x.dtype], _dev_ptr(gamma, "gamma", dev),
                                DTYPE_CODE[gamma.dtype], rows, hidden, float(eps),
                                _stream_on(dev, stream)))


def add_rmsnorm_fwd_ex(out: torch.Tensor, residual: torch.Tensor, partials: Sequence[torch.Tensor],
                       gamma: torch.Tensor, eps: float, stream=None) -> None:
    """Fused form, general layout: residual <- round(p0 + ... + residual) in
    place (in the residual's dtype, which the partials share); out =
    RMSNorm(residual) * gamma in out's dtype.  Every tensor may be a
    [..., H] view with its own row stride."""
    dev = _device(residual, "residual")
    rows, hidden, rs = row_view(residual, "residual")
    orows, ohidden, os_ = row_view(out, "out", dev)
    k = len(partials)
    views = [row_view(p, f"partials[{i}]", dev) for i, p in enumerate(partials)]
    if (orows, ohidden) != (rows, hidden) or gamma.numel() != hidden or \
            any(v[:2] != (rows, hidden) for v in views):
        raise RmsnormError(-2, "shape mismatch between out, residual, partials and gamma")
    if any(p.dtype != residual.dtype for p in partials) or \
            any(t.dtype not in DTYPE_CODE for t in (out, residual, gamma)):
        raise RmsnormError(-3, "partials must share the residual's dtype; dtypes f32/f16/bf16")
    arr = (ctypes.c_void_p * max(k, 1))(*[p.data_ptr() for p in partials])
    strides = (ctypes.c_int64 * max(k, 1))(*[v[2] for v in views])
    _check(lib().add_rmsnorm_fwd_ex(out.data_ptr(), os_, DTYPE_CODE[out.dtype],
                                    residual.data_ptr(), rs, arr, strides, k,
                                    DTYPE_CODE[residual.dtype], _dev_ptr(gamma, "gamma", dev),
                                    DTYPE_CODE[gamma.dtype], rows, hidden, float(eps),
                                    _stream_on(dev, stream)))


def rmsnorm_plan_ex(rows: int, hidden: int, k: int, dtype: str, gamma_dtype: str,
                    out_dtype: str, align: int = 16) -> str:
    buf = ctypes.create_string_buffer(128)
    _check(lib().rmsnorm_plan_ex(rows, hidden, k, DTYPE_NAME[dtype], DTYPE_NAME[gamma_dtype],
                                 DTYPE_NAME[out_dtype], int(align), buf, 128))
    return buf.value.decode()


def rmsnorm_variants_ex(dtype: str, gamma_dtype: str, out_dtype: str) -> list:
    buf = ctypes.create_string_buffer(1 << 16)
    n = lib().rmsnorm_variants_ex(DTYPE_NAME[dtype], DTYPE_NAME[gamma_dtype],
                                  DTYPE_NAME[out_dtype], buf, 1 << 16)
    if n < 0:
        _check(n)
    return [s for s in buf.value.decode().split("\n") if s]


def rmsnorm_plan(rows: int, hidden: int, k: int, dtype: str, align: int = 16) -> str:
    """Name of the kernel variant the dispatcher picks (k = 0: plain; align:
    the alignment in bytes shared by every base pointer)."""
    buf = ctypes.create_string_buffer(128)
    _check(lib().rmsnorm_plan(rows, hidden, k, DTYPE_NAME[dtype], int(align), buf, 128))
    return buf.value.decode()


def rmsnorm_variants(dtype: str) -> list:
    """Names of every compiled kernel variant for dtype."""
    buf = ctypes.create_string_buffer(1 << 16)
    n = lib().rmsnorm_variants(DTYPE_NAME[dtype], buf, 1 << 16)
    if n < 0:
        _check(n)
    return [s for s in buf.value.decode().split("\n") if s]


def tune(variant: Optional[str] = None, grid_cap: int = 0) -> None:
    """Tuning and tests only: force a kernel variant for every later call
    (None: the dispatcher decides) and cap the workgroups per launch
    (0: the default grid).  See rmsnorm_tune in include/rmsnorm.h."""
    _check(lib().rmsnorm_tune(variant.encode() if variant else None, int(grid_cap)))


@contextlib.contextmanager
def forced(variant: Optional[str] = None, grid_cap: int = 0):
    """``with forced(name):`` runs the block with a forced variant and grid
    cap, and restores the dispatcher's choice afterwards."""
    tune(variant, grid_cap)
    try:
        yield
    finally:
        tune(None, 0)


_workspaces = {}
_ws_lock = threading.Lock()


def block_sum_workspace(device=None, stream=None) -> torch.Tensor:
    """A zeroed workspace for block_all_reduce_sum, one per (device, stream):
    calls sharing a workspace must be ordered on one stream."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    sid = _stream_on(dev.index, stream)
    with _ws_lock:
        ws = _workspaces.get((dev.index, sid))
        if ws is None:
            ws = torch.zeros(BRS_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
            # the fill runs on torch's current stream, the sums on `sid`:
            # finish it before a sum on another stream can read the counters
            torch.cuda.current_stream(dev).synchronize()
            _workspaces[(dev.index, sid)] = ws
        return ws


def block_all_reduce_sum_fwd(out: torch.Tensor, x: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> None:
    """out (one float32, or one int32 for int8 x) = sum of every element of x."""
    if x.dtype not in BRS_DTYPE_CODE:
        raise RmsnormError(-3, f"unsupported dtype {x.dtype}")
    want = torch.int32 if x.dtype == torch.int8 else torch.float32
    if out.dtype != want or out.numel() != 1:
        raise RmsnormError(-2, f"out must be one {want}")
    dev = _device(x, "x")
    if workspace is None:
        workspace = block_sum_workspace(x.device, stream)
    _check(lib().block_all_reduce_sum(_dev_ptr(out, "out", dev), _dev_ptr(x, "x") if x.numel()
                                      else x.data_ptr() or None, x.numel(),
                                      BRS_DTYPE_CODE[x.dtype],
                                      _dev_ptr(workspace, "workspace", dev), workspace.numel(),
                                      _stream_on(dev, stream)))


def block_all_reduce_sum_noalloc_fwd(out: torch.Tensor, x: torch.Tensor, stream=None) -> None:
    """block_all_reduce_sum_fwd with the library's own per-GPU scratch instead
    of a workspace (no device allocation anywhere in the call)."""
    if x.dtype not in BRS_DTYPE_CODE:
        raise RmsnormError(-3, f"unsupported dtype {x.dtype}")
    want = torch.int32 if x.dtype == torch.int8 else torch.float32
    if out.dtype != want or out.numel() != 1:
        raise RmsnormError(-2, f"out must be one {want}")
    dev = _device(x, "x")
    _check(lib().block_all_reduce_sum_noalloc(_dev_ptr(out, "out", dev), _dev_ptr(x, "x")
                                              if x.numel() else x.data_ptr() or None, x.numel(),
                                              BRS_DTYPE_CODE[x.dtype], _stream_on(dev, stream)))


def block_sum_tune(groups: int = 0) -> None:
    """Tuning and tests only: launch exactly ``groups`` workgroups per sum (0:
    the size rule)."""
    _check(lib().block_sum_tune(int(groups)))


def block_all_reduce_sum(x: torch.Tensor) -> torch.Tensor:
    out = torch.empty(1, dtype=torch.int32 if x.dtype == torch.int8 else torch.float32,
                      device=x.device)
    block_all_reduce_sum_fwd(out, x)
    return out


# GEMM with a reduce-scatter epilogue -----------------------------------------

def matrix_ld(shape, strides, what: str = "matrix") -> int:
    """Row stride in elements of a 2-D [rows, cols] layout whose elements
    are contiguous within a row.  The tensor's own stride is passed on as it
    is, so that rows which overlap or repeat (a broadcast view has stride 0)
    meet the library's check that a stride is at least a row long, instead of
    being read as if they were distinct rows; a single row's stride does not
    matter and is given as its length."""
    if len(shape) != 2 or (shape[1] > 1 and strides[1] != 1):
        raise RmsnormError(-2, f"{what} must be 2-D with contiguous rows")
    return strides[0] if shape[0] > 1 else shape[1]


def _matrix(t: torch.Tensor, what: str, dev: Optional[int] = None):
    """(pointer, row stride in elements) of a 2-D device tensor (on GPU
    ``dev`` when given) whose elements are contiguous within a row."""
    _device(t, what, dev)
    return t.data_ptr(), matrix_ld(tuple(t.shape), t.stride(), what)


def gemm_scatter_tile_n(m: int, n: int) -> int:
    """The output tile width the automatic choice (tile_n=0) takes for m x n."""
    return int(lib().gemm_scatter_tile_n(m, n))


def gemm_scatter_tile_m(m: int, n: int, tile_n: int = 0) -> int:
    """The output tile height a call with this m, n and tile width uses (256
    for 128-wide tiles; 256, 192 or 160 for 256-wide ones)."""
    return int(lib().gemm_scatter_tile_m(m, n, tile_n))


def gemm_scatter_tiles(m: int, n: int, tile_n: int = 0) -> int:
    return int(lib().gemm_scatter_tiles(m, n, tile_n))


def gemm_scatter_tune(tile_m: int = 0) -> None:
    """For tuning and testing: force the 256-wide tiles' height (256, 192 or
    160) for every later call; 0 restores the automatic choice."""
    _check(lib().gemm_scatter_tune(tile_m))


@contextlib.contextmanager
def gemm_tile_m(tile_m: int):
    """gemm_scatter_tune(tile_m) for the duration of a with-block."""
    gemm_scatter_tune(tile_m)
    try:
        yield
    finally:
        gemm_scatter_tune(0)


def gemm_scatter_schedule(m: int, n: int, world: int, rank: int, tile_n: int = 0):
    """(wg_tile, pos_tile): the tile each workgroup computes, and the tile at
    each position of the remote-first schedule."""
    t = gemm_scatter_tiles(m, n, tile_n)
    if t < 0:
        _check(-2)
    wg = (ctypes.c_int32 * max(t, 1))()
    pos = (ctypes.c_int32 * max(t, 1))()
    _check(lib().gemm_scatter_schedule(m, n, world, rank, tile_n, wg, pos, t))
    return list(wg[:t]), list(pos[:t])


def gemm_scatter_fwd(dst: Sequence[torch.Tensor], a: torch.Tensor, b: torch.Tensor,
                     c: Optional[torch.Tensor] = None, alpha: float = 1.0, beta: float = 0.0,
                     rank: int = 0, flags: Optional[torch.Tensor] = None, epoch: int = 0,
                     stream=None, tile_n: int = 0) -> None:
    """dst[q] = rows [q m/W, (q+1) m/W) of alpha * a @ b.T + beta * c, W = len(dst).

    a [m, k], b [n, k], c [m, n] and every dst[q] [m/W, n] share one 16-bit
    dtype; rows may be strided, elements within a row contiguous.  tile_n is
    the output tile width (128 or 256; 0 picks by shape).  flags
    (uint32/int32, gemm_scatter_tiles(m, n, tile_n) slots) receive ``epoch``
    per finished tile."""
    if a.dtype not in (torch.float16, torch.bfloat16):
        raise RmsnormError(-3, f"unsupported dtype {a.dtype}")
    if a.dim() != 2:
        raise RmsnormError(-2, "a must be 2-D")
    world = len(dst)
    m, k = a.shape
    n = b.shape[0]
    if b.dim() != 2 or b.shape[1] != k or (c is not None and tuple(c.shape) != (m, n)):
        raise RmsnormError(-2, "shape mismatch between a, b and c")
    for t, what in ((b, "b"), (c, "c"), *((d, "dst") for d in dst)):
        if t is not None and t.dtype != a.dtype:
            raise RmsnormError(-3, f"{what} dtype {t.dtype} differs from a's {a.dtype}")
    if world < 1 or world > GEMM_SCATTER_WORLD_MAX or m % world:
        raise RmsnormError(-2, "need 1 <= len(dst) <= 16 dividing m")
    dev = _device(a, "a")
    ldd = None
    ptrs = []
    for d in dst:
        if tuple(d.shape) != (m // world, n):
            raise RmsnormError(-2, f"every dst chunk must be [{m // world}, {n}]")
        p, ld = _matrix(d, "dst", dev)
        if ldd is not None and ld != ldd:
            raise RmsnormError(-2, "dst chunks must share one row stride")
        ldd = ld
        ptrs.append(p)
    pa, lda = _matrix(a, "a")
    pb, ldb = _matrix(b, "b", dev)
    pc, ldc = _matrix(c, "c", dev) if c is not None else (None, 0)
    pf = None
    if flags is not None:
        if flags.dtype not in (torch.int32, torch.uint32) or \
                flags.numel() < gemm_scatter_tiles(m, n, tile_n):
            raise RmsnormError(-2, "flags must be a contiguous int32 tensor with one slot per tile")
        pf = _dev_ptr(flags, "flags", dev)
    arr = (ctypes.c_void_p * world)(*ptrs)
    _check(lib().gemm_scatter_fwd(arr, ldd, world, rank, pa, lda, pb, ldb, pc, ldc,
                                  ctypes.c_float(alpha), ctypes.c_float(beta), m, n, k,
                                  DTYPE_CODE[a.dtype], pf, ctypes.c_uint32(epoch & 0xFFFFFFFF),
                                  tile_n, _stream_on(dev, stream)))


def gemm_scatter(a: torch.Tensor, b: torch.Tensor, world: int, rank: int = 0,
                 c: Optional[torch.Tensor] = None, alpha: float = 1.0,
                 beta: float = 0.0) -> list:
    """Allocating form: returns the ``world`` chunks."""
    m = a.shape[0]
    dst = [torch.empty(m // world, b.shape[0], dtype=a.dtype, device=a.device)
           for _ in range(world)]
    gemm_scatter_fwd(dst, a, b, c, alpha, beta, rank)
    return dst


# convenience wrappers ------------------------------------------------------

def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
            out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """RMSNorm of a [..., H] tensor into a new contiguous tensor (of
    out_dtype, default x's)."""
    out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    if x.is_contiguous() and out.dtype == x.dtype == gamma.dtype:
        rmsnorm_fwd(out, x, gamma, eps)
    else:
        rmsnorm_fwd_ex(out, x, gamma, eps)
    return out


def add_rmsnorm(partials: Sequence[torch.Tensor], residual: torch.Tensor, gamma: torch.Tensor,
                eps: float = 1e-6, out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Fused form; residual is updated in place, the normalised rows are
    returned in a new contiguous tensor (of out_dtype, default residual's)."""
    out = torch.empty(residual.shape, dtype=out_dtype or residual.dtype, device=residual.device)
    simple = residual.is_contiguous() and all(p.is_contiguous() for p in partials) and \
        out.dtype == residual.dtype == gamma.dtype
    if simple:
        add_rmsnorm_fwd(out, residual, partials, gamma, eps)
    else:
        add_rmsnorm_fwd_ex(out, residual, partials, gamma, eps)
    return out
