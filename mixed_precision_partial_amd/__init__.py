"""Python binding of the MI355X mixed-precision partial-sum reduce (``include/ar.h``).

Argument marshalling only: every step of the reduce runs in the HIP library
``libmpp_ar.so`` built from ``csrc/`` for gfx950.  The binding loads that
library and nothing else; if it is missing, importing succeeds but the first
call raises ``RuntimeError`` -- there is no fallback path.

The functions carry the C names:

    ctx = ar_init(device=0, config=None)
    ar_reduce(ctx, dsts, srcs, n, dst_type, wire_type, mode, stream=None)
    ar_reduce_add(ctx, dsts, srcs, n, dst_type, wire_type, mode, residual, residual_len, stream=None)
    ar_reduce_rows(ctx, dsts, srcs, rows, cols, src_stride, dst_stride, dst_type, wire_type, mode,
                   residual=None, res_stride=0, stream=None)
    ar_free(ctx)
    ar_status_str(code)
    ar_plan_query(...), ar_plan_query_add(...), ar_plan_query_rows(...)

``dsts`` / ``srcs`` are sequences of torch tensors or raw integer addresses, or
ready-made ``ptr_array(...)`` arrays (passed through unchanged, which keeps
the per-call marshalling cost low for latency-bound callers); ``stream`` is a
``torch.cuda.Stream``, a raw ``hipStream_t`` integer, or None for the null
stream.

The library sees only pointers, so it cannot tell how large a buffer is.  With
``validate=True`` (the default) the enqueueing calls check, before calling it,
that every tensor argument spans the bytes the call will read or write from its
data pointer (and, for the 1-D calls, that it is contiguous), raising
``ValueError`` otherwise; integer addresses and ``ptr_array`` arrays are the
caller's responsibility, as in C.  ``bind_reduce`` and ``bind_reduce_rows`` check once,
when they bind.
"""
from __future__ import annotations

import ctypes
import os

AR_F32, AR_F16, AR_BF16 = 0, 1, 2
AR_MODE_AUTO, AR_MODE_SINGLE_SHOT, AR_MODE_CHUNKED, AR_MODE_RS_BCAST, AR_MODE_HOST_STAGED = 0, 1, 2, 3, 4
AR_MODE_MASK = 0xFF
AR_SRC_WIRE = 0x100
AR_SRC_INACTIVE_NULL = 0x200
AR_MAX_RANKS = 16

AR_OK, AR_ERR_INVALID, AR_ERR_UNSUPPORTED, AR_ERR_NOMEM, AR_ERR_RUNTIME = 0, 1, 2, 3, 4

MODE_NAMES = {
    AR_MODE_AUTO: "auto", AR_MODE_SINGLE_SHOT: "single_shot", AR_MODE_CHUNKED: "chunked",
    AR_MODE_RS_BCAST: "rs_bcast", AR_MODE_HOST_STAGED: "host_staged",
}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmpp_ar.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "ar.h")


class ArConfig(ctypes.Structure):
    _fields_ = [
        ("single_shot_max_bytes", ctypes.c_size_t),
        ("chunk_bytes", ctypes.c_size_t),
        ("host_chunk_bytes", ctypes.c_size_t),
        ("host_slots", ctypes.c_int),
        ("grid_wgs", ctypes.c_int),
        ("stream_kernel", ctypes.c_int),
        ("store_policy", ctypes.c_int),
        ("host_path", ctypes.c_int),
        ("xcd_run_elems", ctypes.c_size_t),
        ("occupancy_hold", ctypes.c_int),
    ]


class ArPlan(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int),
        ("n_dst", ctypes.c_int),
        ("src_bytes", ctypes.c_int),
        ("wire_bytes", ctypes.c_int),
        ("chunk_elems", ctypes.c_size_t),
        ("n_chunks", ctypes.c_size_t),
        ("slice_start", ctypes.c_size_t * AR_MAX_RANKS),
        ("slice_len", ctypes.c_size_t * AR_MAX_RANKS),
        ("algo_bytes", ctypes.c_size_t),
        ("store_nt", ctypes.c_int),
        ("host_direct", ctypes.c_int),
        ("stream_kernel", ctypes.c_int),
        ("active_mask", ctypes.c_uint),
        ("dst_bytes", ctypes.c_int),
        ("residual_kind", ctypes.c_int),
        ("hold_waves", ctypes.c_int),
    ]


class ArRows(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_size_t),
        ("cols", ctypes.c_size_t),
        ("src_stride", ctypes.c_size_t),
        ("dst_stride", ctypes.c_size_t),
        ("res_stride", ctypes.c_size_t),
    ]


class ArError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {ar_status_str(status)} ({status})" if what else ar_status_str(status))


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmpp_ar.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing: build it with "
            "`python -m mixed_precision_partial_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.ar_init.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.POINTER(ArConfig)]
    lib.ar_init.restype = ctypes.c_int
    lib.ar_reduce.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int, sz,
                              ctypes.c_int, ctypes.c_int, ctypes.c_uint, vp]
    lib.ar_reduce.restype = ctypes.c_int
    lib.ar_reduce_staged_static.argtypes = lib.ar_reduce.argtypes
    lib.ar_reduce_staged_static.restype = ctypes.c_int
    lib.ar_free.argtypes = [vp]
    lib.ar_free.restype = ctypes.c_int
    lib.ar_status_str.argtypes = [ctypes.c_int]
    lib.ar_status_str.restype = ctypes.c_char_p
    lib.ar_plan_query.argtypes = [ctypes.POINTER(ArConfig), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                  ctypes.c_int, sz, ctypes.c_int, ctypes.c_int, ctypes.c_uint,
                                  ctypes.c_int, ctypes.POINTER(ArPlan)]
    lib.ar_plan_query.restype = ctypes.c_int
    lib.ar_reduce_add.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int, sz,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_uint, vp, sz, vp]
    lib.ar_reduce_add.restype = ctypes.c_int
    lib.ar_plan_query_add.argtypes = [ctypes.POINTER(ArConfig), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                      ctypes.c_int, sz, ctypes.c_int, ctypes.c_int, ctypes.c_uint,
                                      vp, sz, ctypes.c_int, ctypes.POINTER(ArPlan)]
    lib.ar_plan_query_add.restype = ctypes.c_int
    lib.ar_reduce_rows.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int, ctypes.POINTER(ArRows),
                                   ctypes.c_int, ctypes.c_int, ctypes.c_uint, vp, vp]
    lib.ar_reduce_rows.restype = ctypes.c_int
    lib.ar_plan_query_rows.argtypes = [ctypes.POINTER(ArConfig), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                       ctypes.c_int, ctypes.POINTER(ArRows), ctypes.c_int, ctypes.c_int,
                                       ctypes.c_uint, vp, ctypes.c_int, ctypes.POINTER(ArPlan)]
    lib.ar_plan_query_rows.restype = ctypes.c_int
    _lib = lib
    return lib


def _addr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"expected a tensor or an integer address, got {type(x).__name__}")


def ptr_array(xs):
    """A C array of pointers (``void *[]``) for dsts / srcs; build it once and
    reuse it across calls on the same buffers."""
    if xs is None:
        return None
    if isinstance(xs, ctypes.Array):
        return xs
    vals = [_addr(x) for x in xs]
    return (ctypes.c_void_p * max(1, len(vals)))(*vals)


_ptr_array = ptr_array

_TYPE_BYTES = {AR_F32: 4, AR_F16: 2, AR_BF16: 2}


def _tensors(xs):
    """The tensor entries of a dsts / srcs argument (addresses, None and
    ready-made pointer arrays are not checkable)."""
    if xs is None or isinstance(xs, ctypes.Array):
        return ()
    return [x for x in xs if x is not None and not isinstance(x, int)]


def _check_flat(xs, need: int, what: str) -> None:
    """1-D calls: each tensor is contiguous and holds at least ``need`` bytes."""
    for x in _tensors(xs):
        if x.nbytes < need or not x.is_contiguous():
            raise ValueError(f"{what}: a tensor of {x.nbytes} bytes{'' if x.is_contiguous() else ' (not contiguous)'}"
                             f" where the call reads or writes {need} contiguous bytes")


def _check_span(xs, need: int, what: str) -> None:
    """Row-strided calls: each tensor's storage holds ``need`` bytes from its data pointer."""
    for x in _tensors(xs):
        have = x.untyped_storage().nbytes() - x.storage_offset() * x.element_size()
        if have < need:
            raise ValueError(f"{what}: {have} bytes from the tensor's data pointer where the call spans {need}")


def _check_counts(dsts, srcs, mode: int, R: int | None = None) -> None:
    """The library reads R source pointers and n_dst destination pointers (n_dst = R
    for AR_MODE_RS_BCAST, else 1) from the arrays it is given: refuse lists shorter
    than that before building them (ctypes arrays and raw addresses are passed
    through as given, as in C).  Counts outside 2..AR_MAX_RANKS are left to the
    library, which rejects them before reading any pointer."""
    R = (len(srcs) if srcs is not None and not isinstance(srcs, ctypes.Array) else None) if R is None else R
    if R is None or not 2 <= R <= AR_MAX_RANKS:
        return
    if srcs is not None and not isinstance(srcs, ctypes.Array) and len(srcs) < R:
        raise ValueError(f"srcs has {len(srcs)} entries for R = {R}")
    n_dst = R if (int(mode) & AR_MODE_MASK) == AR_MODE_RS_BCAST else 1
    if dsts is not None and not isinstance(dsts, ctypes.Array) and len(dsts) < n_dst:
        raise ValueError(f"dsts has {len(dsts)} entries; this mode writes {n_dst} destinations")


def _flat_arrays(dsts, srcs, n: int, dst_type: int, wire_type: int, mode: int, validate: bool):
    """ptr_array(dsts), ptr_array(srcs) of a 1-D call, checking each tensor on the
    way (one pass: the check costs little beyond the pointer conversion); returns
    the arrays and the element width of the destination type (0 when unchecked)."""
    _check_counts(dsts, srcs, mode)
    dst_b = src_b = 0
    if validate and n > 0:
        dst_b = _TYPE_BYTES.get(dst_type, 0)
        src_b = _TYPE_BYTES.get(wire_type if mode & AR_SRC_WIRE else dst_type, 0)
        if not dst_b or not src_b:              # the library rejects the call itself
            dst_b = src_b = 0
    return _checked_array(dsts, n * dst_b, "dsts"), _checked_array(srcs, n * src_b, "srcs"), dst_b


def _checked_array(xs, need: int, what: str):
    """ptr_array(xs); with ``need`` > 0 every tensor must be contiguous and hold that many bytes."""
    if xs is None or isinstance(xs, ctypes.Array):
        return xs
    vals = []
    for x in xs:
        if x is None or isinstance(x, int):
            vals.append(x)
            continue
        vals.append(_addr(x))
        if need and (x.nbytes < need or not x.is_contiguous()):
            _check_flat((x,), need, what)
    return (ctypes.c_void_p * max(1, len(vals)))(*vals)


def _validate_rows(dsts, srcs, rows: int, cols: int, src_stride: int, dst_stride: int, dst_type: int,
                   wire_type: int, mode: int, residual, res_stride: int) -> None:
    dst_b = _TYPE_BYTES.get(int(dst_type))
    src_b = _TYPE_BYTES.get(int(wire_type) if int(mode) & AR_SRC_WIRE else int(dst_type))
    if dst_b is None or src_b is None or int(rows) <= 0 or int(cols) <= 0:
        return

    def extent(stride):
        return ((int(rows) - 1) * int(stride) + int(cols)) if int(stride) > 0 else int(cols)
    _check_span(dsts, extent(dst_stride) * dst_b, "dsts")
    _check_span(srcs, extent(src_stride) * src_b, "srcs")
    if residual is not None:
        _check_span((residual,), extent(res_stride) * dst_b, "residual")


def _stream_handle(stream) -> int | None:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _config(config) -> ArConfig | None:
    if config is None:
        return None
    if isinstance(config, ArConfig):
        return config
    return ArConfig(**config)


def ar_status_str(status: int) -> str:
    return load_library().ar_status_str(int(status)).decode()


def ar_init(device: int = 0, config=None) -> ctypes.c_void_p:
    """Create a reduce context on HIP device ``device`` (raises ArError)."""
    lib = load_library()
    out = ctypes.c_void_p()
    cfg = _config(config)
    rc = lib.ar_init(ctypes.byref(out), int(device), ctypes.byref(cfg) if cfg is not None else None)
    if rc != AR_OK:
        raise ArError(rc, "ar_init")
    return out


def ar_reduce(ctx, dsts, srcs, n: int, dst_type: int = AR_F32, wire_type: int = AR_BF16,
              mode: int = AR_MODE_AUTO, stream=None, check: bool = True, validate: bool = True) -> int:
    """Enqueue one reduce; returns the status (raises ArError on failure if
    ``check``; ValueError before the call if ``validate`` finds a tensor too small)."""
    lib = load_library()
    n, dst_type, wire_type, mode = int(n), int(dst_type), int(wire_type), int(mode)
    dst_arr, src_arr, _ = _flat_arrays(dsts, srcs, n, dst_type, wire_type, mode, validate)
    R = len(srcs) if srcs is not None else 0
    rc = lib.ar_reduce(ctx, dst_arr, src_arr, R, n, dst_type, wire_type, mode, _stream_handle(stream))
    if check and rc != AR_OK:
        raise ArError(rc, "ar_reduce")
    return rc


def ar_reduce_staged_static(ctx, dsts, srcs, n: int, dst_type: int = AR_F32, wire_type: int = AR_BF16,
                            mode: int = AR_MODE_HOST_STAGED, stream=None, check: bool = True,
                            validate: bool = True) -> int:
    """The host-staged reduce with its staging ring in the library's static device
    array (no device allocation); arguments and checks as ar_reduce."""
    lib = load_library()
    n, dst_type, wire_type, mode = int(n), int(dst_type), int(wire_type), int(mode)
    dst_arr, src_arr, _ = _flat_arrays(dsts, srcs, n, dst_type, wire_type, mode, validate)
    R = len(srcs) if srcs is not None else 0
    rc = lib.ar_reduce_staged_static(ctx, dst_arr, src_arr, R, n, dst_type, wire_type, mode, _stream_handle(stream))
    if check and rc != AR_OK:
        raise ArError(rc, "ar_reduce_staged_static")
    return rc


def bind_reduce(ctx, dsts, srcs, n: int, dst_type: int = AR_F32, wire_type: int = AR_BF16,
                mode: int = AR_MODE_AUTO, stream=None, residual=None, residual_len: int | None = None):
    """One reduce with every argument converted to its C type once: returns a
    callable that enqueues the call again each time it is invoked and returns
    the status (no Python-side checks per call; the library still validates
    every call).  For latency-bound callers that issue the same call shape on
    the same buffers many times.  With ``residual`` it binds ``ar_reduce_add``.
    The caller keeps the context and the bound buffers alive while the callable is in use."""
    import functools

    lib = load_library()
    R = len(srcs)
    ctx_val = ctx.value if isinstance(ctx, ctypes.c_void_p) else ctx
    st_val = _stream_handle(stream)
    rlen = int(n) if residual_len is None else int(residual_len)
    if residual is not None and residual_len is None and hasattr(residual, "numel"):
        rlen = int(residual.numel())
    dst_arr, src_arr, dst_b = _flat_arrays(dsts, srcs, int(n), int(dst_type), int(wire_type), int(mode), True)
    if residual is not None and dst_b:
        _check_flat((residual,), rlen * dst_b, "residual")
    fast = _fast_module()
    if fast is not None:
        fn = lib.ar_reduce if residual is None else lib.ar_reduce_add
        return fast.bind(ctypes.cast(fn, ctypes.c_void_p).value, residual is not None, ctx_val or 0,
                         ctypes.addressof(dst_arr), ctypes.addressof(src_arr), R, int(n), int(dst_type),
                         int(wire_type), int(mode), _addr(residual) or 0, rlen, st_val or 0,
                         (dst_arr, src_arr))
    head = (ctypes.c_void_p(ctx_val), dst_arr, src_arr, ctypes.c_int(R), ctypes.c_size_t(int(n)),
            ctypes.c_int(int(dst_type)), ctypes.c_int(int(wire_type)), ctypes.c_uint(int(mode)))
    st = ctypes.c_void_p(st_val)
    if residual is None:
        return functools.partial(lib.ar_reduce, *head, st)
    return functools.partial(lib.ar_reduce_add, *head, ctypes.c_void_p(_addr(residual)), ctypes.c_size_t(rlen), st)


_fast = None


def _fast_module():
    """The compiled fast-call type (csrc/ar_pycall.c), or None when it was not built."""
    global _fast
    if _fast is None:
        try:
            from . import _ar_fast
            _fast = _ar_fast
        except ImportError:
            _fast = False
    return _fast or None


def ar_reduce_add(ctx, dsts, srcs, n: int, dst_type: int, wire_type: int, mode: int, residual,
                  residual_len: int | None = None, stream=None, check: bool = True,
                  validate: bool = True) -> int:
    """Enqueue one reduce followed by a residual add (element-wise when
    ``residual_len == n``, else one broadcast row); ``residual_len`` defaults to
    the residual tensor's element count.  Returns the status (raises ArError on
    failure if ``check``; ValueError before the call if ``validate`` finds a tensor too small)."""
    lib = load_library()
    R = len(srcs) if srcs is not None else 0
    if residual_len is None:
        if not hasattr(residual, "numel"):
            raise TypeError("residual_len is required when the residual is given as an address")
        residual_len = residual.numel()
    dst_arr, src_arr, dst_b = _flat_arrays(dsts, srcs, int(n), int(dst_type), int(wire_type), int(mode), validate)
    if dst_b:
        _check_flat((residual,), int(residual_len) * dst_b, "residual")
    rc = lib.ar_reduce_add(ctx, dst_arr, src_arr, R, int(n), int(dst_type),
                           int(wire_type), int(mode), _addr(residual), int(residual_len),
                           _stream_handle(stream))
    if check and rc != AR_OK:
        raise ArError(rc, "ar_reduce_add")
    return rc


def ar_reduce_rows(ctx, dsts, srcs, rows: int, cols: int, src_stride: int, dst_stride: int, dst_type: int,
                   wire_type: int, mode: int, residual=None, res_stride: int = 0, stream=None,
                   check: bool = True, validate: bool = True) -> int:
    """Enqueue one reduce of row-strided tensors (strides in elements); ``residual``
    None, or a tensor / address laid out with row stride ``res_stride`` (0 = one row
    added to every row).  Returns the status (raises ArError on failure if ``check``;
    ValueError before the call if ``validate`` finds a tensor's storage too small)."""
    lib = load_library()
    R = len(srcs) if srcs is not None else 0
    _check_counts(dsts, srcs, mode)
    if validate:
        _validate_rows(dsts, srcs, rows, cols, src_stride, dst_stride, dst_type, wire_type, mode, residual,
                       res_stride)
    shape = ArRows(int(rows), int(cols), int(src_stride), int(dst_stride), int(res_stride))
    rc = lib.ar_reduce_rows(ctx, _ptr_array(dsts), _ptr_array(srcs), R, ctypes.byref(shape), int(dst_type),
                            int(wire_type), int(mode), _addr(residual), _stream_handle(stream))
    if check and rc != AR_OK:
        raise ArError(rc, "ar_reduce_rows")
    return rc


def bind_reduce_rows(ctx, dsts, srcs, rows: int, cols: int, src_stride: int, dst_stride: int, dst_type: int,
                     wire_type: int, mode: int, residual=None, res_stride: int = 0, stream=None):
    """ar_reduce_rows with every argument converted to its C type once (the tensors'
    spans checked once, as ar_reduce_rows checks them): returns a callable that
    enqueues the call again each time it is invoked and returns the status (the
    library still validates every call).  The caller keeps the context and the
    bound buffers alive while the callable is in use."""
    import functools

    lib = load_library()
    R = len(srcs) if srcs is not None else 0
    _check_counts(dsts, srcs, mode)
    _validate_rows(dsts, srcs, rows, cols, src_stride, dst_stride, dst_type, wire_type, mode, residual, res_stride)
    shape = ctypes.pointer(ArRows(int(rows), int(cols), int(src_stride), int(dst_stride), int(res_stride)))
    ctx_val = ctx.value if isinstance(ctx, ctypes.c_void_p) else ctx
    return functools.partial(lib.ar_reduce_rows, ctypes.c_void_p(ctx_val), _ptr_array(dsts), _ptr_array(srcs),
                             ctypes.c_int(R), shape, ctypes.c_int(int(dst_type)), ctypes.c_int(int(wire_type)),
                             ctypes.c_uint(int(mode)), ctypes.c_void_p(_addr(residual)),
                             ctypes.c_void_p(_stream_handle(stream)))


def ar_free(ctx) -> None:
    rc = load_library().ar_free(ctx)
    if rc != AR_OK:
        raise ArError(rc, "ar_free")


def ar_plan_query(dsts, srcs, n: int, dst_type: int = AR_F32, wire_type: int = AR_BF16,
                  mode: int = AR_MODE_AUTO, srcs_on_host: bool = False, config=None,
                  R: int | None = None):
    """Host-only validation + plan; returns (status, ArPlan)."""
    lib = load_library()
    plan = ArPlan()
    cfg = _config(config)
    R = (len(srcs) if srcs is not None else 0) if R is None else R
    _check_counts(dsts, srcs, mode, R)
    rc = lib.ar_plan_query(ctypes.byref(cfg) if cfg is not None else None, _ptr_array(dsts),
                           _ptr_array(srcs), R, int(n), int(dst_type), int(wire_type), int(mode),
                           int(bool(srcs_on_host)), ctypes.byref(plan))
    return rc, plan


def ar_plan_query_add(dsts, srcs, n: int, dst_type: int, wire_type: int, mode: int, residual,
                      residual_len: int, srcs_on_host: bool = False, config=None, R: int | None = None):
    """Host-only validation + plan of ar_reduce_add; returns (status, ArPlan)."""
    lib = load_library()
    plan = ArPlan()
    cfg = _config(config)
    R = (len(srcs) if srcs is not None else 0) if R is None else R
    _check_counts(dsts, srcs, mode, R)
    rc = lib.ar_plan_query_add(ctypes.byref(cfg) if cfg is not None else None, _ptr_array(dsts),
                               _ptr_array(srcs), R, int(n), int(dst_type), int(wire_type), int(mode),
                               _addr(residual), int(residual_len), int(bool(srcs_on_host)),
                               ctypes.byref(plan))
    return rc, plan


def ar_plan_query_rows(dsts, srcs, rows: int, cols: int, src_stride: int, dst_stride: int, dst_type: int,
                       wire_type: int, mode: int, residual=None, res_stride: int = 0, srcs_on_host: bool = False,
                       config=None, R: int | None = None):
    """Host-only validation + plan of ar_reduce_rows; returns (status, ArPlan)."""
    lib = load_library()
    plan = ArPlan()
    cfg = _config(config)
    R = (len(srcs) if srcs is not None else 0) if R is None else R
    _check_counts(dsts, srcs, mode, R)
    shape = ArRows(int(rows), int(cols), int(src_stride), int(dst_stride), int(res_stride))
    rc = lib.ar_plan_query_rows(ctypes.byref(cfg) if cfg is not None else None, _ptr_array(dsts),
                                _ptr_array(srcs), R, ctypes.byref(shape), int(dst_type), int(wire_type),
                                int(mode), _addr(residual), int(bool(srcs_on_host)), ctypes.byref(plan))
    return rc, plan


class Reducer:
    """Owns one context; ``reducer(dsts, srcs, ...)`` enqueues a reduce."""

    def __init__(self, device: int = 0, config=None):
        self.ctx = ar_init(device, config)

    def __call__(self, dsts, srcs, n=None, dst_type=AR_F32, wire_type=AR_BF16,
                 mode=AR_MODE_AUTO, stream=None):
        if n is None:
            first = next((s for s in srcs if s is not None), None)
            if first is None:
                raise ValueError("n is required when every source is inactive")
            n = first.numel()
        return ar_reduce(self.ctx, dsts, srcs, n, dst_type, wire_type, mode, stream)

    def close(self):
        if self.ctx is not None:
            ar_free(self.ctx)
            self.ctx = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
