"""CPU oracle for the mixed-precision partial-sum reduce.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It is a plain,
slow, scalar C implementation (``ar_oracle.c``) driven through ctypes; it shares
no code with the HIP library in ``mixed_precision_partial_amd`` and the library
never imports it.

Every function here follows the passages cited in ``ar_oracle.c``:

* the per-rank cast to the wire type and the receiver-side rounding of its own
  partial ("CUDA allreduce.cu" page, "Chunked kernel AllReduce" comment block,
  phases 1 and 3, and the "Combined load-convert-add kernel" comment);
* the fixed rank order of the sum and the write to every destination
  ("Hexagon allreduce-ops.c" page, allreduce_thread_dma_1d and op_allreduce);
* the residual added after the ranks, element-wise or as one broadcast row
  (same page, the HAS_ADD and IS_ROW_BCAST forms of the 1-D / 2-D loops);
* narrow destinations that accumulate in their own type (CUDA page, the
  half / nv_bfloat16 instances of the chunked kernel; Hexagon page, the f16
  instances);
* row-strided tensors and the residual row added to every row (Hexagon
  page, allreduce_thread_dma_2d and its IS_ROW_BCAST form).

Parity status: every function below is pinned by ``tests/test_oracle_pins.py``
(exhaustive conversions against torch / numpy, a double-rounding theorem for
the additions, closed forms, hand-worked examples in ``tests/golden/``, brute
force on tiny inputs and planted-mistake checks).  None is "parity unpinned";
the pages' own rounding mode is the one reading that no page fixes (see the
header of ``ar_oracle.c``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, F16, BF16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ar_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle_ar.so")

# The flags are part of the oracle's definition: no fast-math, no contraction.
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fno-semantic-interposition",
          "-fPIC", "-shared", "-std=c11"]


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc.  Returns the path of the shared object."""
    cmd = ["gcc", *CFLAGS, src, "-o", out]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.orc_round_bf16.argtypes = [ctypes.c_uint32]
    lib.orc_round_bf16.restype = ctypes.c_uint16
    lib.orc_round_f16.argtypes = [ctypes.c_uint32]
    lib.orc_round_f16.restype = ctypes.c_uint16
    lib.orc_widen_bf16.argtypes = [ctypes.c_uint16]
    lib.orc_widen_bf16.restype = ctypes.c_uint32
    lib.orc_widen_f16.argtypes = [ctypes.c_uint16]
    lib.orc_widen_f16.restype = ctypes.c_uint32
    for name in ("orc_round_bf16_array", "orc_round_f16_array",
                 "orc_widen_bf16_array", "orc_widen_f16_array"):
        getattr(lib, name).argtypes = [vp, vp, sz]
        getattr(lib, name).restype = None
    lib.orc_add_f32_array.argtypes = [vp, vp, vp, sz]
    lib.orc_add_f32_array.restype = None
    lib.orc_reduce.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.POINTER(vp),
                               ctypes.c_int, sz, ctypes.c_int, ctypes.c_int]
    lib.orc_reduce.restype = ctypes.c_int
    lib.orc_reduce_ex.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp),
                                  ctypes.c_int, sz, ctypes.c_int, ctypes.c_int, vp, sz]
    lib.orc_reduce_ex.restype = ctypes.c_int
    lib.orc_reduce_rows.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp),
                                    ctypes.c_int, sz, sz, sz, sz, ctypes.c_int, ctypes.c_int, vp, sz]
    lib.orc_reduce_rows.restype = ctypes.c_int
    return lib


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (building first if absent) the oracle shared object."""
    global _lib
    if path == LIB_PATH and _lib is not None:
        return _lib
    if not os.path.exists(path):
        if path != LIB_PATH:
            raise FileNotFoundError(path)
        build()
    lib = _bind(ctypes.CDLL(path))
    if path == LIB_PATH:
        _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# --- scalar and array conversions -----------------------------------------

def round_bf16_bits(x_bits: np.ndarray, lib=None) -> np.ndarray:
    """binary32 bit patterns -> bfloat16 bit patterns (RNE)."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.orc_round_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def round_f16_bits(x_bits: np.ndarray, lib=None) -> np.ndarray:
    """binary32 bit patterns -> binary16 bit patterns (RNE)."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.orc_round_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def widen_bf16_bits(h_bits: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    h = np.ascontiguousarray(h_bits, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.uint32)
    lib.orc_widen_bf16_array(_ptr(h), _ptr(out), h.size)
    return out


def widen_f16_bits(h_bits: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    h = np.ascontiguousarray(h_bits, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.uint32)
    lib.orc_widen_f16_array(_ptr(h), _ptr(out), h.size)
    return out


def add_f32(a: np.ndarray, b: np.ndarray, lib=None) -> np.ndarray:
    """Element-wise binary32 addition as the oracle performs it."""
    lib = lib or load()
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.float32)
    lib.orc_add_f32_array(_ptr(a), _ptr(b), _ptr(out), a.size)
    return out


# --- the reduce ------------------------------------------------------------

def reduce(srcs, wire_type: int, n_dst: int = 1, src_type: int | None = None,
           lib=None, dst_type: int = F32, residual=None, n: int | None = None) -> np.ndarray:
    """Reference result of the partial-sum reduce.

    ``srcs``: sequence of R equally sized 1-D arrays.  float32 arrays are the
    caller-typed partials; uint16 arrays hold wire-typed bit patterns (then
    ``src_type`` must equal ``wire_type``).  A ``None`` entry is an inactive
    rank (its partial is all +0.0).
    ``dst_type``: F32, or F16 / BF16 (then wire and sources have that type).
    ``residual``: None, or a 1-D array of the destination type (float32, or
    uint16 bit patterns for a narrow destination) whose length is n (added
    element-wise) or divides n (one row added to every row).
    ``n``: the element count; needed only when every rank is inactive (the
    sources then carry no length), else it must match them.
    Returns an ``(n_dst, n)`` array of the destination type (float32, or
    uint16 bit patterns); every row holds the same bits.
    """
    lib = lib or load()
    srcs = [None if s is None else np.ascontiguousarray(s) for s in srcs]
    R = len(srcs)
    live = [s for s in srcs if s is not None]
    if not live and n is None:
        raise ValueError("every rank is inactive: pass n")
    if live and n is not None and int(n) != live[0].size:
        raise ValueError("n differs from the sources' length")
    n = int(n) if n is not None else live[0].size
    if src_type is None:
        src_type = wire_type if live and live[0].dtype == np.uint16 else F32
    want = np.float32 if src_type == F32 else np.uint16
    for s in live:
        if s.size != n:
            raise ValueError("sources differ in length")
        if s.dtype != want:
            raise TypeError(f"source dtype {s.dtype} does not match src_type {src_type}")
    out_dtype = np.float32 if dst_type == F32 else np.uint16
    res_ptr, res_len = None, 0
    if residual is not None:
        residual = np.ascontiguousarray(residual)
        if residual.dtype != out_dtype:
            raise TypeError(f"residual dtype {residual.dtype} does not match dst_type {dst_type}")
        res_ptr, res_len = residual.ctypes.data, residual.size
    out = np.empty((n_dst, n), dtype=out_dtype)
    dst_ptrs = (ctypes.c_void_p * n_dst)(*[out[d].ctypes.data for d in range(n_dst)])
    src_ptrs = (ctypes.c_void_p * R)(*[None if s is None else s.ctypes.data for s in srcs])
    rc = lib.orc_reduce_ex(dst_ptrs, n_dst, dst_type, src_ptrs, R, n, src_type, wire_type, res_ptr, res_len)
    if rc != 0:
        raise ValueError(f"oracle rejected arguments (rc={rc})")
    return out


def reduce_rows(srcs, wire_type: int, rows: int, cols: int, src_stride: int, dst_stride: int,
                n_dst: int = 1, src_type: int | None = None, dst_type: int = F32, residual=None,
                res_stride: int = 0, dst_init=None, lib=None) -> np.ndarray:
    """Reference result of the reduce over row-strided tensors.

    ``srcs``: R flat arrays holding ``rows`` rows of ``cols`` elements at row stride
    ``src_stride`` (float32, or uint16 patterns of the wire type; None = inactive).
    Destinations are flat arrays of ``(rows - 1) * dst_stride + cols`` elements, copied
    from ``dst_init`` (default: zeros) so the bytes between rows are whatever the
    caller had there.  ``residual``: None, or a flat array of the destination type
    with row stride ``res_stride`` (0 = one row added to every row).
    Returns an ``(n_dst, extent)`` array of the destination type.
    """
    lib = lib or load()
    srcs = [None if s is None else np.ascontiguousarray(s) for s in srcs]
    R = len(srcs)
    live = [s for s in srcs if s is not None]
    if not live:
        raise ValueError("at least one active source is needed")
    if src_type is None:
        src_type = F32 if live[0].dtype == np.float32 else wire_type
    want = np.float32 if src_type == F32 else np.uint16
    need = 0 if rows == 0 else (rows - 1) * src_stride + cols
    for s in live:
        if s.dtype != want or s.size < need:
            raise ValueError("source too short or of the wrong type")
    out_dtype = np.float32 if dst_type == F32 else np.uint16
    extent = 0 if rows == 0 else (rows - 1) * dst_stride + cols
    out = np.zeros((n_dst, extent), dtype=out_dtype)
    if dst_init is not None:
        out[:] = np.asarray(dst_init, dtype=out_dtype)[:extent]
    res_ptr = None
    if residual is not None:
        residual = np.ascontiguousarray(residual)
        if residual.dtype != out_dtype:
            raise TypeError("residual type does not match the destination type")
        res_need = 0 if rows == 0 else (cols if res_stride == 0 else (rows - 1) * res_stride + cols)
        if residual.size < res_need:
            raise ValueError("residual too short")
        res_ptr = residual.ctypes.data
    dst_ptrs = (ctypes.c_void_p * n_dst)(*[out[d].ctypes.data for d in range(n_dst)])
    src_ptrs = (ctypes.c_void_p * R)(*[None if s is None else s.ctypes.data for s in srcs])
    rc = lib.orc_reduce_rows(dst_ptrs, n_dst, dst_type, src_ptrs, R, rows, cols, src_stride, dst_stride,
                             src_type, wire_type, res_ptr, res_stride)
    if rc != 0:
        raise ValueError(f"oracle rejected arguments (rc={rc})")
    return out
