"""Helpers for the GPU parity tests: device buffers from numpy, bit comparison
with the oracle, guard-banded destinations and case logging that survives a
crashed process (written straight to the real stderr, flushed)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

SENTINEL = np.uint32(0x7FA5A5A5)   # a NaN payload no input of these tests produces
SENTINEL16 = np.uint16(0x7FA5)     # a NaN in both binary16 and bfloat16
GUARD = 64                           # elements of guard band on each side (256 B)


def log_case(msg: str) -> None:
    print(f"[case] {msg}", file=sys.__stderr__, flush=True)


def to_device(a: np.ndarray) -> torch.Tensor:
    """float32 or uint16 numpy array -> contiguous device tensor with the same bytes."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_pinned(a: np.ndarray) -> torch.Tensor:
    """numpy array -> pinned host tensor (hipHostMalloc'd by torch) with the same bytes."""
    if a.dtype == np.uint16:
        src = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    else:
        src = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = torch.empty(src.shape, dtype=src.dtype, pin_memory=True)
    t.copy_(src)
    return t


class GuardedDst:
    """A destination of n elements (float32, or 16-bit with ``bits=16``) with
    sentinel-filled guard bands."""

    def __init__(self, n: int, bits: int = 32):
        self.n = n
        self.bits = bits
        if bits == 32:
            host = np.full(n + 2 * GUARD, SENTINEL, dtype=np.uint32)
            self.buf = torch.from_numpy(host.view(np.int32)).cuda()
        else:
            host = np.full(n + 2 * GUARD, SENTINEL16, dtype=np.uint16)
            self.buf = torch.from_numpy(host.view(np.int16)).cuda()
        self.view = self.buf[GUARD:GUARD + n]

    def ptr(self) -> int:
        return self.view.data_ptr()

    def result(self) -> np.ndarray:
        """Interior (float32, or uint16 bit patterns) after checking both guard bands."""
        if self.bits == 32:
            host = self.buf.cpu().numpy().view(np.uint32)
            sentinel = SENTINEL
        else:
            host = self.buf.cpu().numpy().view(np.uint16)
            sentinel = SENTINEL16
        assert np.all(host[:GUARD] == sentinel), "write below the destination"
        assert np.all(host[GUARD + self.n:] == sentinel), "write past the destination"
        inner = host[GUARD:GUARD + self.n]
        return inner.view(np.float32) if self.bits == 32 else inner.copy()


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str) -> None:
    """0-ulp comparison; NaNs compared only as 'is a NaN' (payload not part of the contract)."""
    got = np.ascontiguousarray(got, dtype=np.float32).ravel()
    want = np.ascontiguousarray(want, dtype=np.float32).ravel()
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    gn, wn = np.isnan(got), np.isnan(want)
    if not np.array_equal(gn, wn):
        i = int(np.flatnonzero(gn != wn)[0])
        raise AssertionError(f"{what}: NaN mismatch at {i}: got {got[i]!r} want {want[i]!r}")
    gb, wb = got.view(np.uint32), want.view(np.uint32)
    bad = (gb != wb) & ~gn
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements differ; first at {i}: "
                             f"got {int(gb[i]):#010x} want {int(wb[i]):#010x}")


def is_nan16(h: np.ndarray, wire: int) -> np.ndarray:
    h = h.astype(np.uint32)
    if wire == oracle.BF16:
        return ((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)
    return ((h & 0x7C00) == 0x7C00) & ((h & 0x03FF) != 0)


def assert_bits_equal16(got: np.ndarray, want: np.ndarray, wire: int, what: str) -> None:
    """0-ulp comparison of 16-bit patterns; NaNs compared only as 'is a NaN'."""
    got = np.ascontiguousarray(got, dtype=np.uint16).ravel()
    want = np.ascontiguousarray(want, dtype=np.uint16).ravel()
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    gn, wn = is_nan16(got, wire), is_nan16(want, wire)
    if not np.array_equal(gn, wn):
        i = int(np.flatnonzero(gn != wn)[0])
        raise AssertionError(f"{what}: NaN mismatch at {i}: got {int(got[i]):#06x} want {int(want[i]):#06x}")
    bad = (got != want) & ~gn
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements differ; first at {i}: "
                             f"got {int(got[i]):#06x} want {int(want[i]):#06x}")


def assert_no_sentinel(got: np.ndarray, what: str) -> None:
    left = got.view(np.uint32) == SENTINEL
    assert not left.any(), f"{what}: {int(left.sum())} elements never written"


def oracle_result(srcs, wire, src_type=None) -> np.ndarray:
    return oracle.reduce(srcs, wire, n_dst=1, src_type=src_type)[0]
