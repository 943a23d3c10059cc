"""Helpers for the GPU parity tests: device buffers from numpy, bit comparison
with the oracle, guard-banded destinations and case logging that survives a
crashed process (written straight to the real stderr, flushed)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

SENTINEL = np.uint32(0x7FA5A5A5)   # a NaN payload no input of these tests produces
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
    """A float32 destination of n elements with sentinel-filled guard bands."""

    def __init__(self, n: int):
        self.n = n
        host = np.full(n + 2 * GUARD, SENTINEL, dtype=np.uint32)
        self.buf = torch.from_numpy(host.view(np.int32)).cuda()
        self.view = self.buf[GUARD:GUARD + n]

    def ptr(self) -> int:
        return self.view.data_ptr()

    def result(self) -> np.ndarray:
        """Interior as float32 after checking both guard bands are untouched."""
        host = self.buf.cpu().numpy().view(np.uint32)
        assert np.all(host[:GUARD] == SENTINEL), "write below the destination"
        assert np.all(host[GUARD + self.n:] == SENTINEL), "write past the destination"
        return host[GUARD:GUARD + self.n].view(np.float32)


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


def assert_no_sentinel(got: np.ndarray, what: str) -> None:
    left = got.view(np.uint32) == SENTINEL
    assert not left.any(), f"{what}: {int(left.sum())} elements never written"


def oracle_result(srcs, wire, src_type=None) -> np.ndarray:
    return oracle.reduce(srcs, wire, n_dst=1, src_type=src_type)[0]
