"""The benchmark's ceiling kernels (libmpp_ceiling.so) move every byte they are
timed on.

bench.py compares the reduce with these kernels at the same bytes and access
pattern, so a ceiling kernel that skipped a tile or a stream would overstate
the achievable rate.  The GPU test checks, for every pattern, store policy,
workgroup size, placement and occupancy hold, that every destination receives
at every 32-bit word the wrapping sum of the sources' words (the kernel's only
arithmetic), over a tile count that is not a multiple of the workgroups or of
the placement runs and that fills every CU beyond the hold.  The CPU test checks the launcher's argument validation, which
runs before any HIP call.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import bench

PATTERNS = [(1, 1), (2, 1), (3, 1), (4, 4), (8, 1)]
TILE = 2048


def _arrays(srcs, dsts):
    vp = ctypes.c_void_p
    return (vp * len(srcs))(*srcs), (vp * len(dsts))(*dsts)


def test_launcher_refuses_invalid_requests_before_any_gpu_call():
    lib = bench.ceiling_lib()
    a = [0x10_0000_0000 + i * 0x1_0000_0000 for i in range(12)]   # 16-byte aligned, never dereferenced
    s8, d4 = _arrays(a[:8], a[8:12])
    bad = [
        (3, 2, 0, 256, 4 * TILE, 0, 0),         # no such pattern
        (2, 2, 0, 256, 4 * TILE, 0, 0),
        (2, 1, 3, 256, 4 * TILE, 0, 0),         # store policy
        (2, 1, 0, 128, 4 * TILE, 0, 0),         # workgroup size
        (2, 1, 0, 64, 0, 0, 0),                 # empty
        (2, 1, 0, 64, 4 * TILE + 16, 0, 0),     # not whole tiles
        (2, 1, 0, 64, 4 * TILE, 0, -1),         # occupancy hold
        (2, 1, 0, 64, 4 * TILE, 0, 65),
    ]
    for R, D, sp, block, nbytes, run, hold in bad:
        assert lib.mpp_ceiling_launch(R, D, sp, block, s8, d4, nbytes, run, hold, None) == 1, (R, D, sp, block,
                                                                                              nbytes, hold)
    s_mis, d_ok = _arrays([a[0] + 8, a[1]], a[8:9])
    assert lib.mpp_ceiling_launch(2, 1, 0, 64, s_mis, d_ok, 4 * TILE, 0, 0, None) == 1
    s_null, _ = _arrays([a[0], 0], a[8:9])
    assert lib.mpp_ceiling_launch(2, 1, 0, 64, s_null, d_ok, 4 * TILE, 0, 0, None) == 1


@pytest.mark.gpu
def test_every_pattern_writes_the_word_sum_to_every_destination():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lib = bench.ceiling_lib()
    # several placement runs of 512 KiB, a ragged end, and more one-wave workgroups
    # than 256 CUs hold at 14 waves each (below that the hold is not applied)
    tiles = 16 * 256 + 37
    nbytes = tiles * TILE
    words = nbytes // 4
    rng = np.random.default_rng(20251)
    host = [rng.integers(0, 2**32, size=words, dtype=np.uint32) for _ in range(8)]
    dev = [torch.from_numpy(h.view(np.int32)).cuda() for h in host]
    stream = torch.cuda.current_stream()
    sentinel = np.int32(-0x5A5A5A5B)
    for R, D in PATTERNS:
        want = host[0].copy()
        for r in range(1, R):
            want += host[r]                     # uint32: wraps like the kernel's integer add
        for sp in (0, 1, 2):
            for block in (256, 64):
                for run, hold in ((0, 0), (512 << 10, 0), (512 << 10, 14)):
                    dsts = [torch.full((words,), int(sentinel), dtype=torch.int32, device="cuda") for _ in range(D)]
                    s, d = _arrays([t.data_ptr() for t in dev[:R]], [t.data_ptr() for t in dsts])
                    rc = lib.mpp_ceiling_launch(R, D, sp, block, s, d, nbytes, run, hold,
                                                ctypes.c_void_p(stream.cuda_stream))
                    assert rc == 0, (R, D, sp, block, run, hold)
                    torch.cuda.synchronize()
                    for q, t in enumerate(dsts):
                        got = t.cpu().numpy().view(np.uint32)
                        bad = np.flatnonzero(got != want)
                        assert bad.size == 0, (f"pattern {R}:{D} store {sp} block {block} run {run} hold {hold} "
                                               f"dst {q}: {bad.size} words differ, first at byte "
                                               f"{4 * int(bad[0])}")
