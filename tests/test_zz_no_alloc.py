"""ar_reduce_staged_static (the host-staged reduce staged in the library's static
device array, for callers that cannot allocate) against ar_reduce's own
copy-engine path, bit for bit, on two calls in a row -- the second smaller --
and against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixed_precision_partial_amd as ar
import oracle
import workloads as wl
from gpu_util import GuardedDst, assert_bits_equal, log_case, to_pinned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    # host_path 1: ar_reduce itself takes the copy-engine pipeline (its hipMalloc'd ring)
    c = ar.ar_init(0, {"host_path": 1})
    yield c
    torch.cuda.synchronize()
    ar.ar_free(c)


# (R, n, wire, sources already in the wire type): the first call needs several
# chunks through the static array (one slot of 8 fp32 rank chunks in 64 MiB, so
# each chunk waits for the previous chunk's add); the second is smaller, with
# 16-bit sources
CALLS = [(8, 6_000_037, ar.AR_BF16, False), (3, 40_009, ar.AR_F16, True)]


def test_static_staging_matches_copy_engine_path(ctx):
    for k, (R, n, wire, src_wire) in enumerate(CALLS):
        log_case(f"static staging call {k}: R={R} n={n} wire={wire} src_wire={src_wire}")
        srcs = wl.random_partials(90_000 + k, 0, R, n, dist="normal+outliers")
        if src_wire:
            srcs = [wl.as_wire_typed(s, wire) for s in srcs]
        pinned = [to_pinned(s) for s in srcs]
        mode = ar.AR_MODE_HOST_STAGED | (ar.AR_SRC_WIRE if src_wire else 0)
        ref, new = GuardedDst(n), GuardedDst(n)
        ar.ar_reduce(ctx, [ref.ptr()], pinned, n, ar.AR_F32, wire, mode)
        ar.ar_reduce_staged_static(ctx, [new.ptr()], pinned, n, ar.AR_F32, wire, mode)
        torch.cuda.synchronize()
        got_ref, got_new = ref.result(), new.result()
        assert_bits_equal(got_new, got_ref, f"static staging call {k} vs ar_reduce")
        want = oracle.reduce(srcs, wire, src_type=wire if src_wire else None)[0]
        assert_bits_equal(got_new, want, f"static staging call {k} vs oracle")


def test_static_staging_refusals(ctx):
    n = 1 << 16
    srcs = [torch.randn(n, device="cuda") for _ in range(2)]
    out = torch.empty(n, device="cuda")
    # device sources resolve to a device schedule: not this entry point's
    assert ar.ar_reduce_staged_static(ctx, [out], srcs, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_AUTO,
                                      check=False) == ar.AR_ERR_INVALID
    pinned = [to_pinned(s.cpu().numpy()) for s in srcs]
    assert ar.ar_reduce_staged_static(ctx, [out], pinned, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                                      check=False) == ar.AR_ERR_INVALID
    # a configured copy chunk whose rank chunks (2 ranks x 64 MiB) exceed the array
    big = ar.ar_init(0, {"host_chunk_bytes": 64 << 20})
    try:
        n2 = 1 << 20
        pin2 = [torch.empty(n2, dtype=torch.float32, pin_memory=True) for _ in range(2)]
        out2 = torch.empty(n2, device="cuda")
        assert ar.ar_reduce_staged_static(big, [out2], pin2, n2, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_HOST_STAGED,
                                          check=False) == ar.AR_ERR_NOMEM
    finally:
        torch.cuda.synchronize()
        ar.ar_free(big)
    # n = 0 is a no-op
    assert ar.ar_reduce_staged_static(ctx, [out], pinned, 0, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_HOST_STAGED,
                                      check=False) == ar.AR_OK
    torch.cuda.synchronize()
