"""The occupancy hold (ar_config.occupancy_hold) changes where waves run, never
what they compute: calls large enough for every hold to apply (the grid fills
each CU beyond it) give bit-identical outputs with no hold, the automatic hold
and explicit holds, on the two-rank kernels (plain, element-wise residual,
broadcast row, row-strided, 16-bit), the kernel for a few active partials, the
register-staged and the LDS-staged
kernels (contiguous and broadcast schedules, 16-bit layouts), and the automatic
one matches the oracle.  Each call's plan is checked to name the kernel family
the case is about.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixed_precision_partial_amd as ar
import oracle
import workloads as wl
from gpu_util import assert_bits_equal, assert_bits_equal16, log_case, to_device

pytestmark = pytest.mark.gpu

HOLDS = [0, -1, 6, 12, 18, 32]
N = (1 << 22) + 1000           # 8194 two-rank workgroups: beyond 256 CUs x 32 waves; a ragged tail


def _contexts(extra):
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return {h: ar.ar_init(0, {**extra, "occupancy_hold": h} if h or extra else None) for h in HOLDS}


def _free(made):
    torch.cuda.synchronize()
    for c in made.values():
        ar.ar_free(c)


@pytest.fixture(scope="module")
def ctxs():
    made = _contexts({})
    yield made
    _free(made)


@pytest.fixture(scope="module")
def lds_ctxs():
    """The same holds with the LDS-staged family forced (stream_kernel 2)."""
    made = _contexts({"stream_kernel": 2})
    yield made
    _free(made)


def planned_kernel(dsts, srcs, n, dst_type, wire, mode, config=None):
    rc, plan = ar.ar_plan_query(dsts, srcs, n, dst_type, wire, mode, config=config)
    assert rc == ar.AR_OK, ar.ar_status_str(rc)
    return int(plan.stream_kernel)


def same_everywhere(ctxs, what, run, out):
    """run(ctx) enqueues the call into `out` (a device tensor); every hold's result is
    compared bit for bit with the automatic one's, which is returned."""
    ref = None
    for h, c in ctxs.items():
        log_case(f"hold {h}: {what}")
        out.fill_(float("nan")) if out.dtype.is_floating_point else out.fill_(-1)
        run(c)
        torch.cuda.synchronize()
        got = out.cpu().numpy().copy()
        if ref is None:
            ref = got
        else:
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), f"{what}: hold {h} differs"
    return ref


def test_two_rank_kernels_every_hold(ctxs):
    srcs = wl.random_partials(50_000, 0, 2, N, dist="normal+outliers")
    dev = [to_device(s) for s in srcs]
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    got = same_everywhere(ctxs, "two-rank plain", lambda c: ar.ar_reduce(c, [out], dev, N, ar.AR_F32, ar.AR_BF16,
                                                                          ar.AR_MODE_CHUNKED), out)
    assert_bits_equal(got, oracle.reduce(srcs, ar.AR_BF16)[0], "two-rank plain vs oracle")
    res = wl.residual(50_001, 0, N, ar.AR_F32, dist="wide")
    rd = to_device(res)
    got = same_everywhere(ctxs, "two-rank element-wise residual",
                          lambda c: ar.ar_reduce_add(c, [out], dev, N, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                                                     rd, N), out)
    assert_bits_equal(got, oracle.reduce(srcs, ar.AR_BF16, residual=res)[0], "two-rank residual vs oracle")
    n2 = 1 << 22
    row = wl.residual(50_002, 0, 4096, ar.AR_F32, dist="wide")
    rw = to_device(row)
    out2 = torch.empty(n2, dtype=torch.float32, device="cuda")
    same_everywhere(ctxs, "two-rank broadcast row",
                    lambda c: ar.ar_reduce_add(c, [out2], [d[:n2] for d in dev], n2, ar.AR_F32, ar.AR_BF16,
                                               ar.AR_MODE_CHUNKED, rw, 4096), out2)
    rows, cols, ss, ds = 1100, 4096, 4608, 4352
    a = torch.randn(rows * ss, device="cuda")
    b = torch.randn(rows * ss, device="cuda")
    outr = torch.empty(rows * ds, dtype=torch.float32, device="cuda")
    same_everywhere(ctxs, "two-rank row-strided + bias row",
                    lambda c: ar.ar_reduce_rows(c, [outr], [a, b], rows, cols, ss, ds, ar.AR_F32, ar.AR_BF16,
                                                ar.AR_MODE_CHUNKED, residual=rw, res_stride=0), outr)


def test_16bit_two_rank_kernel_every_hold(ctxs):
    # two bf16 partials into bf16 (512 elements per wave), a ragged tail; every hold applies
    h = [torch.randn(N, device="cuda").bfloat16().view(torch.int16) for _ in range(2)]
    outh = torch.empty(N, dtype=torch.int16, device="cuda")
    assert planned_kernel([outh], h, N, ar.AR_BF16, ar.AR_BF16, ar.AR_MODE_CHUNKED) == 3
    got = same_everywhere(ctxs, "bf16 -> bf16 (two-rank 16-bit)",
                          lambda c: ar.ar_reduce(c, [outh], h, N, ar.AR_BF16, ar.AR_BF16, ar.AR_MODE_CHUNKED), outh)
    srcs = [t.cpu().numpy().view(np.uint16) for t in h]
    want = oracle.reduce(srcs, ar.AR_BF16, dst_type=ar.AR_BF16)[0]
    assert_bits_equal16(got.view(np.uint16), want, ar.AR_BF16, "two-rank 16-bit vs oracle")


def test_few_rank_kernel_every_hold(ctxs):
    # four ranks, rank 2 inactive: the kernel for a few active partials
    srcs = wl.random_partials(50_020, 0, 4, N, dist="normal+outliers")
    srcs[2] = None
    dev = [None if s is None else to_device(s) for s in srcs]
    ptrs = [0 if d is None else d for d in dev]
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    mode = ar.AR_MODE_CHUNKED | ar.AR_SRC_INACTIVE_NULL
    assert planned_kernel([out], ptrs, N, ar.AR_F32, ar.AR_BF16, mode) == 4
    got = same_everywhere(ctxs, "four ranks, one inactive (few active partials)",
                          lambda c: ar.ar_reduce(c, [out], ptrs, N, ar.AR_F32, ar.AR_BF16, mode), out)
    assert_bits_equal(got, oracle.reduce(srcs, ar.AR_BF16)[0], "few active partials vs oracle")


def test_general_kernels_every_hold(ctxs, lds_ctxs):
    # register-staged: eight fp32 partials; LDS-staged: two bf16 partials into bf16
    srcs = wl.random_partials(50_010, 0, 8, N, dist="normal")
    dev = [to_device(s) for s in srcs]
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    assert planned_kernel([out], dev, N, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED) == 1
    got = same_everywhere(ctxs, "R=8 fp32 (register-staged)",
                          lambda c: ar.ar_reduce(c, [out], dev, N, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED), out)
    assert_bits_equal(got, oracle.reduce(srcs, ar.AR_BF16)[0], "R=8 vs oracle")
    # LDS-staged (one wave tile of 4096 16-bit elements per wave): 2^25 elements, so every hold
    # applies; outputs compared across holds (the 16-bit paths' oracle parity is elsewhere)
    n16 = 1 << 25
    h = [torch.randn(n16, device="cuda").bfloat16().view(torch.int16) for _ in range(2)]
    outh = torch.empty(n16, dtype=torch.int16, device="cuda")
    assert planned_kernel([outh], h, n16, ar.AR_BF16, ar.AR_BF16, ar.AR_MODE_CHUNKED, {"stream_kernel": 2}) == 2
    same_everywhere(lds_ctxs, "bf16 -> bf16 (LDS-staged)",
                    lambda c: ar.ar_reduce(c, [outh], h, n16, ar.AR_BF16, ar.AR_BF16, ar.AR_MODE_CHUNKED), outh)
    del h, outh
    # the broadcast schedule: four fp32 partials into four destinations, fp16 wire
    n4 = 1 << 24
    s4 = [torch.randn(n4, device="cuda") for _ in range(4)]
    outs = [torch.empty(n4, dtype=torch.float32, device="cuda") for _ in range(4)]
    ref = None
    for hv, c in ctxs.items():
        log_case(f"hold {hv}: 4-rank broadcast")
        for o in outs:
            o.fill_(float("nan"))
        ar.ar_reduce(c, outs, s4, n4, ar.AR_F32, ar.AR_F16, ar.AR_MODE_RS_BCAST)
        torch.cuda.synchronize()
        got = np.stack([o.cpu().numpy() for o in outs])
        if ref is None:
            ref = got
            assert all(np.array_equal(got[d].view(np.uint32), got[0].view(np.uint32)) for d in range(4))
        else:
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"broadcast: hold {hv} differs"
