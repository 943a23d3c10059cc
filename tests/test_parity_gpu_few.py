"""The kernels for two to four active binary32 partials (``k_few``, plan
stream_kernel 4), bit for bit against the oracle through the C ABI.

They take three or four ranks, or two to four active ranks among up to 16,
compacted in rank order; an inactive rank contributes +0.0 at its place in
the fold, which turns a -0.0 running sum into +0.0.  The inputs therefore
carry signed zeros where every active partial is -0.0 (the sum stays -0.0
only when no inactive rank meets it), values that round to -0.0 on a 16-bit
wire, and the drawn distributions elsewhere.  Every rank pattern is checked
at sizes from one element to several launch tiles with a ragged tail and at
the prefill size, on every wire type, chunked and single-shot, and in place.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixed_precision_partial_amd as ar
import oracle
import workloads as wl
from gpu_util import GuardedDst, assert_bits_equal, log_case, to_device

pytestmark = pytest.mark.gpu

# active flags per rank: three and four ranks, one inactive at each place, two to four
# active among more ranks with inactive ones first, last and adjacent
PATTERNS = [
    (1, 1, 1), (1, 1, 1, 1),
    (0, 1, 1, 1), (1, 0, 1, 1), (1, 1, 0, 1), (1, 1, 1, 0),
    (0, 1, 1), (1, 0, 1), (1, 1, 0),
    (0, 0, 1, 1, 0), (1, 0, 0, 0, 0, 0, 0, 1), (0, 1, 0, 1, 1, 0, 1, 0),
    (0,) * 7 + (1,) + (0,) * 6 + (1, 0),
]
SIZES = [1, 7, 512, 4097, (1 << 20) + 37]
WIRES = [ar.AR_F32, ar.AR_BF16, ar.AR_F16]


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    c = ar.ar_init(0)
    yield c
    torch.cuda.synchronize()
    ar.ar_free(c)


def partials(seed: int, R: int, n: int) -> list[np.ndarray]:
    """R float32 partials; the first 64 elements are -0.0 in every partial, the next 64
    tiny negatives (-0.0 on a 16-bit wire) or -0.0 at random, the rest drawn."""
    p = wl.random_partials(seed, 0, R, n, dist="normal+outliers")
    rng = np.random.default_rng([seed, 7])
    for x in p:
        x[:64] = -0.0
        k = x[64:128]
        k[:] = np.where(rng.random(k.size) < 0.5, np.float32(-1e-30), np.float32(-0.0))
    return p


def run(ctx, active, n, wire, mode, seed, in_place=False, with_res=False):
    R = len(active)
    srcs = partials(seed, R, n)
    residual = None
    if with_res:
        residual = wl.residual(seed + 1, 0, n, ar.AR_F32, dist="wide")
        residual[:32] = -0.0          # -0.0 + -0.0 keeps the sign; +0.0 + -0.0 does not

    used = [s if a else None for s, a in zip(srcs, active)]
    ts = [to_device(s) if a else None for s, a in zip(srcs, active)]
    flags = 0 if all(active) else ar.AR_SRC_INACTIVE_NULL
    first = next(r for r, a in enumerate(active) if a)
    dst = None if in_place else GuardedDst(n)
    dptr = ts[first] if in_place else dst.ptr()
    ptrs = [0 if t is None else t for t in ts]
    what = f"active={active} n={n} wire={wire} mode={mode} in_place={in_place} residual={with_res}"
    if residual is None:
        rc, plan = ar.ar_plan_query([dptr], ptrs, n, ar.AR_F32, wire, mode | flags)
    else:
        rd = to_device(residual)
        rc, plan = ar.ar_plan_query_add([dptr], ptrs, n, ar.AR_F32, wire, mode | flags, rd, n)
    assert rc == ar.AR_OK and plan.stream_kernel == 4, what
    log_case(what)
    if residual is None:
        ar.ar_reduce(ctx, [dptr], ptrs, n, ar.AR_F32, wire, mode | flags)
    else:
        ar.ar_reduce_add(ctx, [dptr], ptrs, n, ar.AR_F32, wire, mode | flags, rd, n)
    torch.cuda.synchronize()
    want = oracle.reduce(used, wire, residual=residual)[0]
    got = ts[first].cpu().numpy() if in_place else dst.result()
    assert_bits_equal(got, want, what)
    # the signed zeros are compared bit for bit too: -0.0 survives only without inactive ranks
    assert np.signbit(want[:32]).all() == all(active), what


@pytest.mark.parametrize("active", PATTERNS, ids=lambda a: "".join(map(str, a)))
def test_rank_patterns(ctx, active):
    for i, n in enumerate(SIZES):
        for wire in WIRES:
            for mode in (ar.AR_MODE_CHUNKED, ar.AR_MODE_SINGLE_SHOT):
                run(ctx, active, n, wire, mode, seed=60_000 + 97 * i + wire)
        # with an element-wise residual
        run(ctx, active, n, ar.AR_BF16, ar.AR_MODE_CHUNKED, seed=62_000 + 97 * i, with_res=True)
        run(ctx, active, n, ar.AR_F16, ar.AR_MODE_SINGLE_SHOT, seed=62_500 + 97 * i, with_res=True)


def test_prefill_size_and_in_place(ctx):
    n = 2048 * 4096
    for active in ((1, 1, 1), (1, 1, 0, 1), (1, 1, 1, 1), (0, 1, 0, 0, 1, 0, 1, 0)):
        run(ctx, active, n, ar.AR_BF16, ar.AR_MODE_CHUNKED, seed=61_000 + len(active))
    run(ctx, (1, 1, 0, 1), n + 1000, ar.AR_F16, ar.AR_MODE_AUTO, seed=61_100)
    for active in ((1, 1, 1), (0, 1, 1, 1), (1, 0, 1, 1, 0)):
        run(ctx, active, (1 << 20) + 37, ar.AR_BF16, ar.AR_MODE_CHUNKED, seed=61_200, in_place=True)
        run(ctx, active, (1 << 20) + 37, ar.AR_BF16, ar.AR_MODE_CHUNKED, seed=61_300, in_place=True,
            with_res=True)
    run(ctx, (1, 1, 1, 1), n, ar.AR_BF16, ar.AR_MODE_CHUNKED, seed=61_400, with_res=True)
    torch.cuda.empty_cache()
