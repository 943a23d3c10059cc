"""Maximum sizes: calls longer than one launch covers (2^30 elements) and, on
the slice + broadcast schedule, calls past 2^32 elements, through the C ABI.

The inputs are drawn on the device with torch's seeded generator; the oracle
checks sampled outputs one by one (every launch-piece, chunk and slice
boundary, the ragged tail and random positions), gathering the same input
elements back to the host.  Properties that hold at any size (all
destinations byte-identical) are checked over the whole tensors.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixed_precision_partial_amd as ar
import oracle
from gpu_util import assert_bits_equal, assert_bits_equal16, log_case

pytestmark = pytest.mark.gpu

LAUNCH = 1 << 30   # elements one launch covers


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    c = ar.ar_init(0)
    yield c
    torch.cuda.synchronize()
    ar.ar_free(c)


def sample_indices(n: int, boundaries, seed: int) -> np.ndarray:
    near = []
    for b in boundaries:
        near.extend(range(max(0, b - 9), min(n, b + 9)))
    near.extend(range(max(0, n - 700), n))
    rnd = np.random.default_rng(seed).integers(0, n, 20_000)
    return np.unique(np.concatenate([np.array(near, dtype=np.int64), rnd.astype(np.int64)]))


def gather(t: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    g = t[torch.from_numpy(idx).to(t.device)].cpu()
    if g.dtype == torch.float32:
        return g.numpy()
    return g.view(torch.int16).numpy().view(np.uint16)


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_beyond_one_launch(ctx):
    """n = 2^30 + 2^20 + 4099 fp32 partials, bf16 wire: every schedule cuts the call into
    launch pieces; with an element-wise residual and without."""
    n = LAUNCH + (1 << 20) + 4099
    g = torch.Generator(device="cuda")
    g.manual_seed(20_001)
    srcs = [torch.randn(n, device="cuda", generator=g) for _ in range(2)]
    res = torch.randn(n, device="cuda", generator=g)
    rc, plan = ar.ar_plan_query([0x10_0000_0000], [0x20_0000_0000, 0x30_0000_0000], n, ar.AR_F32, ar.AR_BF16,
                                ar.AR_MODE_CHUNKED)
    chunk_bounds = list(range(0, n, plan.chunk_elems))
    idx = sample_indices(n, [LAUNCH, 1 << 29, 3 << 28] + chunk_bounds[:64] + chunk_bounds[-64:], 7)
    s_host = [gather(s, idx) for s in srcs]
    r_host = gather(res, idx)
    want_plain = oracle.reduce(s_host, ar.AR_BF16)[0]
    want_res = oracle.reduce(s_host, ar.AR_BF16, residual=r_host)[0]
    out = torch.empty(n, device="cuda")
    for mode_name, mode in (("chunked", ar.AR_MODE_CHUNKED), ("single_shot", ar.AR_MODE_SINGLE_SHOT)):
        for with_res in (False, True):
            what = f"n={n} {mode_name} residual={with_res}"
            log_case(what)
            out.fill_(float("nan"))
            if with_res:
                ar.ar_reduce_add(ctx, [out], srcs, n, ar.AR_F32, ar.AR_BF16, mode, res, n)
            else:
                ar.ar_reduce(ctx, [out], srcs, n, ar.AR_F32, ar.AR_BF16, mode)
            torch.cuda.synchronize()
            assert not torch.isnan(out).any().item(), f"{what}: some element left unwritten"
            assert_bits_equal(gather(out, idx), want_res if with_res else want_plain, what)
    del out
    # slice + broadcast: both destinations identical over the whole tensor
    log_case(f"n={n} rs_bcast residual")
    dsts = [torch.empty(n, device="cuda") for _ in range(2)]
    ar.ar_reduce_add(ctx, dsts, srcs, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_RS_BCAST, res, n)
    torch.cuda.synchronize()
    assert torch.equal(dsts[0].view(torch.int32), dsts[1].view(torch.int32))
    assert_bits_equal(gather(dsts[1], idx), want_res, "rs_bcast residual")
    del dsts, srcs, res
    free()


def test_two_rank_16bit_beyond_one_launch(ctx):
    """n = 2^30 + 2^20 + 4099 bf16 partials into a bf16 destination, on the two-rank 16-bit
    kernel: both schedules cut the call into launch pieces, the last one with a ragged tail."""
    n = LAUNCH + (1 << 20) + 4099
    rc, plan = ar.ar_plan_query([0x10_0000_0000], [0x20_0000_0000, 0x30_0000_0000], n, ar.AR_BF16, ar.AR_BF16,
                                ar.AR_MODE_CHUNKED)
    assert rc == ar.AR_OK and plan.stream_kernel == 3
    g = torch.Generator(device="cuda")
    g.manual_seed(20_005)
    srcs = [torch.randn(n, device="cuda", generator=g).bfloat16().view(torch.int16) for _ in range(2)]
    idx = sample_indices(n, [LAUNCH, LAUNCH - 512, 1 << 29, n - 4099], 9)
    want = oracle.reduce([gather(s, idx) for s in srcs], ar.AR_BF16, dst_type=ar.AR_BF16)[0]
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    for mode_name, mode in (("chunked", ar.AR_MODE_CHUNKED), ("single_shot", ar.AR_MODE_SINGLE_SHOT)):
        what = f"n={n} bf16 -> bf16 {mode_name}"
        log_case(what)
        out.fill_(-1)         # 0xffff, a NaN pattern the finite inputs never produce
        ar.ar_reduce(ctx, [out], srcs, n, ar.AR_BF16, ar.AR_BF16, mode)
        torch.cuda.synchronize()
        assert not (out == -1).any().item(), f"{what}: some element left unwritten"
        assert_bits_equal16(gather(out, idx), want, ar.AR_BF16, what)
    del out, srcs
    free()


def test_few_partials_beyond_one_launch(ctx):
    """n = 2^30 + 2^20 + 4099, four fp32 partials with rank 2 inactive (the kernel for a few
    active partials), with and without an element-wise residual: every launch piece takes
    its own slice of the compacted sources and of the residual."""
    n = LAUNCH + (1 << 20) + 4099
    g = torch.Generator(device="cuda")
    g.manual_seed(20_006)
    srcs = [None if r == 2 else torch.randn(n, device="cuda", generator=g) for r in range(4)]
    res = torch.randn(n, device="cuda", generator=g)
    ptrs = [0 if s is None else s for s in srcs]
    mode = ar.AR_MODE_CHUNKED | ar.AR_SRC_INACTIVE_NULL
    fake = [0x20_0000_0000, 0x30_0000_0000, 0, 0x40_0000_0000]
    rc, plan = ar.ar_plan_query([0x10_0000_0000], fake, n, ar.AR_F32, ar.AR_BF16, mode)
    assert rc == ar.AR_OK and plan.stream_kernel == 4
    rc, plan = ar.ar_plan_query_add([0x10_0000_0000], fake, n, ar.AR_F32, ar.AR_BF16, mode, 0x50_0000_0000, n)
    assert rc == ar.AR_OK and plan.stream_kernel == 4
    idx = sample_indices(n, [LAUNCH, LAUNCH - 512, 1 << 29, n - 4099], 10)
    s_host = [None if s is None else gather(s, idx) for s in srcs]
    r_host = gather(res, idx)
    out = torch.empty(n, device="cuda")
    for with_res in (False, True):
        what = f"n={n} four ranks, rank 2 inactive, residual={with_res}"
        log_case(what)
        out.fill_(float("nan"))
        if with_res:
            ar.ar_reduce_add(ctx, [out], ptrs, n, ar.AR_F32, ar.AR_BF16, mode, res, n)
        else:
            ar.ar_reduce(ctx, [out], ptrs, n, ar.AR_F32, ar.AR_BF16, mode)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any().item(), f"{what}: some element left unwritten"
        want = oracle.reduce(s_host, ar.AR_BF16, residual=r_host if with_res else None)[0]
        assert_bits_equal(gather(out, idx), want, what)
    del out, srcs, res
    free()


def test_beyond_one_launch_row_residual(ctx):
    """n = 2^30 + 8 with a broadcast row of 24 elements (which does not divide 2^30): the
    second launch piece starts 16 elements into the row.  Two fp32 partials, bf16 wire."""
    n, L = LAUNCH + 8, 24
    assert n % L == 0 and LAUNCH % L != 0
    g = torch.Generator(device="cuda")
    g.manual_seed(20_002)
    srcs = [torch.randn(n, device="cuda", generator=g) for _ in range(2)]
    row = torch.randn(L, device="cuda", generator=g)
    rc, plan = ar.ar_plan_query_add([0x10_0000_0000], [0x20_0000_0000, 0x30_0000_0000], n, ar.AR_F32,
                                    ar.AR_BF16, ar.AR_MODE_CHUNKED, 0x40_0000_0000, L)
    assert rc == ar.AR_OK and plan.stream_kernel == 3 and plan.residual_kind == 2
    idx = sample_indices(n, [LAUNCH, LAUNCH - 512, 1 << 29], 8)
    s_host = [gather(s, idx) for s in srcs]
    want = oracle.reduce(s_host, ar.AR_BF16, residual=row.cpu().numpy()[idx % L])[0]
    out = torch.empty(n, device="cuda")
    out.fill_(float("nan"))
    log_case(f"n={n} chunked row residual L={L}")
    ar.ar_reduce_add(ctx, [out], srcs, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, row, L)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item(), "some element left unwritten"
    assert_bits_equal(gather(out, idx), want, "row residual beyond one launch")
    del out, srcs
    free()


def test_slice_broadcast_past_2_32(ctx):
    """n = 8200 x 523,779 (past 2^32) bf16 partials (R=2), slice + broadcast to 2 fp32
    destinations, with a broadcast row of 8200 elements (which does not divide 2^32, so a
    row index taken from a position cut to 32 bits would be wrong): element positions
    past 2^32 inside one launch."""
    L = 8200
    n = L * (-(-(1 << 32) // L) + 1)
    assert n > (1 << 32) and (1 << 32) % L != 0
    g = torch.Generator(device="cuda")
    g.manual_seed(20_002)
    srcs = [torch.randn(n, device="cuda", dtype=torch.bfloat16, generator=g) for _ in range(2)]
    row = torch.randn(L, device="cuda", generator=g)
    fake = [k << 40 for k in range(1, 5)]   # well separated addresses: the plan only reads them
    rc, plan = ar.ar_plan_query(fake[:2], fake[2:], n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_RS_BCAST | ar.AR_SRC_WIRE)
    assert rc == ar.AR_OK
    bounds = [plan.slice_start[r] for r in range(2)] + [LAUNCH, 2 * LAUNCH, 3 * LAUNCH, 1 << 32]
    bounds += [plan.slice_start[1] + LAUNCH, plan.slice_start[1] + 2 * LAUNCH]
    idx = sample_indices(n, bounds, 8)
    s_host = [gather(s, idx) for s in srcs]
    r_host = row.cpu().numpy()[idx % L]
    want = oracle.reduce(s_host, ar.AR_BF16, src_type=ar.AR_BF16, residual=r_host)[0]
    dsts = [torch.empty(n, device="cuda") for _ in range(2)]
    log_case(f"n={n} rs_bcast bf16 sources, row residual L={L}")
    ar.ar_reduce_add(ctx, dsts, srcs, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_RS_BCAST | ar.AR_SRC_WIRE, row, L)
    torch.cuda.synchronize()
    assert torch.equal(dsts[0].view(torch.int32), dsts[1].view(torch.int32))
    assert_bits_equal(gather(dsts[0], idx), want, "past 2^32 rs_bcast row residual")
    del dsts, srcs
    free()


def test_beyond_one_launch_rows(ctx):
    """Row-strided two-rank reduce of 2^18 + 3 rows of 4096 (past one launch: the rows are
    cut into launch pieces of 2^18 rows) with padded strides and a bias row; sampled rows
    around the piece boundary and at random against the oracle, and the padding after
    them untouched."""
    rows, cols, ss, ds = (1 << 18) + 3, 4096, 4096 + 64, 4096 + 128
    rc, plan = ar.ar_plan_query_rows([0x10_0000_0000], [0x20_0000_0000, 0x30_0000_0000], rows, cols, ss, ds,
                                     ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, residual=0x40_0000_0000,
                                     res_stride=0)
    assert rc == ar.AR_OK and plan.stream_kernel == 3
    g = torch.Generator(device="cuda")
    g.manual_seed(20_003)
    src_len, dst_len = (rows - 1) * ss + cols, (rows - 1) * ds + cols
    srcs = [torch.randn(src_len, device="cuda", generator=g) for _ in range(2)]
    bias = torch.randn(cols, device="cuda", generator=g)
    out = torch.empty(dst_len, device="cuda")
    out.fill_(float("nan"))
    log_case(f"rows {rows}x{cols} strides {ss}/{ds} bias row, two-rank kernel in launch pieces")
    ar.ar_reduce_rows(ctx, [out], srcs, rows, cols, ss, ds, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                      residual=bias, res_stride=0)
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([np.arange(4), np.arange((1 << 18) - 3, (1 << 18) + 3),
                                     np.arange(rows - 3, rows),
                                     np.random.default_rng(9).integers(0, rows, 40)]))
    idx_src = (pick[:, None] * ss + np.arange(cols)[None, :]).ravel()
    idx_dst = (pick[:, None] * ds + np.arange(cols)[None, :]).ravel()
    s_host = [gather(s, idx_src) for s in srcs]
    want = oracle.reduce(s_host, ar.AR_BF16, residual=np.tile(bias.cpu().numpy(), pick.size))[0]
    assert_bits_equal(gather(out, idx_dst), want, "rows beyond one launch")
    gap = (pick[pick < rows - 1][:, None] * ds + cols + np.arange(ds - cols)[None, :]).ravel()
    assert np.isnan(gather(out, gap)).all(), "written between rows"
    del srcs, out
    free()
