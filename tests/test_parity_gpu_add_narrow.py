"""HIP path against the CPU oracle, bit for bit, for the residual add
(``ar_reduce_add``: element-wise and broadcast-row residuals) and for narrow
(binary16 / bfloat16) destinations, through the C ABI.

Every schedule, every kernel family that has the form, rank buckets, ragged
tails, edge values, inactive ranks, in-place use and the full-size workload
shapes are covered; the oracle computes the expected bytes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixed_precision_partial_amd as ar
import oracle
import workloads as wl
from gpu_util import GuardedDst, assert_bits_equal, assert_bits_equal16, log_case, to_device, to_pinned

pytestmark = pytest.mark.gpu

MODES = {
    "single_shot": ar.AR_MODE_SINGLE_SHOT,
    "chunked": ar.AR_MODE_CHUNKED,
    "rs_bcast": ar.AR_MODE_RS_BCAST,
    "host_staged": ar.AR_MODE_HOST_STAGED,
}
WIRES = {"f32": ar.AR_F32, "bf16": ar.AR_BF16, "f16": ar.AR_F16}
NARROW = {"bf16": ar.AR_BF16, "f16": ar.AR_F16}

# (host-staged calls go through the copy-engine pipeline where host_path is 1)
KERNEL_CONFIGS = {
    "default": {},
    "reg_cached": {"stream_kernel": 1, "store_policy": 1, "host_path": 1},
    "reg_streaming": {"stream_kernel": 1, "store_policy": 2, "host_path": 1},
    "lds_cached": {"stream_kernel": 2, "store_policy": 1, "host_path": 1},
    "lds_streaming": {"stream_kernel": 2, "store_policy": 2, "host_path": 1},
    "host_direct": {"host_path": 2},
    "small_chunks": {"chunk_bytes": 4096, "host_chunk_bytes": 1 << 14, "host_path": 1},
}


@pytest.fixture(scope="module")
def kctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ctxs = {k: ar.ar_init(0, v or None) for k, v in KERNEL_CONFIGS.items()}
    yield ctxs
    torch.cuda.synchronize()
    for c in ctxs.values():
        ar.ar_free(c)


def run_and_check(ctx, srcs, wire, mode, what, dst_type=ar.AR_F32, src_wire=False, residual=None,
                  active=None):
    """One call through the C ABI (ar_reduce, or ar_reduce_add with a residual), every
    destination compared with the oracle.  ``srcs`` are float32 draws, or uint16
    patterns for wire-typed / narrow sources; ``active`` masks ranks (None = all)."""
    R = len(srcs)
    n = srcs[0].size
    base = mode & ar.AR_MODE_MASK
    n_dst = R if base == ar.AR_MODE_RS_BCAST else 1
    narrow = dst_type != ar.AR_F32
    if src_wire and not narrow:
        srcs = [wl.as_wire_typed(s, wire) if s.dtype == np.float32 else s for s in srcs]
    active = [True] * R if active is None else list(active)
    put = to_pinned if base == ar.AR_MODE_HOST_STAGED else to_device
    ts = [put(s) if a else None for s, a in zip(srcs, active)]
    dsts = [GuardedDst(n, 16 if narrow else 32) for _ in range(n_dst)]
    flags = (ar.AR_SRC_WIRE if src_wire else 0) | (0 if all(active) else ar.AR_SRC_INACTIVE_NULL)
    log_case(what)
    ptrs = [0 if t is None else t for t in ts]
    if residual is None:
        ar.ar_reduce(ctx, [d.ptr() for d in dsts], ptrs, n, dst_type, wire, mode | flags)
    else:
        res_dev = to_device(residual)
        ar.ar_reduce_add(ctx, [d.ptr() for d in dsts], ptrs, n, dst_type, wire, mode | flags, res_dev,
                         residual.size)
    torch.cuda.synchronize()
    used = [s if a else None for s, a in zip(srcs, active)]
    src_type = wire if (src_wire or narrow) and wire != ar.AR_F32 else None
    want = oracle.reduce(used, wire, src_type=src_type, dst_type=dst_type, residual=residual, n=n)[0]
    for d, g in enumerate(dsts):
        got = g.result()
        if narrow:
            assert_bits_equal16(got, want, dst_type, f"{what} dst {d}")
        else:
            assert_bits_equal(got, want, f"{what} dst {d}")


def residual_for(case, n, length, dtype=ar.AR_F32):
    r = wl.residual(case, 0, length, dtype, dist="wide")
    if dtype == ar.AR_F32:
        g = np.concatenate([wl.special_values(), wl.nan_values()])
    else:
        g = np.concatenate([wl.special_values16(dtype), wl.nan_values16(dtype)])
    k = min(g.size, length)
    r[:k] = g[:k]
    return r


# (R, rows, row length): n = rows x row length, ragged against 512-element tiles
SHAPES = [(2, 17, 4104), (3, 9, 520), (5, 1001, 8), (8, 3, 65_544), (16, 2, 1_032)]


# --------------------------------------------------------------------------
# residual add, binary32 destinations
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kname", ["default", "reg_cached", "reg_streaming", "lds_cached", "lds_streaming",
                                   "host_direct", "small_chunks"])
@pytest.mark.parametrize("mode_name", ["single_shot", "chunked", "rs_bcast", "host_staged"])
def test_residual_every_schedule(kctx, kname, mode_name):
    mode = MODES[mode_name]
    for i, (R, rows, L) in enumerate(SHAPES):
        n = rows * L
        srcs = wl.random_partials(11_000 + i, 0, R, n, dist="wide")
        for wire_name, wire in WIRES.items():
            for src_wire in ([False, True] if wire != ar.AR_F32 else [False]):
                for form, res in (("elementwise", residual_for(11_100 + i, n, n)),
                                  ("row", residual_for(11_200 + i, n, L))):
                    what = (f"residual {form} {kname} {mode_name} R={R} n={n} L={res.size} "
                            f"wire={wire_name} src_wire={src_wire}")
                    run_and_check(kctx[kname], srcs, wire, mode, what, src_wire=src_wire, residual=res)


@pytest.mark.parametrize("mode_name", ["single_shot", "chunked", "rs_bcast", "host_staged"])
def test_residual_with_inactive_ranks(kctx, mode_name):
    rng = np.random.default_rng(12)
    for i, (R, rows, L) in enumerate(SHAPES):
        n = rows * L
        srcs = wl.random_partials(12_000 + i, 0, R, n, dist="wide")
        res = residual_for(12_100 + i, n, L if i % 2 else n)
        for trial in range(2):
            active = rng.random(R) < 0.5
            if trial == 1:
                active[:] = False
            for wire_name, wire in WIRES.items():
                what = (f"residual inactive {mode_name} R={R} n={n} L={res.size} wire={wire_name} "
                        f"active={active.astype(int).tolist()}")
                run_and_check(kctx["default"], srcs, wire, MODES[mode_name], what, residual=res, active=active)


def test_residual_in_place(kctx):
    """x += reduce(partials): the element-wise residual is the destination itself."""
    for mode_name in ("single_shot", "chunked", "rs_bcast"):
        n, R = 70_001, 4
        srcs = wl.random_partials(13_000, 0, R, n, dist="wide")
        res = wl.residual(13_000, 1, n)
        want = oracle.reduce(srcs, ar.AR_BF16, residual=res)[0]
        base = MODES[mode_name]
        dev = [to_device(s) for s in srcs]
        n_dst = R if base == ar.AR_MODE_RS_BCAST else 1
        dsts = [to_device(res) for _ in range(n_dst)]
        log_case(f"residual in place {mode_name}")
        ar.ar_reduce_add(kctx["default"], dsts, dev, n, ar.AR_F32, ar.AR_BF16, base, dsts[0], n)
        torch.cuda.synchronize()
        assert_bits_equal(dsts[0].cpu().numpy(), want, f"residual in place {mode_name}")
        # with a residual that is also a source (read only)
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        ar.ar_reduce_add(kctx["default"], [out], dev, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, dev[1], n)
        torch.cuda.synchronize()
        assert_bits_equal(out.cpu().numpy(), oracle.reduce(srcs, ar.AR_BF16, residual=srcs[1])[0],
                          "residual aliasing a source")


# two-rank kernels with a residual: broadcast rows shorter than, equal to and longer
# than one 512-element wave tile (several wraps per tile, none, at most one), ragged
# row counts, element-wise, in place
PAIR_ROWS = [(8, 3001), (24, 999), (504, 33), (512, 17), (520, 9), (4096, 5), (4104, 3), (12_288, 2)]


def test_two_rank_kernel_with_residual(kctx):
    for i, (L, rows) in enumerate(PAIR_ROWS):
        n = L * rows
        rc, plan = ar.ar_plan_query_add([0x10_0000_0000], [0x20_0000_0000, 0x30_0000_0000], n, ar.AR_F32,
                                        ar.AR_BF16, ar.AR_MODE_CHUNKED, 0x40_0000_0000, L)
        assert rc == ar.AR_OK and plan.stream_kernel == 3 and plan.residual_kind == 2, (L, rows)
        srcs = wl.random_partials(14_000 + i, 0, 2, n, dist="wide")
        for wire_name, wire in WIRES.items():
            for form, res in (("row", residual_for(14_100 + i, n, L)), ("elementwise", residual_for(14_200 + i, n, n))):
                what = f"pair residual {form} n={n} L={res.size} wire={wire_name}"
                run_and_check(kctx["default"], srcs, wire, ar.AR_MODE_CHUNKED, what, residual=res)
    # in place: x = reduce(partials) + x
    n = (1 << 18) + 40
    srcs = wl.random_partials(14_300, 0, 2, n, dist="normal+outliers")
    res = wl.residual(14_300, 1, n)
    want = oracle.reduce(srcs, ar.AR_BF16, residual=res)[0]
    dev = [to_device(s) for s in srcs]
    x = to_device(res)
    log_case(f"pair residual in place n={n}")
    ar.ar_reduce_add(kctx["default"], [x], dev, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, x, n)
    torch.cuda.synchronize()
    assert_bits_equal(x.cpu().numpy(), want, "pair residual in place")


def test_residual_errors(kctx):
    n = 4096
    dev = [to_device(np.ones(n, dtype=np.float32)) for _ in range(2)]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    res_host = to_pinned(np.ones(n, dtype=np.float32))
    res_pageable = np.ones(n, dtype=np.float32)
    res_short = torch.ones(n // 2, dtype=torch.float32, device="cuda")
    c = kctx["default"]
    log_case("residual error paths")
    E = ar.AR_ERR_INVALID
    # pinned host residual: invalid (device memory only)
    assert ar.ar_reduce_add(c, [out], dev, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, res_host, n,
                            check=False) == E
    # pageable host memory
    assert ar.ar_reduce_add(c, [out], dev, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                            res_pageable.ctypes.data, n, check=False) == E
    # a row that does not divide n (longer than the tensor too: the library's checks are the
    # ones exercised, so the binding's size check is switched off)
    assert ar.ar_reduce_add(c, [out], dev, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, res_short, 3000,
                            check=False, validate=False) == E
    # a broadcast row overlapping the destination
    assert ar.ar_reduce_add(c, [out], dev, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, out, 512,
                            check=False) == E
    torch.cuda.synchronize()
    ar.ar_reduce_add(c, [out], dev, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, res_short, n // 2)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 3.0)


# --------------------------------------------------------------------------
# narrow destinations
# --------------------------------------------------------------------------

NARROW_CASES = [(2, 70_001), (3, 4_097), (4, 131_072 + 515), (7, 9_000), (8, 65_537), (13, 2_049),
                (16, 20_483), (2, 1), (2, 511), (5, 513)]


@pytest.mark.parametrize("kname", list(KERNEL_CONFIGS))
@pytest.mark.parametrize("mode_name", ["single_shot", "chunked", "rs_bcast", "host_staged"])
def test_narrow_every_schedule(kctx, kname, mode_name):
    for i, (R, n) in enumerate(NARROW_CASES):
        for t_name, t in NARROW.items():
            srcs = wl.random_narrow(14_000 + i, 0, R, n, t, dist="wide")
            g = np.concatenate([wl.special_values16(t), wl.nan_values16(t)])
            k = min(g.size, n)
            srcs[0][:k] = g[:k]
            srcs[-1][:k] = g[::-1][:k]
            for src_flag in (False, True):
                what = f"narrow {kname} {mode_name} R={R} n={n} type={t_name} AR_SRC_WIRE={src_flag}"
                run_and_check(kctx[kname], srcs, t, MODES[mode_name], what, dst_type=t, src_wire=src_flag)


@pytest.mark.parametrize("mode_name", ["single_shot", "chunked", "rs_bcast", "host_staged"])
def test_narrow_edge_pairs(kctx, mode_name):
    """Every ordered pair and a grid of triples of 16-bit edge patterns."""
    for t_name, t in NARROW.items():
        g = np.concatenate([wl.special_values16(t), wl.nan_values16(t)])
        a, b = np.meshgrid(g, g, indexing="ij")
        pairs = [a.ravel().copy(), b.ravel().copy()]
        x, y, z = np.meshgrid(g, g, g, indexing="ij")
        triples = [x.ravel().copy(), y.ravel().copy(), z.ravel().copy()]
        for srcs in (pairs, triples):
            what = f"narrow edge {mode_name} R={len(srcs)} type={t_name} n={srcs[0].size}"
            run_and_check(kctx["default"], srcs, t, MODES[mode_name], what, dst_type=t)


@pytest.mark.parametrize("kname", ["default", "reg_streaming", "lds_cached", "lds_streaming", "host_direct"])
@pytest.mark.parametrize("mode_name", ["single_shot", "chunked", "rs_bcast", "host_staged"])
def test_narrow_with_residual_and_inactive(kctx, kname, mode_name):
    rng = np.random.default_rng(15)
    for i, (R, rows, L) in enumerate(SHAPES):
        n = rows * L
        for t_name, t in NARROW.items():
            srcs = wl.random_narrow(15_000 + i, 0, R, n, t, dist="wide")
            for form, res in (("elementwise", residual_for(15_100 + i, n, n, t)),
                              ("row", residual_for(15_200 + i, n, L, t))):
                active = rng.random(R) < 0.7
                what = (f"narrow residual {form} {kname} {mode_name} R={R} n={n} L={res.size} type={t_name} "
                        f"active={active.astype(int).tolist()}")
                run_and_check(kctx[kname], srcs, t, MODES[mode_name], what, dst_type=t, residual=res,
                              active=active)


def test_narrow_in_place(kctx):
    n, R = 100_003, 3
    for t_name, t in NARROW.items():
        srcs = wl.random_narrow(16_000, 0, R, n, t)
        want = oracle.reduce(srcs, t, src_type=t, dst_type=t)[0]
        dev = [to_device(s) for s in srcs]
        log_case(f"narrow in place {t_name}")
        ar.ar_reduce(kctx["default"], [dev[1]], dev, n, t, t, ar.AR_MODE_CHUNKED)
        torch.cuda.synchronize()
        assert_bits_equal16(dev[1].cpu().numpy().view(np.uint16), want, t, f"narrow in place {t_name}")


def test_two_rank_16bit_kernel(kctx):
    """Two 16-bit partials into their own type without a residual take the two-rank 16-bit
    kernel (k_pair16): sizes around the 512-element tile, a ragged prefill shape, single-shot
    and chunked, in place too; bit for bit against the oracle."""
    sizes = [1, 7, 511, 512, 513, 4097, 65_536 + 5, (1 << 20) + 123, 2048 * 4096 + 1000]
    for t_name, t in NARROW.items():
        g = np.concatenate([wl.special_values16(t), wl.nan_values16(t)])
        for i, n in enumerate(sizes):
            srcs = wl.random_narrow(17_000 + i, 0, 2, n, t, dist="wide")
            k = min(g.size, n)
            srcs[0][:k] = g[:k]
            srcs[1][:k] = g[::-1][:k]
            for mode in ((ar.AR_MODE_SINGLE_SHOT, ar.AR_MODE_CHUNKED) if n < (1 << 21) else (ar.AR_MODE_CHUNKED,)):
                rc, plan = ar.ar_plan_query([0x10_0000_0000], [0x20_0000_0000, 0x30_0000_0000], n, t, t, mode)
                assert rc == ar.AR_OK and plan.stream_kernel == 3, (t_name, n, mode)
                run_and_check(kctx["default"], srcs, t, mode, f"two-rank 16-bit {t_name} n={n} mode={mode}",
                              dst_type=t)
        n = 100_003
        srcs = wl.random_narrow(17_100, 0, 2, n, t)
        want = oracle.reduce(srcs, t, src_type=t, dst_type=t)[0]
        dev = [to_device(s) for s in srcs]
        log_case(f"two-rank 16-bit in place {t_name}")
        ar.ar_reduce(kctx["default"], [dev[0]], dev, n, t, t, ar.AR_MODE_CHUNKED)
        torch.cuda.synchronize()
        assert_bits_equal16(dev[0].cpu().numpy().view(np.uint16), want, t, f"two-rank 16-bit in place {t_name}")


# --------------------------------------------------------------------------
# the workload shapes at full size
# --------------------------------------------------------------------------

def test_prefill_shape_with_residual(kctx):
    """2048 x 4096, R=2 fp32 partials through a bf16 wire, plus the hidden-state residual
    (element-wise) and a bias-like broadcast row of 4096."""
    w = wl.WORKLOADS["prefill_bf16"]
    srcs = wl.partials(w, 0)
    res = wl.residual(w.case, 0, w.n)
    run_and_check(kctx["default"], srcs, w.wire, ar.AR_MODE_CHUNKED, "prefill + residual", residual=res)
    row = wl.residual(w.case, 1, 4096)
    run_and_check(kctx["default"], srcs, w.wire, ar.AR_MODE_CHUNKED, "prefill + row", residual=row)


def test_slice_bcast_shape_narrow(kctx):
    """2048 x 8192, R=4 fp16 partials reduced in fp16 to 4 fp16 destinations."""
    w = wl.WORKLOADS["slice_bcast_f16"]
    srcs = [wl.as_wire_typed(p, ar.AR_F16) for p in wl.partials(w, 0)]
    run_and_check(kctx["default"], srcs, ar.AR_F16, ar.AR_MODE_RS_BCAST, "slice bcast fp16 dst",
                  dst_type=ar.AR_F16)


def test_prefill_shape_narrow_bf16(kctx):
    w = wl.WORKLOADS["prefill_bf16"]
    srcs = [wl.as_wire_typed(p, ar.AR_BF16) for p in wl.partials(w, 2)]
    res = wl.residual(w.case, 2, w.n, ar.AR_BF16)
    run_and_check(kctx["default"], srcs, ar.AR_BF16, ar.AR_MODE_CHUNKED, "prefill bf16 dst + residual",
                  dst_type=ar.AR_BF16, residual=res)


def test_decode_shape_with_residual(kctx):
    w = wl.WORKLOADS["decode_bf16"]
    for c in range(8):
        srcs = wl.partials(w, c)
        res = wl.residual(w.case, c, w.n)
        run_and_check(kctx["default"], srcs, w.wire, ar.AR_MODE_SINGLE_SHOT, f"decode + residual call {c}",
                      residual=res)
