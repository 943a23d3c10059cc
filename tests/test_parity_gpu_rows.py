"""HIP path against the CPU oracle, bit for bit, for row-strided tensors
(``ar_reduce_rows``), through the C ABI.

Sources carry NaN in the elements between rows (a kernel that read them would
turn results into NaN); destinations start filled with a sentinel NaN pattern
that must survive between the rows and in the guard bands.  Every schedule,
both streaming families, the host-staged copy pipeline (2-D copies) and the
direct host reads, all wire types, narrow destinations, residual rows
(strided and broadcast) and inactive ranks are covered, plus a prefill-shaped
block inside wider rows at full size.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixed_precision_partial_amd as ar
import oracle
import workloads as wl
from gpu_util import (SENTINEL, SENTINEL16, GuardedDst, assert_bits_equal, assert_bits_equal16, log_case,
                      to_device, to_pinned)

pytestmark = pytest.mark.gpu

MODES = {
    "single_shot": ar.AR_MODE_SINGLE_SHOT,
    "chunked": ar.AR_MODE_CHUNKED,
    "rs_bcast": ar.AR_MODE_RS_BCAST,
    "host_staged": ar.AR_MODE_HOST_STAGED,
}
WIRES = {"f32": ar.AR_F32, "bf16": ar.AR_BF16, "f16": ar.AR_F16}
# (host-staged calls go through the 2-D copy-engine pipeline where host_path is 1)
KERNEL_CONFIGS = {
    "default": {},
    "reg_streaming": {"stream_kernel": 1, "store_policy": 2, "host_path": 1},
    "lds_cached": {"stream_kernel": 2, "store_policy": 1, "host_path": 1},
    "host_direct": {"host_path": 2},
    "small_chunks": {"host_chunk_bytes": 1 << 13, "host_path": 1},
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


def span(rows, cols, stride):
    return 0 if rows == 0 or cols == 0 else (rows - 1) * stride + cols


def strided(rows, cols, stride, dense: np.ndarray, fill) -> np.ndarray:
    """Flat array of a row-strided tensor: rows of `dense` (rows x cols), `fill` between rows."""
    out = np.full(span(rows, cols, stride), fill, dtype=dense.dtype)
    for i in range(rows):
        out[i * stride:i * stride + cols] = dense[i * cols:(i + 1) * cols]
    return out


def run_rows_case(ctx, rows, cols, ss, ds, R, wire, mode, what, dst_type=ar.AR_F32, src_wire=False,
                  res_kind=None, rs=0, active=None, seed=0):
    narrow = dst_type != ar.AR_F32
    base = mode & ar.AR_MODE_MASK
    n_dst = R if base == ar.AR_MODE_RS_BCAST else 1
    n = rows * cols
    dense = wl.random_partials(30_000 + seed, 0, R, n, dist="wide")
    if narrow or src_wire:
        dense = [wl.as_wire_typed(d, wire) for d in dense]
        pad = np.uint16(0x7FC0 if wire == ar.AR_BF16 else 0x7E00)   # a NaN of the wire type
    else:
        pad = np.float32(np.nan)
    flats = [strided(rows, cols, ss, d, pad) for d in dense]
    active = [True] * R if active is None else list(active)
    put = to_pinned if base == ar.AR_MODE_HOST_STAGED else to_device
    ts = [put(f) if a else None for f, a in zip(flats, active)]
    residual = None
    res_dev = None
    if res_kind is not None:
        res_dense = wl.residual(30_500 + seed, 0, cols if res_kind == "row" else n, dst_type, dist="wide")
        if res_kind == "row":
            residual = res_dense
            rs = 0
        else:
            rpad = (np.uint16(0x7FC0 if dst_type == ar.AR_BF16 else 0x7E00)) if narrow else np.float32(np.nan)
            residual = strided(rows, cols, rs, res_dense, rpad)
        res_dev = to_device(residual)
    ext = span(rows, cols, ds)
    dsts = [GuardedDst(max(ext, 1), 16 if narrow else 32) for _ in range(n_dst)]
    flags = (ar.AR_SRC_WIRE if src_wire else 0) | (0 if all(active) else ar.AR_SRC_INACTIVE_NULL)
    log_case(what)
    ar.ar_reduce_rows(ctx, [g.ptr() for g in dsts], [0 if t is None else t for t in ts], rows, cols, ss, ds,
                      dst_type, wire, mode | flags, residual=res_dev, res_stride=rs)
    torch.cuda.synchronize()
    src_type = wire if (src_wire or narrow) and wire != ar.AR_F32 else None
    init = np.full(ext, SENTINEL16 if narrow else SENTINEL, dtype=np.uint16 if narrow else np.uint32)
    init = init if narrow else init.view(np.float32)
    used = [f if a else None for f, a in zip(flats, active)]
    if all(u is None for u in used):
        used[0] = np.zeros_like(flats[0])
    want = oracle.reduce_rows(used, wire, rows, cols, ss, ds, src_type=src_type, dst_type=dst_type,
                              residual=residual, res_stride=rs, dst_init=init)[0]
    for d, g in enumerate(dsts):
        got = g.result()[:ext]
        if narrow:
            assert_bits_equal16(got, want, dst_type, f"{what} dst {d}")
        else:
            assert_bits_equal(got, want, f"{what} dst {d}")
        # the elements between rows keep the sentinel bits exactly (not just "a NaN")
        mask = np.ones(ext, dtype=bool)
        for i in range(rows):
            mask[i * ds:i * ds + cols] = False
        gb = got.view(np.uint16 if narrow else np.uint32)[mask]
        assert np.all(gb == (SENTINEL16 if narrow else SENTINEL)), f"{what} dst {d}: written between rows"


# (rows, cols, src stride, dst stride, residual stride), strides keep 16-byte row starts for
# both 4- and 2-byte elements
SHAPES = [(7, 520, 528, 536, 544), (33, 64, 72, 64, 80), (3, 4104, 4112, 4104, 4104), (130, 8, 16, 8, 8),
          (1, 1000, 1000, 1000, 1000), (5, 1031, 1040, 1048, 1032)]


@pytest.mark.parametrize("kname", list(KERNEL_CONFIGS))
@pytest.mark.parametrize("mode_name", list(MODES))
def test_rows_every_schedule(kctx, kname, mode_name):
    for i, (rows, cols, ss, ds, rs) in enumerate(SHAPES):
        R = [2, 3, 4, 8, 2, 16][i]
        for wire_name, wire in WIRES.items():
            for src_wire in ([False, True] if wire != ar.AR_F32 else [False]):
                what = (f"rows {kname} {mode_name} {rows}x{cols} strides {ss}/{ds} R={R} wire={wire_name} "
                        f"src_wire={src_wire}")
                run_rows_case(kctx[kname], rows, cols, ss, ds, R, wire, MODES[mode_name], what,
                              src_wire=src_wire, seed=i)


@pytest.mark.parametrize("kname", ["default", "lds_cached"])
@pytest.mark.parametrize("mode_name", list(MODES))
def test_rows_residual_narrow_inactive(kctx, kname, mode_name):
    rng = np.random.default_rng(31)
    for i, (rows, cols, ss, ds, rs) in enumerate(SHAPES):
        R = [2, 3, 4, 8, 2, 16][i]
        for res_kind in ("strided", "row"):
            for dst_name, dst_type in (("f32", ar.AR_F32), ("bf16", ar.AR_BF16), ("f16", ar.AR_F16)):
                wire = ar.AR_BF16 if dst_type == ar.AR_F32 else dst_type
                active = rng.random(R) < 0.75
                what = (f"rows residual={res_kind} dst={dst_name} {kname} {mode_name} {rows}x{cols} R={R} "
                        f"active={active.astype(int).tolist()}")
                run_rows_case(kctx[kname], rows, cols, ss, ds, R, wire, MODES[mode_name], what,
                              dst_type=dst_type, res_kind=res_kind, rs=rs, active=active, seed=100 + i)


# rows of whole wave tiles for the two-rank row-strided kernel: tiles per row a power of two
# (shift) and not (division), dense and padded strides
PAIR_SHAPES = [(9, 512, 520, 528, 536), (17, 1024, 1024, 1100, 1028), (5, 2560, 2568, 2560, 2576),
               (4, 5120, 5200, 5124, 5120), (3, 7168, 7168, 7168, 7172), (100, 4096, 4608, 4352, 4160)]


@pytest.mark.parametrize("mode_name", ["chunked", "single_shot"])
def test_rows_two_rank_kernel(kctx, mode_name):
    for i, (rows, cols, ss, ds, rs) in enumerate(PAIR_SHAPES):
        rc, plan = ar.ar_plan_query_rows([0x10_0000_0000], [0x20_0000_0000, 0x30_0000_0000], rows, cols, ss, ds,
                                         ar.AR_F32, ar.AR_BF16, MODES[mode_name])
        assert rc == ar.AR_OK and plan.stream_kernel == 3, (rows, cols, plan.stream_kernel)
        for wire_name, wire in WIRES.items():
            for res_kind in (None, "strided", "row"):
                what = f"rows two-rank {mode_name} {rows}x{cols} strides {ss}/{ds}/{rs} wire={wire_name} res={res_kind}"
                run_rows_case(kctx["default"], rows, cols, ss, ds, 2, wire, MODES[mode_name], what,
                              res_kind=res_kind, rs=rs, seed=200 + i)
    # in place: the destination is the first source (equal strides)
    rows, cols, st = 6, 1536, 1600
    dense = wl.random_partials(30_300, 0, 2, rows * cols, dist="normal+outliers")
    flats = [strided(rows, cols, st, d, np.float32(np.nan)) for d in dense]
    want = oracle.reduce_rows(flats, ar.AR_BF16, rows, cols, st, st, dst_init=flats[0].copy())[0]
    a, b = to_device(flats[0]), to_device(flats[1])
    log_case(f"rows two-rank in place {rows}x{cols} stride {st}")
    ar.ar_reduce_rows(kctx["default"], [a], [a, b], rows, cols, st, st, ar.AR_F32, ar.AR_BF16, MODES[mode_name])
    torch.cuda.synchronize()
    assert_bits_equal(a.cpu().numpy(), want, "rows two-rank in place")


def test_rows_empty_and_errors(kctx):
    c = kctx["default"]
    dev = [to_device(np.ones(64, dtype=np.float32)) for _ in range(2)]
    out = torch.zeros(64, dtype=torch.float32, device="cuda")
    log_case("rows no-ops and errors")
    assert ar.ar_reduce_rows(c, [out], dev, 0, 16, 16, 16, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED) == ar.AR_OK
    assert ar.ar_reduce_rows(c, [out], dev, 4, 0, 16, 16, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED) == ar.AR_OK
    # rows reaching past the allocation (the library's check; the binding's is switched off)
    assert ar.ar_reduce_rows(c, [out], dev, 4, 16, 1 << 20, 16, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                             check=False, validate=False) == ar.AR_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    ar.ar_reduce_rows(c, [out], dev, 4, 12, 16, 16, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(4, 16)
    assert np.all(got[:, :12] == 2.0) and np.all(got[:, 12:] == 0.0)


def test_rows_prefill_block_full_size(kctx):
    """A 2048 x 4096 block of fp32 partials inside rows of 4608 (the tokens x hidden
    activation of the prefill workload as a view of a wider buffer), bf16 wire, with a
    broadcast bias row; sampled rows against the oracle plus padding checks on all rows."""
    w = wl.WORKLOADS["prefill_bf16"]
    rows, cols, ss, ds = 2048, 4096, 4608, 4352
    dense = wl.partials(w, 0)
    flats = [strided(rows, cols, ss, d, np.float32(np.nan)) for d in dense]
    row = wl.residual(w.case, 7, cols)
    srcs = [to_device(f) for f in flats]
    res = to_device(row)
    ext = span(rows, cols, ds)
    g = GuardedDst(ext)
    log_case("rows prefill block 2048x4096 in 4608 / 4352")
    ar.ar_reduce_rows(kctx["default"], [g.ptr()], srcs, rows, cols, ss, ds, ar.AR_F32, w.wire,
                      ar.AR_MODE_CHUNKED, residual=res, res_stride=0)
    torch.cuda.synchronize()
    got = g.result()[:ext]
    pick = np.unique(np.concatenate([np.arange(8), np.arange(rows - 8, rows),
                                     np.random.default_rng(3).integers(0, rows, 48)]))
    sub = [np.concatenate([f[i * ss:i * ss + cols] for i in pick]) for f in flats]
    want = oracle.reduce(sub, w.wire, residual=np.tile(row, pick.size))[0]
    got_rows = np.concatenate([got[i * ds:i * ds + cols] for i in pick])
    assert_bits_equal(got_rows, want, "prefill block sampled rows")
    pad = got.view(np.uint32).reshape(-1)[:ext]
    for i in range(rows - 1):
        assert np.all(pad[i * ds + cols:(i + 1) * ds] == SENTINEL), f"row {i}: written between rows"
