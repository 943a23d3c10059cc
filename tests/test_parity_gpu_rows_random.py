"""A seeded random sweep over row-strided calls (``ar_reduce_rows``), bit for bit
against the oracle, through the C ABI.

Each case draws a rank count, a row count, a row length (whole 512-element
wave tiles, multiples of 8, or any length), padded or dense strides for the
sources, the destination and a strided residual, the wire and destination
types, 16-bit sources, a residual (none, strided, or one broadcast row),
inactive ranks, the schedule and a context configuration (kernel family,
store policy, host path, grid size, chunk sizes, copy slots, XCD placement,
occupancy hold).
The parametrised row tests cover each feature on its own; this sweep covers
them in combination, including the two-rank row-strided kernel under every
configuration that leaves it eligible.  Sources carry NaN between rows and
destinations a sentinel that must survive there (``run_rows_case``).
"""
from __future__ import annotations

import numpy as np
import pytest

import mixed_precision_partial_amd as ar
from test_parity_gpu_rows import run_rows_case

N_CASES = 160
BATCH = 20
MODES = [ar.AR_MODE_SINGLE_SHOT, ar.AR_MODE_CHUNKED, ar.AR_MODE_RS_BCAST, ar.AR_MODE_HOST_STAGED,
         ar.AR_MODE_AUTO]
MAX_ELEMS = 1 << 22        # rows x source stride x ranks, to keep a case well under a second


def round8(x: int) -> int:
    return (x + 7) // 8 * 8


def draw_rows_case(i: int) -> dict:
    rng = np.random.default_rng(np.random.SeedSequence([41_000, i]))
    R = int(rng.choice([2, 2, 2, 3, 4, 8, 16]))
    narrow = rng.random() < 0.2
    if narrow:
        wire = int(rng.choice([ar.AR_BF16, ar.AR_F16]))
        dst_type, src_wire = wire, False
    else:
        wire = int(rng.choice([ar.AR_F32, ar.AR_BF16, ar.AR_BF16, ar.AR_F16]))
        dst_type = ar.AR_F32
        src_wire = wire != ar.AR_F32 and rng.random() < 0.35
    u = rng.random()
    if u < 0.4:
        cols = 512 * int(rng.integers(1, 17))        # whole wave tiles
    elif u < 0.7:
        cols = 8 * int(rng.integers(1, 700))
    else:
        cols = int(rng.integers(1, 3000))
    # strides in elements keep every row start 16-byte aligned for 2- and 4-byte elements
    pads = [0, 0, 8, 16, 72, 512]
    ss, ds, rs = (round8(cols) + int(rng.choice(pads)) for _ in range(3))
    rows = int(np.exp(rng.uniform(0.0, np.log(400))))
    while rows > 1 and rows * ss * R > MAX_ELEMS:
        rows //= 2
    res_form = str(rng.choice(["none", "none", "strided", "row"]))
    inactive = rng.random(R) < 0.3 if rng.random() < 0.2 else np.zeros(R, dtype=bool)
    cfg = {
        "stream_kernel": int(rng.choice([0, 0, 0, 1, 2])),
        "store_policy": int(rng.choice([0, 0, 1, 2])),
        "host_path": int(rng.choice([0, 1, 2])),
        "grid_wgs": int(rng.choice([0, 0, 0, 1, 7, 64, 300])),
        "chunk_bytes": int(rng.choice([0, 0, 4096, 65536])),
        "host_chunk_bytes": int(rng.choice([0, 0, 1 << 14, 1 << 16])),
        "host_slots": int(rng.choice([0, 1, 2])),
        "xcd_run_elems": int(rng.choice([0, 0, 1, 512, 4096, 1 << 15, 1 << 17])),
        "occupancy_hold": int(np.random.default_rng([41_001, i]).choice([0, 0, 0, -1, 2, 6, 10, 14, 18, 32])),
    }
    mode = int(rng.choice(MODES))
    if rng.random() < 0.25:
        # a call the two-rank row-strided kernel takes: two active fp32 partials into
        # fp32, rows of whole wave tiles, single-shot or chunked, library-chosen kernel
        # and grid, kept stores; everything else stays as drawn
        R, narrow, src_wire, dst_type = 2, False, False, ar.AR_F32
        inactive = np.zeros(R, dtype=bool)
        cols = 512 * max(1, cols // 512)
        ss, ds, rs = (cols + int(rng.choice(pads)) for _ in range(3))
        rows = int(np.exp(rng.uniform(0.0, np.log(400))))
        while rows > 1 and rows * ss * R > MAX_ELEMS:
            rows //= 2
        mode = int(rng.choice([ar.AR_MODE_SINGLE_SHOT, ar.AR_MODE_CHUNKED, ar.AR_MODE_AUTO]))
        cfg.update(stream_kernel=0, grid_wgs=0, store_policy=int(rng.choice([0, 1])))
    return dict(i=i, R=R, rows=rows, cols=cols, ss=ss, ds=ds, rs=rs, wire=wire, dst_type=dst_type,
                src_wire=src_wire, res_form=res_form, inactive=[bool(x) for x in inactive],
                mode=mode, cfg=cfg)


def plan_of(c: dict):
    """The library's plan for the case's call (host-only; far-apart fake addresses)."""
    base = [0x20_0000_0000 + k * 0x4_0000_0000 for k in range(40)]
    R = c["R"]
    n_dst = R if c["mode"] == ar.AR_MODE_RS_BCAST else 1
    srcs = [0 if off else base[k] for k, off in enumerate(c["inactive"])]
    dsts = base[20:20 + n_dst]
    flags = (ar.AR_SRC_WIRE if c["src_wire"] else 0) | (ar.AR_SRC_INACTIVE_NULL if any(c["inactive"]) else 0)
    residual = None if c["res_form"] == "none" else base[39]
    return ar.ar_plan_query_rows(dsts, srcs, c["rows"], c["cols"], c["ss"], c["ds"], c["dst_type"], c["wire"],
                                 c["mode"] | flags, residual=residual,
                                 res_stride=c["rs"] if c["res_form"] == "strided" else 0,
                                 srcs_on_host=c["mode"] == ar.AR_MODE_HOST_STAGED, config=c["cfg"], R=R)


def test_rows_case_generator_is_valid_and_varied():
    cases = [draw_rows_case(i) for i in range(N_CASES)]
    assert cases[:3] == [draw_rows_case(i) for i in range(3)]
    kernels = []
    for c in cases:
        rc, plan = plan_of(c)
        assert rc == ar.AR_OK, (c, ar.ar_status_str(rc))
        kernels.append(int(plan.stream_kernel))
    # the two-rank row-strided kernel, both streaming families and the single-shot kernel all occur
    assert kernels.count(3) >= 8 and {0, 1, 2, 3} <= set(kernels)
    assert len({(c["mode"], c["res_form"], c["dst_type"] != ar.AR_F32) for c in cases}) >= 20
    assert any(any(c["inactive"]) for c in cases) and any(c["cols"] % 8 for c in cases)


@pytest.fixture(scope="module")
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


@pytest.mark.gpu
@pytest.mark.parametrize("start", range(0, N_CASES, BATCH))
def test_rows_random_sweep(gpu, start):
    import torch

    for i in range(start, min(start + BATCH, N_CASES)):
        c = draw_rows_case(i)
        what = (f"rows random case {i}: R={c['R']} {c['rows']}x{c['cols']} strides {c['ss']}/{c['ds']}/{c['rs']} "
                f"wire={c['wire']} dst={c['dst_type']} src_wire={c['src_wire']} mode={c['mode']} "
                f"residual={c['res_form']} inactive={c['inactive']} cfg={c['cfg']}")
        ctx = ar.ar_init(0, c["cfg"])
        try:
            run_rows_case(ctx, c["rows"], c["cols"], c["ss"], c["ds"], c["R"], c["wire"], c["mode"], what,
                          dst_type=c["dst_type"], src_wire=c["src_wire"],
                          res_kind=None if c["res_form"] == "none" else c["res_form"], rs=c["rs"],
                          active=[not x for x in c["inactive"]], seed=2_000 + i)
        finally:
            torch.cuda.synchronize()
            ar.ar_free(ctx)
    torch.cuda.empty_cache()
