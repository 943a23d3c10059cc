"""A seeded random sweep over the whole call space, bit for bit against the
oracle, through the C ABI.

Each case draws a rank count, a length (ragged against every tile and chunk
size), the wire and destination types, whether the sources hold the wire type
already, the schedule, a residual (none, element-wise, or a broadcast row),
inactive ranks, exact in-place use, and a context configuration (kernel
family, store policy, host path, grid size, chunk sizes, copy slots, XCD
placement, occupancy hold).  A quarter of the cases are drawn so that the
two-rank kernels take them (binary32 with each residual form, and 16-bit).
The parametrised tests cover each feature on its own; this sweep covers them
in combination.  Cases are generated from a fixed seed, so a failure names a
case that reruns identically.  The CPU half checks that every drawn call is
valid and which kernel each plan picks.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import mixed_precision_partial_amd as ar
import oracle
import workloads as wl
from gpu_util import GuardedDst, assert_bits_equal, assert_bits_equal16, log_case, to_device, to_pinned

SCHEDULES = [ar.AR_MODE_SINGLE_SHOT, ar.AR_MODE_CHUNKED, ar.AR_MODE_RS_BCAST, ar.AR_MODE_HOST_STAGED,
             ar.AR_MODE_AUTO]
N_CASES = 400
BATCH = 25
# MPP_RANDOM_CASES="start:stop" runs another range of the same generator
# (e.g. MPP_RANDOM_CASES=400:3400); the default is cases 0-399
_range = os.environ.get("MPP_RANDOM_CASES", "")
CASE_START, CASE_STOP = (int(x) for x in _range.split(":")) if _range else (0, N_CASES)


def draw_case(i: int) -> dict:
    rng = np.random.default_rng(np.random.SeedSequence([40_000, i]))
    R = int(rng.choice([2, 2, 3, 4, 5, 7, 8, 9, 16]))
    narrow = rng.random() < 0.2
    if narrow:
        wire = int(rng.choice([ar.AR_BF16, ar.AR_F16]))
        dst_type, src_wire = wire, True
    else:
        wire = int(rng.choice([ar.AR_F32, ar.AR_BF16, ar.AR_BF16, ar.AR_F16]))
        dst_type = ar.AR_F32
        src_wire = wire != ar.AR_F32 and rng.random() < 0.35
    res_form = rng.choice(["none", "none", "elementwise", "row"])
    if res_form == "row":
        L = 8 * int(rng.integers(1, 700))
        n = L * int(rng.integers(1, max(2, (1 << 21) // L)))
    else:
        L = 0
        n = int(np.exp(rng.uniform(0.0, np.log(1 << 21))))
    mode = int(rng.choice(SCHEDULES))
    inactive = rng.random(R) < 0.3 if rng.random() < 0.2 else np.zeros(R, dtype=bool)
    in_place = (not narrow and not src_wire and res_form != "row" and
                mode in (ar.AR_MODE_SINGLE_SHOT, ar.AR_MODE_CHUNKED) and not inactive[0] and rng.random() < 0.5)
    cfg = {
        "stream_kernel": int(rng.choice([0, 0, 1, 2])),
        "store_policy": int(rng.choice([0, 0, 1, 2])),
        "host_path": int(rng.choice([0, 1, 2])),
        "grid_wgs": int(rng.choice([0, 0, 0, 1, 7, 64, 300])),
        "chunk_bytes": int(rng.choice([0, 0, 4096, 65536])),
        "host_chunk_bytes": int(rng.choice([0, 0, 1 << 14, 1 << 16])),
        "host_slots": int(rng.choice([0, 1, 2])),
        # XCD placement runs: automatic, none, and runs from one workgroup to 4 Mi elements
        "xcd_run_elems": int(rng.choice([0, 0, 1, 512, 4096, 1 << 15, 1 << 17, 1 << 22])),
        # the occupancy hold, from a generator of its own so the other draws stay as they were
        "occupancy_hold": int(np.random.default_rng([40_001, i]).choice([0, 0, 0, -1, 2, 6, 10, 14, 18, 32])),
    }
    dist = str(rng.choice(["wide", "normal", "normal+outliers"]))
    # a quarter of the cases are redrawn as calls the two-rank kernels take, from a generator of
    # their own so the other draws stay as they were: two active ranks, single-shot, chunked or
    # automatic schedule, library-chosen kernel and grid, kept stores; binary32 partials into
    # binary32 with the drawn residual form, or two 16-bit partials into their own type without one
    pr = np.random.default_rng([40_002, i])
    if pr.random() < 0.25:
        R, inactive = 2, np.zeros(2, dtype=bool)
        mode = int(pr.choice([ar.AR_MODE_SINGLE_SHOT, ar.AR_MODE_CHUNKED, ar.AR_MODE_AUTO]))
        cfg.update(stream_kernel=0, grid_wgs=0, store_policy=int(pr.choice([0, 1])))
        if narrow:
            res_form, L = "none", 0
        src_wire = False if not narrow else src_wire
        in_place = (not narrow and res_form != "row" and mode != ar.AR_MODE_AUTO and pr.random() < 0.3)
    return dict(i=i, R=R, n=n, wire=wire, dst_type=dst_type, src_wire=src_wire, res_form=str(res_form), L=L,
                mode=mode, inactive=[bool(x) for x in inactive], in_place=bool(in_place), cfg=cfg, dist=dist)


def plan_of(c: dict):
    """The library's plan for the case's call (host-only; far-apart fake addresses)."""
    base = [0x20_0000_0000 + k * 0x4_0000_0000 for k in range(40)]
    R = c["R"]
    n_dst = R if c["mode"] == ar.AR_MODE_RS_BCAST else 1
    srcs = [0 if off else base[k] for k, off in enumerate(c["inactive"])]
    dsts = [srcs[0]] if c["in_place"] else base[20:20 + n_dst]
    flags = (ar.AR_SRC_WIRE if c["src_wire"] else 0) | (ar.AR_SRC_INACTIVE_NULL if any(c["inactive"]) else 0)
    host = c["mode"] == ar.AR_MODE_HOST_STAGED
    if c["res_form"] == "none":
        return ar.ar_plan_query(dsts, srcs, c["n"], c["dst_type"], c["wire"], c["mode"] | flags,
                                srcs_on_host=host, config=c["cfg"], R=R)
    rl = c["n"] if c["res_form"] == "elementwise" else c["L"]
    return ar.ar_plan_query_add(dsts, srcs, c["n"], c["dst_type"], c["wire"], c["mode"] | flags, base[39], rl,
                                srcs_on_host=host, config=c["cfg"], R=R)


def run_case(c: dict) -> None:
    R, n, wire, dst_type = c["R"], c["n"], c["wire"], c["dst_type"]
    narrow = dst_type != ar.AR_F32
    what = (f"random case {c['i']}: R={R} n={n} wire={wire} dst={dst_type} src_wire={c['src_wire']} "
            f"mode={c['mode']} residual={c['res_form']} L={c['L']} inactive={c['inactive']} "
            f"in_place={c['in_place']} cfg={c['cfg']}")
    if narrow:
        srcs = wl.random_narrow(40_100 + c["i"], 0, R, n, dst_type, dist="wide")
    else:
        srcs = wl.random_partials(40_100 + c["i"], 0, R, n, dist=c["dist"])
        if c["src_wire"]:
            srcs = [wl.as_wire_typed(s, wire) for s in srcs]
    residual = None
    if c["res_form"] == "elementwise":
        residual = wl.residual(40_200 + c["i"], 0, n, dst_type, dist="wide")
    elif c["res_form"] == "row":
        residual = wl.residual(40_200 + c["i"], 0, c["L"], dst_type, dist="wide")
    active = [not x for x in c["inactive"]]
    host = c["mode"] == ar.AR_MODE_HOST_STAGED
    put = to_pinned if host else to_device
    ts = [put(s) if a else None for s, a in zip(srcs, active)]
    base = c["mode"]
    n_dst = R if base == ar.AR_MODE_RS_BCAST else 1
    flags = (ar.AR_SRC_WIRE if c["src_wire"] else 0) | (0 if all(active) else ar.AR_SRC_INACTIVE_NULL)
    ctx = ar.ar_init(0, c["cfg"])
    try:
        log_case(what)
        if c["in_place"]:
            dsts = None
            dptrs = [ts[0]]
        else:
            dsts = [GuardedDst(n, 16 if narrow else 32) for _ in range(n_dst)]
            dptrs = [d.ptr() for d in dsts]
        ptrs = [0 if t is None else t for t in ts]
        if residual is None:
            ar.ar_reduce(ctx, dptrs, ptrs, n, dst_type, wire, base | flags)
        else:
            ar.ar_reduce_add(ctx, dptrs, ptrs, n, dst_type, wire, base | flags, to_device(residual), residual.size)
        torch.cuda.synchronize()
    finally:
        ar.ar_free(ctx)
    src_type = wire if (c["src_wire"] or narrow) and wire != ar.AR_F32 else None
    used = [s if a else None for s, a in zip(srcs, active)]
    want = oracle.reduce(used, wire, src_type=src_type, dst_type=dst_type, residual=residual, n=n)[0]
    if c["in_place"]:
        assert_bits_equal(ts[0].cpu().numpy(), want, what + " (in place)")
        return
    for d, g in enumerate(dsts):
        got = g.result()
        if narrow:
            assert_bits_equal16(got, want, dst_type, f"{what} dst {d}")
        else:
            assert_bits_equal(got, want, f"{what} dst {d}")


def test_case_generator_is_deterministic_and_varied():
    cases = [draw_case(i) for i in range(N_CASES)]
    assert cases[:3] == [draw_case(i) for i in range(3)]
    seen = {(c["mode"], c["res_form"], c["dst_type"] != ar.AR_F32) for c in cases}
    assert len(seen) >= 20
    assert any(c["in_place"] for c in cases) and any(any(c["inactive"]) for c in cases)
    # every plan is valid; the two-rank kernels (binary32, with each residual form, and 16-bit)
    # occur beside the single-shot and both streaming families
    kinds = []
    for c in cases:
        rc, plan = plan_of(c)
        assert rc == ar.AR_OK, (c, ar.ar_status_str(rc))
        kinds.append((int(plan.stream_kernel), int(plan.dst_bytes), c["res_form"]))
    kernels = {k for k, _, _ in kinds}
    assert {0, 1, 2, 3, 4} <= kernels
    pair32 = [r for k, b, r in kinds if k == 3 and b == 4]
    assert len(pair32) >= 40 and {"none", "elementwise", "row"} <= set(pair32)
    assert sum(1 for k, b, _ in kinds if k == 3 and b == 2) >= 5


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


@pytest.mark.gpu
@pytest.mark.parametrize("start", range(CASE_START, CASE_STOP, BATCH))
def test_random_sweep(gpu, start):
    for i in range(start, min(start + BATCH, CASE_STOP)):
        run_case(draw_case(i))
    torch.cuda.empty_cache()
