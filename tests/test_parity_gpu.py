"""HIP path against the CPU oracle, bit for bit (0 ulp; NaN compared as NaN).

Every call goes through the C ABI (``libmpp_ar.so``) via the thin binding.
The five workload shapes run at full size; tails, edge values, every schedule,
every wire type, source widths, in-place use, guard bands and error paths run
at sizes the oracle finishes in seconds.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixed_precision_partial_amd as ar
import oracle
import workloads as wl
from gpu_util import (GuardedDst, assert_bits_equal, assert_bits_equal16, assert_no_sentinel, log_case,
                      oracle_result, to_device, to_pinned)

pytestmark = pytest.mark.gpu

MODES = {
    "single_shot": ar.AR_MODE_SINGLE_SHOT,
    "chunked": ar.AR_MODE_CHUNKED,
    "rs_bcast": ar.AR_MODE_RS_BCAST,
    "host_staged": ar.AR_MODE_HOST_STAGED,
}
WIRES = {"f32": ar.AR_F32, "bf16": ar.AR_BF16, "f16": ar.AR_F16}


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    c = ar.ar_init(0)
    yield c
    torch.cuda.synchronize()
    ar.ar_free(c)


def run_case(ctx, srcs_np, wire, mode, src_wire=False, R=None, config_ctx=None, guarded=True):
    """Run one reduce on the GPU and return the list of destination arrays."""
    c = config_ctx or ctx
    R = len(srcs_np)
    n = srcs_np[0].size
    base = mode & ar.AR_MODE_MASK
    n_dst = R if base == ar.AR_MODE_RS_BCAST else 1
    if src_wire:
        srcs_np = [wl.as_wire_typed(s, wire) if s.dtype == np.float32 else s for s in srcs_np]
    if base == ar.AR_MODE_HOST_STAGED:
        srcs_t = [to_pinned(s) for s in srcs_np]
    else:
        srcs_t = [to_device(s) for s in srcs_np]
    dsts = [GuardedDst(n) for _ in range(n_dst)]
    flags = ar.AR_SRC_WIRE if src_wire else 0
    ar.ar_reduce(c, [d.ptr() for d in dsts], srcs_t, n, ar.AR_F32, wire, mode | flags)
    torch.cuda.synchronize()
    return [d.result() for d in dsts], srcs_np


def check_against_oracle(ctx, srcs_np, wire, mode, src_wire=False, what="", config_ctx=None):
    outs, used = run_case(ctx, srcs_np, wire, mode, src_wire, config_ctx=config_ctx)
    src_type = wire if src_wire and wire != ar.AR_F32 else None
    want = oracle_result(used, wire, src_type=src_type)
    for d, got in enumerate(outs):
        assert_bits_equal(got, want, f"{what} dst {d}")
    return outs, want


# --------------------------------------------------------------------------
# the five workloads at full size
# --------------------------------------------------------------------------

def test_decode_fp32_wire(ctx):
    w = wl.WORKLOADS["decode_f32"]
    log_case(f"decode_f32 R={w.R} n={w.n} single_shot")
    srcs = wl.partials(w, 0)
    outs, want = check_against_oracle(ctx, srcs, w.wire, ar.AR_MODE_SINGLE_SHOT, what="decode_f32")
    # fp32 wire: the plain ordered float32 sum
    assert_bits_equal(outs[0], srcs[0] + srcs[1], "decode_f32 vs float32 sum")


def test_decode_bf16_wire_all_calls(ctx):
    """10,000 sequential single-shot calls, each with fresh seeded data; every output checked."""
    w = wl.WORKLOADS["decode_bf16"]
    log_case(f"decode_bf16 R={w.R} n={w.n} calls={w.calls}")
    n, calls = w.n, w.calls
    host = np.empty((calls, w.R, n), dtype=np.float32)
    for c in range(calls):
        for r, p in enumerate(wl.partials(w, c)):
            host[c, r] = p
    dev = torch.from_numpy(host).cuda()
    out = torch.empty((calls, n), dtype=torch.float32, device="cuda")
    esz = 4
    base_in, base_out = dev.data_ptr(), out.data_ptr()
    for c in range(calls):
        srcs = [base_in + (c * w.R + r) * n * esz for r in range(w.R)]
        ar.ar_reduce(ctx, [base_out + c * n * esz], srcs, n, ar.AR_F32, w.wire, ar.AR_MODE_SINGLE_SHOT)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.reduce([host[:, r, :].ravel() for r in range(w.R)], w.wire)[0]
    assert_bits_equal(got.ravel(), want, "decode_bf16 all calls")


def test_prefill_bf16_chunked(ctx):
    w = wl.WORKLOADS["prefill_bf16"]
    log_case(f"prefill_bf16 R={w.R} n={w.n} chunked 4MiB")
    srcs = wl.partials(w, 0)
    check_against_oracle(ctx, srcs, w.wire, ar.AR_MODE_CHUNKED, what="prefill_bf16")


def test_prefill_bf16_auto_selects_chunked(ctx):
    w = wl.WORKLOADS["prefill_bf16"]
    rc, plan = ar.ar_plan_query([0x10_0000_0000], [0x20_0000_0000, 0x30_0000_0000], w.n,
                                ar.AR_F32, w.wire, ar.AR_MODE_AUTO)
    assert rc == ar.AR_OK and plan.mode == ar.AR_MODE_CHUNKED and plan.n_chunks == 4
    log_case("prefill_bf16 auto")
    srcs = wl.partials(w, 1)
    check_against_oracle(ctx, srcs, w.wire, ar.AR_MODE_AUTO, what="prefill_bf16 auto")


def test_slice_bcast_f16(ctx):
    w = wl.WORKLOADS["slice_bcast_f16"]
    log_case(f"slice_bcast_f16 R={w.R} n={w.n} rs_bcast")
    srcs = wl.partials(w, 0)
    outs, want = check_against_oracle(ctx, srcs, w.wire, ar.AR_MODE_RS_BCAST, what="slice_bcast_f16")
    assert len(outs) == 4
    for d in range(1, 4):
        assert np.array_equal(outs[0].view(np.uint32), outs[d].view(np.uint32))


def test_host_staged_bf16_and_hbm(ctx):
    """R=8, 8192 x 8192: wire-typed partials in pinned host memory, then the same shape from HBM."""
    w = wl.WORKLOADS["host_staged_bf16"]
    n = w.n
    log_case(f"host_staged_bf16 R={w.R} n={n}")
    srcs32 = wl.partials(w, 0)
    pre = [wl.as_wire_typed(s, w.wire) for s in srcs32]
    want_wire = oracle.reduce(pre, w.wire, src_type=w.wire)[0]
    outs, _ = run_case(ctx, pre, w.wire, ar.AR_MODE_HOST_STAGED, src_wire=True)
    assert_bits_equal(outs[0], want_wire, "host_staged bf16")
    log_case("host_staged_bf16 copy-engine pipeline")
    c = ar.ar_init(0, {"host_path": 1})
    try:
        outs, _ = run_case(ctx, pre, w.wire, ar.AR_MODE_HOST_STAGED, src_wire=True, config_ctx=c)
        assert_bits_equal(outs[0], want_wire, "host_staged bf16 copy engine")
    finally:
        torch.cuda.synchronize()
        ar.ar_free(c)
    log_case("host_staged_bf16 same shape from HBM, wire-typed sources")
    outs, _ = run_case(ctx, pre, w.wire, ar.AR_MODE_CHUNKED, src_wire=True)
    assert_bits_equal(outs[0], want_wire, "hbm chunked bf16 sources")
    log_case("host_staged_bf16 same shape from HBM, fp32 sources")
    want32 = oracle.reduce(srcs32, w.wire)[0]
    outs, _ = run_case(ctx, srcs32, w.wire, ar.AR_MODE_CHUNKED)
    assert_bits_equal(outs[0], want32, "hbm chunked fp32 sources")


# --------------------------------------------------------------------------
# tails, rank counts, wire types, source widths, schedules
# --------------------------------------------------------------------------

TAIL_N = [1, 3, 7, 8, 9, 63, 64, 65, 511, 512, 513, 1023, 1025, 2047, 2048, 2049, 4095, 4097,
          8191, 8193, 12289, 65537, 131071]


# Kernel instances: register / LDS-staged streaming family x cached / streaming stores
# (host-staged calls in the first four go through the copy-engine pipeline)
KERNEL_CONFIGS = {
    "reg_cached": {"stream_kernel": 1, "store_policy": 1, "host_path": 1},
    "reg_streaming": {"stream_kernel": 1, "store_policy": 2, "host_path": 1},
    "lds_cached": {"stream_kernel": 2, "store_policy": 1, "host_path": 1},
    "lds_streaming": {"stream_kernel": 2, "store_policy": 2, "host_path": 1},
    "host_direct": {"host_path": 2},
}


@pytest.fixture(scope="module")
def kctx():
    """One context per kernel-instance configuration."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ctxs = {k: ar.ar_init(0, v) for k, v in KERNEL_CONFIGS.items()}
    yield ctxs
    torch.cuda.synchronize()
    for c in ctxs.values():
        ar.ar_free(c)


@pytest.mark.parametrize("mode_name", ["single_shot", "chunked", "rs_bcast"])
def test_tails_all_wires_and_widths(ctx, mode_name):
    mode = MODES[mode_name]
    rng = np.random.default_rng(1234)
    for i, n in enumerate(TAIL_N):
        R = int(rng.choice([2, 3, 4, 5, 8, 9, 16]))
        for wire_name, wire in WIRES.items():
            for src_wire in ([False, True] if wire != ar.AR_F32 else [False]):
                what = f"{mode_name} n={n} R={R} wire={wire_name} src_wire={src_wire}"
                log_case(what)
                srcs = wl.random_partials(2000 + i, wire, R, n, dist="wide")
                check_against_oracle(ctx, srcs, wire, mode, src_wire, what)


@pytest.mark.parametrize("kname", list(KERNEL_CONFIGS))
@pytest.mark.parametrize("mode_name", ["chunked", "rs_bcast", "host_staged"])
def test_every_kernel_instance(kctx, kname, mode_name):
    """Both streaming families x both store policies x chunk / slice ranges, every rank
    bucket, both source widths, ragged tails."""
    mode = MODES[mode_name]
    cases = [(2, 70_001), (3, 4097), (4, 131_072 + 515), (7, 9_000), (8, 65_536 + 1), (13, 2_049),
             (16, 20_480 + 3)]
    for i, (R, n) in enumerate(cases):
        for wire_name, wire in WIRES.items():
            for src_wire in ([False, True] if wire != ar.AR_F32 else [False]):
                what = f"{kname} {mode_name} R={R} n={n} wire={wire_name} src_wire={src_wire}"
                log_case(what)
                srcs = wl.random_partials(8000 + i, wire, R, n, dist="wide")
                check_against_oracle(kctx[kname], srcs, wire, mode, src_wire, what)


PAIR_N = [1, 2, 63, 64, 511, 512, 513, 1023, 2047, 2048, 2049, 4097, 131_072 + 511, (1 << 20) + 3,
          2048 * 4096]


def test_two_rank_contiguous_kernel(ctx):
    """The two-rank contiguous kernel (plan stream_kernel 3): every wire type, tiles with and
    without a remainder, grids below and above one placement run, the prefill size, in place."""
    for i, n in enumerate(PAIR_N):
        # chunked at every size; single-shot (the decode form) at the smaller ones
        modes = [("chunked", ar.AR_MODE_CHUNKED)] + ([("single_shot", ar.AR_MODE_SINGLE_SHOT)] if n <= 4097 else [])
        for mode_name, mode in modes:
            rc, plan = ar.ar_plan_query([0x10_0000_0000], [0x20_0000_0000, 0x30_0000_0000], n, ar.AR_F32,
                                        ar.AR_BF16, mode)
            assert rc == ar.AR_OK and plan.stream_kernel == 3, (n, mode_name, plan.stream_kernel)
            for wire_name, wire in WIRES.items():
                what = f"pair {mode_name} n={n} wire={wire_name}"
                log_case(what)
                srcs = wl.random_partials(9100 + i, wire, 2, n, dist="wide")
                check_against_oracle(ctx, srcs, wire, mode, what=what)
    # in place: the destination is the first source
    n = (1 << 18) + 77
    srcs = wl.random_partials(9199, 0, 2, n, dist="normal+outliers")
    want = oracle_result(srcs, ar.AR_BF16)
    a, b = to_device(srcs[0]), to_device(srcs[1])
    log_case(f"pair in place n={n}")
    ar.ar_reduce(ctx, [a], [a, b], n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED)
    torch.cuda.synchronize()
    assert_bits_equal(a.cpu().numpy(), want, "pair in place")


def test_small_chunks_many_ranges(ctx):
    """Chunk plan with many chunks and a ragged last chunk."""
    cfg = ar.ar_init(0, {"chunk_bytes": 4096})
    try:
        for n in [2048 * 3 + 17, 100_003, 1 << 18]:
            for wire in (ar.AR_BF16, ar.AR_F16, ar.AR_F32):
                what = f"chunked 4 KiB chunks n={n} wire={wire}"
                log_case(what)
                srcs = wl.random_partials(3000, n % 97, 3, n, dist="normal")
                check_against_oracle(ctx, srcs, wire, ar.AR_MODE_CHUNKED, what=what, config_ctx=cfg)
    finally:
        torch.cuda.synchronize()
        ar.ar_free(cfg)


# --------------------------------------------------------------------------
# edge values and exact rounding
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mode_name", ["single_shot", "chunked", "rs_bcast", "host_staged"])
def test_edge_value_pairs(ctx, mode_name):
    """Every ordered pair (R=2) and a grid of triples (R=3) of edge values, NaN included."""
    g = np.concatenate([wl.special_values(), wl.nan_values()])
    a, b = np.meshgrid(g, g, indexing="ij")
    pairs = [a.ravel().copy(), b.ravel().copy()]
    g3 = g[::3]
    x, y, z = np.meshgrid(g3, g3, g3, indexing="ij")
    triples = [x.ravel().copy(), y.ravel().copy(), z.ravel().copy()]
    for wire_name, wire in WIRES.items():
        for srcs in (pairs, triples):
            what = f"edge {mode_name} R={len(srcs)} wire={wire_name} n={srcs[0].size}"
            log_case(what)
            check_against_oracle(ctx, srcs, wire, MODES[mode_name], what=what)


@pytest.mark.parametrize("wire_name", ["bf16", "f16"])
def test_rounding_sampled_patterns(ctx, wire_name):
    """round_W over every upper 16 bits x 64 lower patterns (4 Mi inputs): src1 = -0 keeps
    x + (-0) == x exactly, so the destination is the widened wire value of src0."""
    wire = WIRES[wire_name]
    rng = np.random.default_rng(99)
    hi = np.repeat(np.arange(1 << 16, dtype=np.uint32) << 16, 64)
    lo = rng.integers(0, 1 << 16, hi.size, dtype=np.uint32)
    lo[::64] = 0x8000            # exact ties for bf16
    lo[1::64] = 0x1000 & 0xFFFF  # ties for f16 in the low bits
    x = (hi | lo).view(np.float32)
    negz = np.full(x.size, -0.0, dtype=np.float32)
    log_case(f"rounding sampled {wire_name} n={x.size}")
    check_against_oracle(ctx, [x, negz], wire, ar.AR_MODE_CHUNKED, what=f"rounding {wire_name}")


# --------------------------------------------------------------------------
# schedules agree, in place, streams, host-staged pipelining
# --------------------------------------------------------------------------

def test_all_schedules_byte_identical(ctx):
    n = 300_001
    srcs = wl.random_partials(4000, 0, 5, n, dist="normal+outliers")
    results = {}
    for name in ("single_shot", "chunked", "rs_bcast", "host_staged"):
        log_case(f"schedule {name} n={n}")
        outs, _ = run_case(ctx, srcs, ar.AR_BF16, MODES[name])
        results[name] = outs
    ref = results["chunked"][0].view(np.uint32)
    for name, outs in results.items():
        for d, o in enumerate(outs):
            assert np.array_equal(o.view(np.uint32), ref), f"{name} dst {d} differs from chunked"
    assert_bits_equal(results["chunked"][0], oracle_result(srcs, ar.AR_BF16), "schedules vs oracle")


def test_in_place(ctx):
    n = 70_001
    for mode_name in ("single_shot", "chunked", "rs_bcast"):
        R = 4
        srcs = wl.random_partials(5000, 1, R, n, dist="wide")
        want = oracle_result(srcs, ar.AR_BF16)
        dev = [to_device(s) for s in srcs]
        base = MODES[mode_name]
        dsts = dev if base == ar.AR_MODE_RS_BCAST else [dev[0]]
        log_case(f"in place {mode_name}")
        ar.ar_reduce(ctx, dsts, dev, n, ar.AR_F32, ar.AR_BF16, base)
        torch.cuda.synchronize()
        for d in dsts:
            assert_bits_equal(d.cpu().numpy(), want, f"in place {mode_name}")


def test_aliased_sources(ctx):
    """The same buffer passed for several ranks (sources are read only, so aliasing them
    is allowed): the fold sees that partial once per rank that names it."""
    n = 50_003
    a, b = wl.random_partials(5100, 0, 2, n, dist="wide")
    dev_a, dev_b = to_device(a), to_device(b)
    for mode_name in ("single_shot", "chunked", "rs_bcast"):
        base = MODES[mode_name]
        srcs = [dev_a, dev_b, dev_a, dev_a]
        want = oracle_result([a, b, a, a], ar.AR_F16)
        dsts = [torch.empty(n, device="cuda") for _ in range(4 if base == ar.AR_MODE_RS_BCAST else 1)]
        log_case(f"aliased sources {mode_name}")
        ar.ar_reduce(ctx, dsts, srcs, n, ar.AR_F32, ar.AR_F16, base)
        torch.cuda.synchronize()
        for d in dsts:
            assert_bits_equal(d.cpu().numpy(), want, f"aliased sources {mode_name}")


def test_non_default_stream(ctx):
    n = 1 << 20
    srcs = wl.random_partials(6000, 0, 2, n)
    dev = [to_device(s) for s in srcs]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    log_case("non-default stream")
    with torch.cuda.stream(s):
        ar.ar_reduce(ctx, [out], dev, n, ar.AR_F32, ar.AR_F16, ar.AR_MODE_CHUNKED, stream=s)
    s.synchronize()
    assert_bits_equal(out.cpu().numpy(), oracle_result(srcs, ar.AR_F16), "side stream")


@pytest.mark.parametrize("slots", [1, 2, 4])
def test_host_staged_back_to_back(ctx, slots):
    """Several host-staged calls enqueued without a sync in between, small chunks,
    few slots: a missing wait on slot reuse would mix chunks of different calls."""
    c = ar.ar_init(0, {"host_slots": slots, "host_chunk_bytes": 1 << 16, "host_path": 1})
    try:
        n, R, calls = 200_000 + slots, 3, 4
        inputs = [wl.random_partials(7000 + slots, k, R, n) for k in range(calls)]
        pinned = [[to_pinned(s) for s in srcs] for srcs in inputs]
        outs = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(calls)]
        log_case(f"host staged back to back slots={slots}")
        for k in range(calls):
            ar.ar_reduce(c, [outs[k]], pinned[k], n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_HOST_STAGED)
        torch.cuda.synchronize()
        for k in range(calls):
            assert_bits_equal(outs[k].cpu().numpy(), oracle_result(inputs[k], ar.AR_BF16), f"call {k}")
    finally:
        torch.cuda.synchronize()
        ar.ar_free(c)


def test_zero_elements_no_op(ctx):
    d = GuardedDst(16)
    s = [to_device(np.ones(16, dtype=np.float32)) for _ in range(2)]
    ar.ar_reduce(ctx, [d.ptr()], s, 0, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED)
    torch.cuda.synchronize()
    got = d.result()
    assert np.all(got.view(np.uint32) == np.uint32(0x7FA5A5A5))


# --------------------------------------------------------------------------
# errors detected on the host before anything is enqueued
# --------------------------------------------------------------------------

def test_error_paths(ctx):
    n = 4096
    dev = [to_device(np.ones(n, dtype=np.float32)) for _ in range(2)]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    host_pageable = [np.ones(n, dtype=np.float32) for _ in range(2)]
    pinned = [to_pinned(np.ones(n, dtype=np.float32)) for _ in range(2)]
    E = ar.AR_ERR_INVALID
    log_case("error paths")
    # pageable host memory as a source of a device mode
    rc = ar.ar_reduce(ctx, [out], [h.ctypes.data for h in host_pageable], n, ar.AR_F32, ar.AR_BF16,
                      ar.AR_MODE_CHUNKED, check=False)
    assert rc == E
    # pinned host sources outside host-staged mode
    assert ar.ar_reduce(ctx, [out], pinned, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, check=False) == E
    # device sources in host-staged mode
    assert ar.ar_reduce(ctx, [out], dev, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_HOST_STAGED, check=False) == E
    # host destination
    assert ar.ar_reduce(ctx, [pinned[0]], dev, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, check=False) == E
    # a range running past the allocation (the binding's own size check, which would
    # raise first, is switched off so that the library's check is the one exercised)
    assert ar.ar_reduce(ctx, [out], dev, 1 << 28, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, check=False,
                        validate=False) == E
    # misaligned source
    assert ar.ar_reduce(ctx, [out], [dev[0].data_ptr() + 4, dev[1]], n - 4, ar.AR_F32, ar.AR_BF16,
                        ar.AR_MODE_CHUNKED, check=False) == E
    # a narrow destination with a different wire type
    assert ar.ar_reduce(ctx, [out], dev, n, ar.AR_F16, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                        check=False) == ar.AR_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    # the context still works afterwards
    ar.ar_reduce(ctx, [out], dev, n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 2.0)


def test_graph_capture_replays(ctx):
    """Decode-sized calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed
    several times, with eager work and synchronisation between replays; every replay is
    checked against the oracle.  The device schedules enqueue kernels only (no memsets,
    no host synchronisation), so they can be captured."""
    w = wl.WORKLOADS["decode_bf16"]
    calls, n, R = 16, w.n, w.R
    host = np.stack([np.stack(wl.partials(w, c)) for c in range(calls)])   # (calls, R, n)
    want = oracle.reduce([host[:, r, :].ravel() for r in range(R)], w.wire)[0].reshape(calls, n)
    dev = torch.from_numpy(host).cuda()
    out = torch.empty((calls, n), dtype=torch.float32, device="cuda")
    big_n = 300_001
    big_src = [to_device(s) for s in wl.random_partials(9100, 0, 3, big_n)]
    big_want = oracle_result([s.cpu().numpy() for s in big_src], ar.AR_F16)
    big_out = torch.empty(big_n, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log_case("graph capture: 16 single-shot calls + 1 chunked call")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        st = torch.cuda.current_stream()
        for c in range(calls):
            ar.ar_reduce(ctx, [out[c]], [dev[c, r] for r in range(R)], n, ar.AR_F32, w.wire,
                         ar.AR_MODE_SINGLE_SHOT, stream=st)
        ar.ar_reduce(ctx, [big_out], big_src, big_n, ar.AR_F32, ar.AR_F16, ar.AR_MODE_CHUNKED, stream=st)
    for rep in range(3):
        out.fill_(float("nan"))
        big_out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(out.cpu().numpy(), want, f"graph replay {rep} decode")
        assert_bits_equal(big_out.cpu().numpy(), big_want, f"graph replay {rep} chunked")


def test_bound_calls_match_plain_calls(ctx):
    """ar.bind_reduce: the pre-converted call gives the same bytes as ar_reduce /
    ar_reduce_add, every time it is invoked."""
    n = 4096 * 33
    srcs = [to_device(x) for x in wl.random_partials(9300, 0, 3, n, dist="wide")]
    row = to_device(wl.residual(9301, 0, 4096))
    want = torch.empty(n, device="cuda")
    got = torch.empty(n, device="cuda")
    log_case("bound calls: plain and residual, single-shot and chunked")
    for mode in (ar.AR_MODE_SINGLE_SHOT, ar.AR_MODE_CHUNKED):
        for res in (None, row):
            if res is None:
                ar.ar_reduce(ctx, [want], srcs, n, ar.AR_F32, ar.AR_BF16, mode)
            else:
                ar.ar_reduce_add(ctx, [want], srcs, n, ar.AR_F32, ar.AR_BF16, mode, res)
            f = ar.bind_reduce(ctx, [got], srcs, n, ar.AR_F32, ar.AR_BF16, mode, residual=res)
            for _ in range(2):
                got.fill_(float("nan"))
                assert f() == ar.AR_OK
                torch.cuda.synchronize()
                assert torch.equal(got.view(torch.int32), want.view(torch.int32))
    # row-strided: rows of 4096 inside 4608-wide partial rows, with a bias row
    rows, cols, ss, ds = 33, 4096, 4608, 4352
    rsrcs = [torch.randn(rows * ss, device="cuda") for _ in range(2)]
    rwant = torch.full((rows * ds,), float("nan"), device="cuda")
    rgot = torch.full((rows * ds,), float("nan"), device="cuda")
    ar.ar_reduce_rows(ctx, [rwant], rsrcs, rows, cols, ss, ds, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                      residual=row, res_stride=0)
    f = ar.bind_reduce_rows(ctx, [rgot], rsrcs, rows, cols, ss, ds, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                            residual=row, res_stride=0)
    for _ in range(2):
        assert f() == ar.AR_OK
        torch.cuda.synchronize()
        assert torch.equal(rgot.view(torch.int32), rwant.view(torch.int32))
        rgot.fill_(float("nan"))


def test_contexts_on_threads_and_streams():
    """Two host threads, each with its own context and stream, issue interleaved calls
    (single-shot, chunked, slice + broadcast) at the same time; every result matches the
    oracle.  The library keeps no global mutable state, so separate contexts need no
    locking."""
    import threading

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    cases = []
    for t in range(2):
        srcs = wl.random_partials(9400 + t, 0, 4, 200_003, dist="wide")
        cases.append((srcs, oracle.reduce(srcs, ar.AR_BF16)[0]))
    errors = []

    def worker(t):
        try:
            torch.cuda.set_device(0)
            c = ar.ar_init(0)
            stream = torch.cuda.Stream()
            srcs, want = cases[t]
            dev = [to_device(x) for x in srcs]
            outs = [torch.empty(200_003, device="cuda") for _ in range(4)]
            torch.cuda.synchronize()
            for k in range(30):
                mode = (ar.AR_MODE_SINGLE_SHOT, ar.AR_MODE_CHUNKED, ar.AR_MODE_RS_BCAST)[k % 3]
                dsts = outs if mode == ar.AR_MODE_RS_BCAST else outs[:1]
                with torch.cuda.stream(stream):
                    for d in dsts:
                        d.fill_(float("nan"))
                ar.ar_reduce(c, dsts, dev, 200_003, ar.AR_F32, ar.AR_BF16, mode, stream=stream)
                stream.synchronize()
                for d in dsts:
                    assert_bits_equal(d.cpu().numpy(), want, f"thread {t} call {k} mode {mode}")
            ar.ar_free(c)
        except BaseException as e:   # re-raised in the main thread
            errors.append(e)

    log_case("two threads, two contexts, two streams")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=90)
    assert not any(th.is_alive() for th in threads), "a worker did not finish"
    if errors:
        raise errors[0]


def test_graph_capture_every_capturable_path(ctx):
    """One graph holding a call of every capturable kind -- slice + broadcast, the
    residual add (element-wise and broadcast row), a narrow destination, a row-strided
    call with a bias row, and host-staged sources read directly -- replayed three times
    with eager work between replays, each replay checked against the oracle.  A
    host-staged call on the copy-engine path is refused under capture (status
    AR_ERR_UNSUPPORTED, nothing recorded) and the capture stays usable."""
    cases = []   # (output tensor, expected, 16-bit?)
    n = 100_003
    s3 = wl.random_partials(9200, 0, 3, n, dist="wide")
    d3 = [torch.empty(n, device="cuda") for _ in range(3)]
    cases += [(d, oracle.reduce(s3, ar.AR_F16)[0], False) for d in d3]
    s2 = wl.random_partials(9201, 0, 2, 4096 * 24)
    ew = wl.residual(9202, 0, s2[0].size)
    row = wl.residual(9203, 0, 4096)
    d_ew = torch.empty(s2[0].size, device="cuda")
    d_row = torch.empty(s2[0].size, device="cuda")
    cases += [(d_ew, oracle.reduce(s2, ar.AR_BF16, residual=ew)[0], False),
              (d_row, oracle.reduce(s2, ar.AR_BF16, residual=np.tile(row, 24))[0], False)]
    sn = wl.random_narrow(9204, 0, 4, 70_001, ar.AR_BF16)
    d_n = torch.empty(70_001, dtype=torch.int16, device="cuda")
    cases.append((d_n, oracle.reduce(sn, ar.AR_BF16, src_type=ar.AR_BF16, dst_type=ar.AR_BF16)[0], True))
    rows, cols, ss, ds = 37, 520, 528, 536
    sr = wl.random_partials(9205, 0, 2, rows * ss)
    bias = wl.residual(9206, 0, cols)
    d_r = torch.zeros(rows * ds, device="cuda")
    dense = [np.concatenate([x[i * ss:i * ss + cols] for i in range(rows)]) for x in sr]
    want_r = oracle.reduce(dense, ar.AR_BF16, residual=np.tile(bias, rows))[0]
    sh = [wl.as_wire_typed(x, ar.AR_BF16) for x in wl.random_partials(9207, 0, 4, 65_536)]
    d_h = torch.empty(65_536, device="cuda")
    cases.append((d_h, oracle.reduce(sh, ar.AR_BF16, src_type=ar.AR_BF16)[0], False))

    t3 = [to_device(x) for x in s3]
    t2 = [to_device(x) for x in s2]
    t_ew, t_row, t_bias = to_device(ew), to_device(row), to_device(bias)
    tn = [to_device(x) for x in sn]
    tr = [to_device(x) for x in sr]
    th = [to_pinned(x) for x in sh]
    ctx_copy = ar.ar_init(0, {"host_path": 1})
    torch.cuda.synchronize()
    log_case("graph capture: broadcast, residual adds, narrow, rows, host direct; copy-engine refused")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        st = torch.cuda.current_stream()
        ar.ar_reduce(ctx, d3, t3, n, ar.AR_F32, ar.AR_F16, ar.AR_MODE_RS_BCAST, stream=st)
        ar.ar_reduce_add(ctx, [d_ew], t2, s2[0].size, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, t_ew, stream=st)
        ar.ar_reduce_add(ctx, [d_row], t2, s2[0].size, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, t_row, stream=st)
        ar.ar_reduce(ctx, [d_n], tn, 70_001, ar.AR_BF16, ar.AR_BF16, ar.AR_MODE_CHUNKED, stream=st)
        ar.ar_reduce_rows(ctx, [d_r], tr, rows, cols, ss, ds, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                          residual=t_bias, res_stride=0, stream=st)
        ar.ar_reduce(ctx, [d_h], th, 65_536, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE,
                     stream=st)
        refused = ar.ar_reduce(ctx_copy, [d_h], th, 65_536, ar.AR_F32, ar.AR_BF16,
                               ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE, stream=st, check=False)
    assert refused == ar.AR_ERR_UNSUPPORTED
    for rep in range(3):
        for out, _, _ in cases:
            out.fill_(0 if out.dtype == torch.int16 else float("nan"))
        d_r.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (out, want, is16) in enumerate(cases):
            if is16:
                assert_bits_equal16(out.cpu().view(torch.int16).numpy().view(np.uint16), want, ar.AR_BF16,
                                    f"graph replay {rep} output {k}")
            else:
                assert_bits_equal(out.cpu().numpy(), want, f"graph replay {rep} output {k}")
        got = d_r.cpu().numpy()
        assert_bits_equal(np.concatenate([got[i * ds:i * ds + cols] for i in range(rows)]), want_r,
                          f"graph replay {rep} rows")
    # the refused copy-engine call still works outside a capture
    d_h.fill_(float("nan"))
    ar.ar_reduce(ctx_copy, [d_h], th, 65_536, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE)
    torch.cuda.synchronize()
    assert_bits_equal(d_h.cpu().numpy(), cases[-1][1], "copy-engine call after the capture")
    del g
    ar.ar_free(ctx_copy)


@pytest.mark.parametrize("wire_name", ["bf16", "f16"])
def test_rounding_exhaustive_all_patterns(ctx, wire_name):
    """Every one of the 2^32 binary32 patterns through the GPU cast: src0 = the pattern,
    src1 = -0.0, so dst = widen(round_W(x)) exactly (x + (-0) == x for every x, NaN aside).
    Expected values come from the oracle's conversion, computed in parallel on the host."""
    from concurrent.futures import ThreadPoolExecutor

    wire = WIRES[wire_name]
    orc = oracle.load()
    chunk = 1 << 28
    negz = torch.full((chunk,), -0.0, dtype=torch.float32, device="cuda")
    out = torch.empty(chunk, dtype=torch.float32, device="cuda")
    round_fn = oracle.round_bf16_bits if wire == ar.AR_BF16 else oracle.round_f16_bits
    widen_fn = oracle.widen_bf16_bits if wire == ar.AR_BF16 else oracle.widen_f16_bits

    def expected(start):
        x = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        parts = np.array_split(x, 16)
        with ThreadPoolExecutor(16) as pool:
            res = list(pool.map(lambda p: widen_fn(round_fn(p, orc), orc), parts))
        return np.concatenate(res).view(np.float32)

    for k in range(1 << 32 >> 28):
        start = k * chunk
        log_case(f"exhaustive rounding {wire_name} chunk {k}")
        x = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda").to(torch.int32)
        x = x.view(torch.float32)
        ar.ar_reduce(ctx, [out], [x, negz], chunk, ar.AR_F32, wire, ar.AR_MODE_CHUNKED)
        torch.cuda.synchronize()
        del x
        got = out.cpu().numpy()
        assert_bits_equal(got, expected(start), f"exhaustive {wire_name} chunk {k}")


@pytest.mark.parametrize("kname", ["reg_cached", "reg_streaming", "lds_cached", "lds_streaming", "host_direct"])
@pytest.mark.parametrize("mode_name", ["single_shot", "chunked", "rs_bcast", "host_staged"])
def test_inactive_ranks(kctx, kname, mode_name):
    """NULL sources with AR_SRC_INACTIVE_NULL: inactive ranks contribute +0.0 (rank 0
    inactive, middle ranks inactive, all inactive), edge values included."""
    mode = MODES[mode_name] | ar.AR_SRC_INACTIVE_NULL
    g = np.concatenate([wl.special_values(), wl.nan_values()])
    rng = np.random.default_rng(77)
    for i, (R, n) in enumerate([(2, 4097), (3, 70_001), (5, 2_048), (8, 65_536 + 9), (16, 9_001)]):
        srcs = wl.random_partials(9500 + i, 0, R, n, dist="wide")
        srcs[-1][:g.size] = g
        for trial in range(3):
            active = rng.random(R) < 0.5
            if trial == 0:
                active[0] = False
            if trial == 2:
                active[:] = False
            for wire_name, wire in WIRES.items():
                for src_wire in ([False, True] if wire != ar.AR_F32 else [False]):
                    what = (f"inactive {kname} {mode_name} R={R} n={n} wire={wire_name} "
                            f"src_wire={src_wire} active={active.astype(int).tolist()}")
                    log_case(what)
                    used = [wl.as_wire_typed(s, wire) if src_wire else s for s in srcs]
                    c = kctx[kname]
                    base = mode & ar.AR_MODE_MASK
                    n_dst = R if base == ar.AR_MODE_RS_BCAST else 1
                    if base == ar.AR_MODE_HOST_STAGED:
                        ts = [to_pinned(s) if a else None for s, a in zip(used, active)]
                    else:
                        ts = [to_device(s) if a else None for s, a in zip(used, active)]
                    dsts = [GuardedDst(n) for _ in range(n_dst)]
                    flags = ar.AR_SRC_WIRE if src_wire else 0
                    ar.ar_reduce(c, [d.ptr() for d in dsts], [0 if t is None else t for t in ts], n,
                                 ar.AR_F32, wire, mode | flags)
                    torch.cuda.synchronize()
                    want = oracle.reduce([s if a else None for s, a in zip(used, active)], wire,
                                         src_type=wire if src_wire else None, n=n)[0]
                    for d in dsts:
                        assert_bits_equal(d.result(), want, what)


# XCD placement: runs from one workgroup's share up to far beyond the grid, with
# grids that are and are not multiples of 8 runs (the tail keeps its numbering),
# through both streaming families, every streaming schedule, 16-bit sources, a
# residual and 8 ranks -- every result bit-exact against the oracle.
PLACEMENT_RUNS = [1, 512, 2048, 1 << 13, 1 << 17, 1 << 24]


@pytest.mark.parametrize("run", PLACEMENT_RUNS)
def test_xcd_placement_every_run(run):
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    cases = [
        # (R, n, wire, mode, extra config, src_wire)
        (2, (1 << 21) + 77, ar.AR_BF16, ar.AR_MODE_CHUNKED, {}, False),
        (3, 1_000_003, ar.AR_F16, ar.AR_MODE_CHUNKED, {"grid_wgs": 9}, False),
        (4, (1 << 20) + 4 * 512 + 3, ar.AR_F16, ar.AR_MODE_RS_BCAST, {}, False),
        (4, 777_777, ar.AR_BF16, ar.AR_MODE_RS_BCAST, {"stream_kernel": 2, "grid_wgs": 100}, False),
        (2, (1 << 20) + 5, ar.AR_BF16, ar.AR_MODE_CHUNKED, {"stream_kernel": 2, "chunk_bytes": 1 << 16}, True),
        (8, 600_001, ar.AR_BF16, ar.AR_MODE_CHUNKED, {"stream_kernel": 1}, False),
        (2, 3 * 1024 * 512, ar.AR_F32, ar.AR_MODE_CHUNKED, {"grid_wgs": 1000}, False),
    ]
    for i, (R, n, wire, mode, extra, src_wire) in enumerate(cases):
        c = ar.ar_init(0, {"xcd_run_elems": run, **extra})
        try:
            log_case(f"placement run={run} case {i}: R={R} n={n} wire={wire} mode={mode} cfg={extra} "
                     f"src_wire={src_wire}")
            srcs = wl.random_partials(70_000 + i, run % 997, R, n, dist="normal+outliers")
            got, used = run_case(None, srcs, wire, mode, src_wire=src_wire, config_ctx=c)
        finally:
            torch.cuda.synchronize()
            ar.ar_free(c)
        want = oracle_result(used, wire, src_type=wire if src_wire else None)
        for d, g in enumerate(got):
            assert_bits_equal(g, want, f"placement run={run} case {i} dst {d}")
    # a residual (register family, 128-thread workgroups) and a row-strided call
    c = ar.ar_init(0, {"xcd_run_elems": run})
    try:
        n = (1 << 21) + 8 * 3
        srcs = wl.random_partials(70_100, 1, 2, n, dist="normal")
        res = wl.residual(70_101, 0, n)
        dst = GuardedDst(n)
        log_case(f"placement run={run}: residual n={n}")
        ar.ar_reduce_add(c, [dst.ptr()], [to_device(s) for s in srcs], n, ar.AR_F32, ar.AR_BF16,
                         ar.AR_MODE_CHUNKED, to_device(res), n)
        torch.cuda.synchronize()
        assert_bits_equal(dst.result(), oracle.reduce(srcs, oracle.BF16, residual=res)[0], f"placement {run} res")
    finally:
        torch.cuda.synchronize()
        ar.ar_free(c)
