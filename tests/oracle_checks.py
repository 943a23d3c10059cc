"""Pins of the CPU oracle against things other than itself.

Each ``check_*`` function takes a loaded oracle library handle and raises
``AssertionError`` on disagreement.  ``test_oracle_pins.py`` runs them on the
real oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle with
a planted mistake and requires that at least one check fails for each.

What pins what:

* wire rounding        -- exhaustive over all 2^32 binary32 patterns against
                          torch's CPU bfloat16 / float16 conversions (IEEE
                          round-to-nearest-even), numpy's float16 conversion on
                          a sample, and the hand-worked rows of
                          ``golden/worked_examples.txt``;
* widening             -- exhaustive over all 2^16 patterns against torch and
                          numpy;
* each binary32 add    -- a theorem: for binary32 a, b, RN32(a+b) equals
                          float32(float64(a) + float64(b)) because binary64 has
                          at least 2p+2 significand bits (double rounding is
                          innocuous, Figueroa 1995);
* the ordered fold     -- numpy's sequential float32 accumulation, the fp64
                          route above, brute force over every ordered tuple of
                          a grid of edge values, and the hand-worked rows;
* the whole reduce     -- a closed form: partials k * 2^-6 with |k| <= 127 are
                          exact in every wire type and every partial sum for
                          R <= 16 is exact in binary32, so the result is
                          (sum k) * 2^-6, computed with integers;
* the residual         -- the fp64 route with the residual as one more,
                          unrounded, last term; the closed form with a k * 2^-6
                          residual; a broadcast row equals the element-wise
                          residual tiled over the rows; hand-worked rows;
* narrow destinations  -- numpy's float16 and torch's CPU bfloat16 arithmetic
                          (each add correctly rounded in that type, since
                          binary32 has >= 2p+2 bits for p = 11 and p = 8),
                          binary64 then one conversion for float16, brute force
                          over ordered pairs and triples of 16-bit edge
                          patterns, a closed form exact in the narrow type, and
                          hand-worked rows;
* row-strided tensors  -- the rows gathered by numpy slicing and reduced by the
                          1-D routes above (fp64 route, library 16-bit
                          arithmetic), scattered back by slicing; the bytes
                          between rows keep their prior contents; a stride
                          equal to the row length is the 1-D reduce.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import workloads

F32, F16, BF16 = oracle.F32, oracle.F16, oracle.BF16
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.txt")
WIRE_BY_NAME = {"f32": F32, "f16": F16, "bf16": BF16}


# --- independent routes built only from library routines ---------------------

def lib_round_bits(x: np.ndarray, wire: int) -> np.ndarray:
    """Wire pattern of each float32 via torch's CPU conversion (uint16)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if wire == BF16:
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if wire == F16:
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(wire)


def lib_wire_value(x: np.ndarray, wire: int) -> np.ndarray:
    """float32 value of round_W(x), via torch's conversions both ways."""
    if wire == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    dt = torch.bfloat16 if wire == BF16 else torch.float16
    return t.to(dt).to(torch.float32).numpy()


def fp64_route_fold(ws: list[np.ndarray]) -> np.ndarray:
    """Left fold where each binary32 add is done as float32(float64 + float64)."""
    acc = ws[0].astype(np.float32)
    for w in ws[1:]:
        acc = (acc.astype(np.float64) + w.astype(np.float64)).astype(np.float32)
    return acc


def is_nan16(h: np.ndarray, wire: int) -> np.ndarray:
    h = h.astype(np.uint32)
    if wire == BF16:
        return ((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)
    return ((h & 0x7C00) == 0x7C00) & ((h & 0x03FF) != 0)


def assert_same_f32(got: np.ndarray, want: np.ndarray, what: str) -> None:
    """Bit equality of float32 arrays, NaN compared only as 'is a NaN'."""
    got = np.ascontiguousarray(got, dtype=np.float32)
    want = np.ascontiguousarray(want, dtype=np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    if not np.array_equal(gn, wn):
        i = int(np.flatnonzero(gn != wn)[0])
        raise AssertionError(f"{what}: NaN mismatch at {i}: got {got[i]!r} want {want[i]!r}")
    gb = got.view(np.uint32)[~gn]
    wb = want.view(np.uint32)[~wn]
    if not np.array_equal(gb, wb):
        j = int(np.flatnonzero(gb != wb)[0])
        raise AssertionError(f"{what}: bits differ (first non-NaN mismatch {gb[j]:#010x} vs {wb[j]:#010x})")


# --- golden worked examples --------------------------------------------------

def load_golden() -> list[dict]:
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            body = line.split("#", 1)[0].strip()
            if not body:
                continue
            parts = body.split()
            rid, op, wire, inputs, expected = parts[0], parts[1], parts[2], parts[3], parts[4]
            rows.append({
                "id": rid, "op": op, "wire": WIRE_BY_NAME[wire],
                "inputs": [None if h == "-" else int(h, 16) for h in inputs.split(",")],
                "expected": None if expected == "NAN" else int(expected, 16),
            })
    return rows


def check_golden(lib) -> None:
    rows = load_golden()
    assert len(rows) >= 50
    for row in rows:
        if row["op"] in ("dreduce", "dradd"):
            _check_golden_narrow(lib, row)
            continue
        if row["op"] == "radd":
            vals = np.array(row["inputs"], dtype=np.uint32).view(np.float32)
            srcs = [vals[i:i + 1] for i in range(len(vals) - 1)]
            got = oracle.reduce(srcs, row["wire"], lib=lib, residual=vals[-1:])[0, 0]
            _check_golden_f32(row, got)
            continue
        if row["op"] == "reduce":
            srcs = [None if v is None else np.array([v], dtype=np.uint32).view(np.float32)
                    for v in row["inputs"]]
            if all(s is None for s in srcs):
                got = _reduce_all_inactive(lib, len(row["inputs"]), row["wire"])
            else:
                got = oracle.reduce(srcs, row["wire"], lib=lib)[0, 0]
            _check_golden_f32(row, got)
            continue
        x = np.array(row["inputs"], dtype=np.uint32)
        if row["op"] == "round":
            fn = oracle.round_bf16_bits if row["wire"] == BF16 else oracle.round_f16_bits
            got = int(fn(x, lib)[0])
            if row["expected"] is None:
                assert bool(is_nan16(np.array([got]), row["wire"])[0]), row["id"]
            else:
                assert got == row["expected"], f"{row['id']}: {got:#06x} != {row['expected']:#06x}"
        else:
            raise AssertionError(f"unknown golden op {row['op']!r} in {row['id']}")


def _check_golden_f32(row, got) -> None:
    if row["expected"] is None:
        assert np.isnan(got), row["id"]
    else:
        gb = int(np.array([got], dtype=np.float32).view(np.uint32)[0])
        assert gb == row["expected"], f"{row['id']}: {gb:#010x} != {row['expected']:#010x}"


def _check_golden_narrow(lib, row) -> None:
    w = row["wire"]
    vals = np.array(row["inputs"], dtype=np.uint16)
    k = len(vals) - 1 if row["op"] == "dradd" else len(vals)
    srcs = [vals[i:i + 1] for i in range(k)]
    res = vals[k:k + 1] if row["op"] == "dradd" else None
    got = int(oracle.reduce(srcs, w, src_type=w, dst_type=w, residual=res, lib=lib)[0, 0])
    if row["expected"] is None:
        assert bool(is_nan16(np.array([got]), w)[0]), row["id"]
    else:
        assert got == row["expected"], f"{row['id']}: {got:#06x} != {row['expected']:#06x}"


def _reduce_all_inactive(lib, R: int, wire: int) -> float:
    """The oracle with every rank inactive (n = 1), through the raw C entry point."""
    import ctypes

    out = np.empty(1, dtype=np.float32)
    dst = (ctypes.c_void_p * 1)(out.ctypes.data)
    srcs = (ctypes.c_void_p * R)(*([None] * R))
    rc = lib.orc_reduce(dst, 1, srcs, R, 1, F32, wire)
    assert rc == 0
    return out[0]


def check_inactive_ranks(lib, seed: int = 31) -> None:
    """An inactive (NULL) rank equals an all-(+0.0) partial: compared with the fp64
    route over library-rounded partials where inactive ranks are zero arrays."""
    rng = np.random.default_rng(seed)
    g = _edge_grid()
    for R in (2, 3, 5, 8, 16):
        n = 2000
        srcs = workloads.random_partials(960, R, R, n, dist="wide")
        srcs[0][:g.size] = g                      # edge values incl. -0 and NaN
        for trial in range(3):
            active = rng.random(R) < 0.6
            if trial == 0:
                active[0] = False                 # rank 0 inactive: the fold starts at +0
            mixed = [s if a else None for s, a in zip(srcs, active)]
            if not any(active):
                continue
            for wire in (F32, BF16, F16):
                got = oracle.reduce(mixed, wire, n_dst=2, lib=lib)
                zeros = [s if a else np.zeros(n, dtype=np.float32) for s, a in zip(srcs, active)]
                with np.errstate(all="ignore"):
                    want = fp64_route_fold([lib_wire_value(z, wire) for z in zeros])
                assert_same_f32(got[0], want, f"inactive R={R} wire={wire} active={active.tolist()}")
                assert np.array_equal(got[0].view(np.uint32), got[1].view(np.uint32))
    # every rank inactive, through the wrapper with an explicit n: +0.0 everywhere
    # (a zeroed shard, never -0), in every destination; with a residual the result
    # is 0 + residual (so -0 in the residual becomes +0); the same in 16-bit types
    n = 777
    for wire in (F32, BF16, F16):
        got = oracle.reduce([None] * 3, wire, n_dst=2, lib=lib, n=n)
        assert got.shape == (2, n) and not got.view(np.uint32).any(), f"all inactive, wire {wire}"
    res = workloads.random_partials(961, 0, 1, n, dist="wide")[0]
    res[:g.size] = g
    got = oracle.reduce([None, None], BF16, lib=lib, residual=res, n=n)[0]
    with np.errstate(all="ignore"):
        want = (np.float64(0.0) + res.astype(np.float64)).astype(np.float32)
    assert_same_f32(got, want, "all inactive + residual")
    for w in (F16, BF16):
        got16 = oracle.reduce([None, None, None, None], w, src_type=w, dst_type=w, lib=lib, n=n)[0]
        assert got16.dtype == np.uint16 and not got16.any(), f"all inactive narrow {w}"
    try:
        oracle.reduce([None, None], F32, lib=lib)
    except ValueError:
        pass
    else:
        raise AssertionError("all-inactive call without n must be refused")


# --- conversions -------------------------------------------------------------

def _round_chunk_ok(lib, wire: int, start: int, size: int) -> None:
    x = np.arange(start, start + size, dtype=np.uint64).astype(np.uint32)
    fn = oracle.round_bf16_bits if wire == BF16 else oracle.round_f16_bits
    got = fn(x, lib)
    want = lib_round_bits(x.view(np.float32), wire)
    gn, wn = is_nan16(got, wire), is_nan16(want, wire)
    if not np.array_equal(gn, wn):
        i = int(np.flatnonzero(gn != wn)[0])
        raise AssertionError(f"wire {wire}: NaN class differs at input {int(x[i]):#010x}")
    bad = (got != want) & ~gn
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"wire {wire}: round({int(x[i]):#010x}) = {int(got[i]):#06x}, "
                             f"library gives {int(want[i]):#06x}")


def check_round_exhaustive(lib, wire: int, chunk_log2: int = 22, workers: int = 8) -> None:
    """All 2^32 binary32 patterns against torch's conversion."""
    size = 1 << chunk_log2
    starts = range(0, 1 << 32, size)
    threads = torch.get_num_threads()
    torch.set_num_threads(1)            # parallelism comes from the chunk pool
    try:
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(lambda s: _round_chunk_ok(lib, wire, s, size), starts))
    finally:
        torch.set_num_threads(threads)


def check_round_sampled(lib, wire: int, n: int = 1 << 20, seed: int = 7) -> None:
    """Random patterns plus the edge grid (cheap form of the exhaustive pin)."""
    rng = np.random.default_rng(seed)
    x = np.concatenate([rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32),
                        workloads.special_values().view(np.uint32),
                        workloads.nan_values().view(np.uint32)])
    fn = oracle.round_bf16_bits if wire == BF16 else oracle.round_f16_bits
    got = fn(x, lib)
    want = lib_round_bits(x.view(np.float32), wire)
    gn, wn = is_nan16(got, wire), is_nan16(want, wire)
    assert np.array_equal(gn, wn), f"wire {wire}: NaN class differs"
    bad = (got != want) & ~gn
    assert not bad.any(), f"wire {wire}: {int(bad.sum())} rounding mismatches"


def check_round_f16_numpy_sample(lib, n: int = 1 << 22, seed: int = 11) -> None:
    """Second witness for float16: numpy's own conversion on a random sample."""
    rng = np.random.default_rng(seed)
    x = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    got = oracle.round_f16_bits(x, lib)
    with np.errstate(over="ignore", invalid="ignore"):
        want = x.view(np.float32).astype(np.float16).view(np.uint16)
    gn, wn = is_nan16(got, F16), is_nan16(want, F16)
    assert np.array_equal(gn, wn)
    assert np.array_equal(got[~gn], want[~wn])


def check_widen_exhaustive(lib) -> None:
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got_b = oracle.widen_bf16_bits(h, lib).view(np.float32)
    want_b = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    assert_same_f32(got_b, want_b, "widen bf16 vs torch")
    got_h = oracle.widen_f16_bits(h, lib).view(np.float32)
    want_h = h.view(np.float16).astype(np.float32)
    assert_same_f32(got_h, want_h, "widen f16 vs numpy")
    want_h2 = torch.from_numpy(h.view(np.int16).copy()).view(torch.float16).to(torch.float32).numpy()
    assert_same_f32(got_h, want_h2, "widen f16 vs torch")


# --- additions and folds -----------------------------------------------------

def _edge_grid() -> np.ndarray:
    return np.concatenate([workloads.special_values(), workloads.nan_values()[:1]])


def check_add_theorem(lib, n: int = 1 << 20, seed: int = 3) -> None:
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    b = (a.view(np.uint32) ^ rng.integers(0, 1 << 12, n, dtype=np.uint32)).view(np.float32)
    # near-cancellations, random far-apart pairs and the full edge grid x grid
    g = _edge_grid()
    ga, gb = np.meshgrid(g, g, indexing="ij")
    a = np.concatenate([a, -b, ga.ravel()])
    b = np.concatenate([b, rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32).view(np.float32),
                        gb.ravel()])
    got = oracle.add_f32(a, b, lib)
    with np.errstate(all="ignore"):
        want64 = (a.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
        want32 = a + b
    assert_same_f32(got, want64, "add vs fp64 route")
    assert_same_f32(got, want32, "add vs numpy float32")


def check_fold_bruteforce(lib, R: int, grid: np.ndarray | None = None) -> None:
    """Every ordered R-tuple of the edge grid, every wire type, fp64 route."""
    g = _edge_grid() if grid is None else grid
    cols = [c.ravel() for c in np.meshgrid(*([g] * R), indexing="ij")]
    for wire in (F32, BF16, F16):
        got = oracle.reduce(cols, wire, lib=lib)[0]
        with np.errstate(all="ignore"):
            want = fp64_route_fold([lib_wire_value(c, wire) for c in cols])
        assert_same_f32(got, want, f"fold R={R} wire={wire}")


def check_ordered_sum(lib, R: int = 5, n: int = 1 << 16, seed: int = 5) -> None:
    """fp32 wire: the result is the plain left-to-right float32 sum."""
    srcs = workloads.random_partials(900 + seed, 0, R, n, dist="wide")
    got = oracle.reduce(srcs, F32, lib=lib)[0]
    acc = srcs[0].copy()
    with np.errstate(all="ignore"):
        for s in srcs[1:]:
            acc += s
    assert_same_f32(got, acc, "fp32-wire ordered sum")
    # the same reduce through any narrower wire equals the sum of the library-rounded partials
    for wire in (BF16, F16):
        got_w = oracle.reduce(srcs, wire, lib=lib)[0]
        ws = [lib_wire_value(s, wire) for s in srcs]
        acc = ws[0].copy()
        with np.errstate(all="ignore"):
            for w in ws[1:]:
                acc += w
        assert_same_f32(got_w, acc, f"wire {wire} ordered sum")


def check_closed_form(lib, seed: int = 17) -> None:
    """k * 2^-6 partials: result must be (sum k) * 2^-6 exactly, any wire, any R."""
    rng = np.random.default_rng(seed)
    for R in (2, 3, 4, 7, 8, 16):
        n = 4099
        ks = [rng.integers(-127, 128, n) for _ in range(R)]
        srcs = [(k.astype(np.float32) * np.float32(2.0 ** -6)) for k in ks]
        total = np.sum(ks, axis=0)                       # integer arithmetic
        want = total.astype(np.float32) * np.float32(2.0 ** -6)
        for wire in (F32, BF16, F16):
            got = oracle.reduce(srcs, wire, n_dst=2, lib=lib)
            assert_same_f32(got[0], want, f"closed form R={R} wire={wire}")
            assert np.array_equal(got[0].view(np.uint32), got[1].view(np.uint32))
            if wire != F32:
                pre = [lib_round_bits(s, wire) for s in srcs]
                got_w = oracle.reduce(pre, wire, src_type=wire, lib=lib)[0]
                assert_same_f32(got_w, want, f"closed form (wire-typed srcs) R={R} wire={wire}")


def check_order_sensitivity(lib) -> None:
    """The fold is taken in rank order: a reordered sum must differ where rounding bites."""
    a = np.array([2.0 ** 24], dtype=np.float32)
    one = np.array([1.0], dtype=np.float32)
    fwd = oracle.reduce([a, one, one], F32, lib=lib)[0, 0]
    rev = oracle.reduce([one, one, a], F32, lib=lib)[0, 0]
    assert fwd == np.float32(2.0 ** 24) and rev == np.float32(2.0 ** 24 + 2)


def check_broadcast_and_wire_srcs(lib, seed: int = 23) -> None:
    """Every destination row is identical; pre-rounded wire-typed sources give the same bytes."""
    srcs = workloads.random_partials(950, seed, 6, 3001, dist="wide")
    for wire in (F32, BF16, F16):
        out = oracle.reduce(srcs, wire, n_dst=6, lib=lib)
        for d in range(1, 6):
            assert np.array_equal(out[0].view(np.uint32), out[d].view(np.uint32))
        if wire != F32:
            pre = [lib_round_bits(s, wire) for s in srcs]
            out_w = oracle.reduce(pre, wire, src_type=wire, lib=lib)[0]
            assert_same_f32(out_w, out[0], f"wire-typed sources wire={wire}")


# --- residual ------------------------------------------------------------------

def check_residual(lib, seed: int = 41) -> None:
    """The residual is one more binary32 add after the last rank, never wire-rounded:
    the fp64 route over library-rounded partials with the raw residual appended."""
    g = _edge_grid()
    for R in (2, 3, 8):
        n = 3000
        srcs = workloads.random_partials(970, seed, R, n, dist="wide")
        res = workloads.residual(970, seed, n, dist="wide")
        res[:g.size] = g
        srcs[-1][g.size:2 * g.size] = g
        for wire in (F32, BF16, F16):
            got = oracle.reduce(srcs, wire, n_dst=2, residual=res, lib=lib)
            with np.errstate(all="ignore"):
                want = fp64_route_fold([lib_wire_value(s, wire) for s in srcs] + [res])
            assert_same_f32(got[0], want, f"residual R={R} wire={wire}")
            assert np.array_equal(got[0].view(np.uint32), got[1].view(np.uint32))
            # one broadcast row == the element-wise residual tiled over the rows
            row = res[:600]
            got_row = oracle.reduce(srcs, wire, residual=row, lib=lib)[0]
            want_row = oracle.reduce(srcs, wire, residual=np.tile(row, n // 600), lib=lib)[0]
            assert_same_f32(got_row, want_row, f"row broadcast R={R} wire={wire}")
            with np.errstate(all="ignore"):
                want_row2 = fp64_route_fold([lib_wire_value(s, wire) for s in srcs] + [np.tile(row, n // 600)])
            assert_same_f32(got_row, want_row2, f"row broadcast fp64 route R={R} wire={wire}")
    # closed form: k * 2^-6 residual, exact everywhere
    rng = np.random.default_rng(seed)
    for R in (2, 5, 15):
        n = 2053
        ks = [rng.integers(-127, 128, n) for _ in range(R + 1)]
        vals = [k.astype(np.float32) * np.float32(2.0 ** -6) for k in ks]
        want = np.sum(ks, axis=0).astype(np.float32) * np.float32(2.0 ** -6)
        for wire in (F32, BF16, F16):
            got = oracle.reduce(vals[:R], wire, residual=vals[R], lib=lib)[0]
            assert_same_f32(got, want, f"residual closed form R={R} wire={wire}")
    # inactive ranks with a residual: zeros in their place
    srcs = workloads.random_partials(971, seed, 4, 999, dist="wide")
    res = workloads.residual(971, seed, 999)
    got = oracle.reduce([srcs[0], None, srcs[2], None], BF16, residual=res, lib=lib)[0]
    z = np.zeros(999, dtype=np.float32)
    with np.errstate(all="ignore"):
        want = fp64_route_fold([lib_wire_value(s, BF16) for s in (srcs[0], z, srcs[2], z)] + [res])
    assert_same_f32(got, want, "residual with inactive ranks")


# --- narrow destinations --------------------------------------------------------

def lib_narrow_fold(ws16: list[np.ndarray], dtype: int) -> np.ndarray:
    """Left fold of 16-bit values with every add done by a library in that type:
    numpy float16 arithmetic, torch CPU bfloat16 arithmetic.  Returns uint16."""
    if dtype == F16:
        acc = ws16[0].view(np.float16).copy()
        with np.errstate(all="ignore"):
            for w in ws16[1:]:
                acc = acc + w.view(np.float16)
        return acc.view(np.uint16)
    acc = torch.from_numpy(ws16[0].view(np.int16).copy()).view(torch.bfloat16)
    for w in ws16[1:]:
        acc = acc + torch.from_numpy(w.view(np.int16).copy()).view(torch.bfloat16)
    return acc.view(torch.int16).numpy().view(np.uint16)


def f64_narrow_fold_f16(ws16: list[np.ndarray]) -> np.ndarray:
    """binary16 fold where each add is float64(a) + float64(b) converted once to binary16."""
    acc = ws16[0].view(np.float16)
    with np.errstate(all="ignore"):
        for w in ws16[1:]:
            acc = (acc.astype(np.float64) + w.view(np.float16).astype(np.float64)).astype(np.float16)
    return acc.view(np.uint16)


def assert_same_16(got: np.ndarray, want: np.ndarray, wire: int, what: str) -> None:
    """Bit equality of 16-bit patterns, NaN compared only as 'is a NaN'."""
    got = np.ascontiguousarray(got, dtype=np.uint16)
    want = np.ascontiguousarray(want, dtype=np.uint16)
    gn, wn = is_nan16(got, wire), is_nan16(want, wire)
    if not np.array_equal(gn, wn):
        i = int(np.flatnonzero(gn != wn)[0])
        raise AssertionError(f"{what}: NaN mismatch at {i}: got {int(got[i]):#06x} want {int(want[i]):#06x}")
    bad = (got != want) & ~gn
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} differ, first at {i}: "
                             f"{int(got[i]):#06x} vs {int(want[i]):#06x}")


def _grid16(dtype: int) -> np.ndarray:
    return np.concatenate([workloads.special_values16(dtype), workloads.nan_values16(dtype)[:1]])


def check_narrow_dst(lib, seed: int = 43) -> None:
    """fp16 / bf16 destinations accumulate in their own type, one rounding per add."""
    for dtype in (F16, BF16):
        g = _grid16(dtype)
        # brute force: every ordered pair and triple of the edge grid
        for R in (2, 3):
            cols = [c.ravel().astype(np.uint16) for c in np.meshgrid(*([g] * R), indexing="ij")]
            got = oracle.reduce(cols, dtype, src_type=dtype, dst_type=dtype, lib=lib)[0]
            assert_same_16(got, lib_narrow_fold(cols, dtype), dtype, f"narrow brute force R={R} dtype={dtype}")
            if dtype == F16:
                assert_same_16(got, f64_narrow_fold_f16(cols), dtype, f"narrow fp64 route R={R}")
        # random partials, several rank counts, residual element-wise and broadcast
        for R in (2, 4, 7, 16):
            n = 2400
            srcs = workloads.random_narrow(980, seed + R, R, n, dtype, dist="wide")
            srcs[0][:g.size] = g
            res = workloads.residual(980, seed + R, n, dtype, dist="wide")
            out = oracle.reduce(srcs, dtype, n_dst=3, src_type=dtype, dst_type=dtype, lib=lib)
            assert_same_16(out[0], lib_narrow_fold(srcs, dtype), dtype, f"narrow R={R} dtype={dtype}")
            for d in (1, 2):
                assert np.array_equal(out[0], out[d])
            got = oracle.reduce(srcs, dtype, src_type=dtype, dst_type=dtype, residual=res, lib=lib)[0]
            assert_same_16(got, lib_narrow_fold(srcs + [res], dtype), dtype, f"narrow residual R={R}")
            row = res[:480]
            got = oracle.reduce(srcs, dtype, src_type=dtype, dst_type=dtype, residual=row, lib=lib)[0]
            assert_same_16(got, lib_narrow_fold(srcs + [np.tile(row, n // 480)], dtype), dtype,
                           f"narrow row residual R={R}")
            # inactive ranks are +0 in the destination type
            mixed = [s if r % 3 else None for r, s in enumerate(srcs)]
            zero = np.zeros(n, dtype=np.uint16)
            got = oracle.reduce(mixed, dtype, src_type=dtype, dst_type=dtype, lib=lib)[0]
            assert_same_16(got, lib_narrow_fold([zero if s is None else s for s in mixed], dtype), dtype,
                           f"narrow inactive R={R}")
        # closed form: k * 2^-6, every partial sum exact in the narrow type
        rng = np.random.default_rng(seed)
        kmax = 127 if dtype == F16 else 7
        for R in (2, 8, 16):
            n = 1031
            ks = [rng.integers(-kmax, kmax + 1, n) for _ in range(R)]
            srcs = [workloads.as_wire_typed(k.astype(np.float32) * np.float32(2.0 ** -6), dtype) for k in ks]
            want = workloads.as_wire_typed(np.sum(ks, axis=0).astype(np.float32) * np.float32(2.0 ** -6), dtype)
            got = oracle.reduce(srcs, dtype, src_type=dtype, dst_type=dtype, lib=lib)[0]
            assert_same_16(got, want, dtype, f"narrow closed form R={R} dtype={dtype}")


# --- row-strided tensors ----------------------------------------------------------

def _scatter_rows(flat_init, rows_vals, rows, cols, stride):
    out = flat_init.copy()
    for i in range(rows):
        out[i * stride:i * stride + cols] = rows_vals[i]
    return out


def check_rows(lib, seed: int = 47) -> None:
    """Row-strided reduce: gathered rows through the independent 1-D routes."""
    rng = np.random.default_rng(seed)
    cases = [(5, 16, 20, 24, 16), (3, 520, 528, 520, 0), (7, 9, 12, 16, 9), (1, 33, 33, 40, 40),
             (4, 8, 8, 8, 0), (0, 8, 8, 8, 8)]
    for k, (rows, cols, ss, ds, rs) in enumerate(cases):
        R = 2 + k % 3
        n_src = max(1, (rows - 1) * ss + cols) if rows else 1
        srcs = workloads.random_partials(990 + k, seed, R, n_src, dist="wide")
        extent = (rows - 1) * ds + cols if rows else 0
        init = rng.integers(0, 1 << 32, extent, dtype=np.uint64).astype(np.uint32).view(np.float32)
        for wire in (F32, BF16, F16):
            for with_res in (False, True):
                res = None
                if with_res:
                    res_n = cols if rs == 0 else max(1, (rows - 1) * rs + cols)
                    res = workloads.residual(991 + k, seed, res_n, dist="wide")
                got = oracle.reduce_rows(srcs, wire, rows, cols, ss, ds, n_dst=2, residual=res,
                                         res_stride=rs, dst_init=init, lib=lib)
                g_rows = [np.stack([s[i * ss:i * ss + cols] for i in range(rows)]) if rows else
                          np.zeros((0, cols), np.float32) for s in srcs]
                terms = [lib_wire_value(g.ravel(), wire) for g in g_rows]
                if with_res:
                    r_rows = np.stack([res[(0 if rs == 0 else i * rs):(0 if rs == 0 else i * rs) + cols]
                                       for i in range(rows)]) if rows else np.zeros((0, cols), np.float32)
                    terms.append(r_rows.ravel())
                with np.errstate(all="ignore"):
                    flat = fp64_route_fold(terms) if rows else np.zeros(0, np.float32)
                want = _scatter_rows(init, flat.reshape(rows, cols), rows, cols, ds)
                what = f"rows case {k} wire={wire} residual={with_res}"
                assert_same_f32(got[0], want, what)
                assert np.array_equal(got[0].view(np.uint32), got[1].view(np.uint32)), what
    # narrow destination with row-strided tensors, through library 16-bit arithmetic
    for t in (F16, BF16):
        rows, cols, ss, ds = 6, 24, 32, 40
        srcs = workloads.random_narrow(995, seed, 3, (rows - 1) * ss + cols, t, dist="wide")
        res = workloads.residual(996, seed, cols, t, dist="wide")
        init = rng.integers(0, 1 << 16, (rows - 1) * ds + cols, dtype=np.uint32).astype(np.uint16)
        got = oracle.reduce_rows(srcs, t, rows, cols, ss, ds, src_type=t, dst_type=t, residual=res,
                                 res_stride=0, dst_init=init, lib=lib)[0]
        g = [np.concatenate([s[i * ss:i * ss + cols] for i in range(rows)]) for s in srcs]
        flat = lib_narrow_fold(g + [np.tile(res, rows)], t)
        assert_same_16(got, _scatter_rows(init, flat.reshape(rows, cols), rows, cols, ds), t, f"rows narrow {t}")
    # a stride equal to the row length is the 1-D reduce
    srcs = workloads.random_partials(997, seed, 4, 12 * 64, dist="wide")
    got = oracle.reduce_rows(srcs, BF16, 12, 64, 64, 64, lib=lib)[0]
    assert_same_f32(got, oracle.reduce(srcs, BF16, lib=lib)[0], "rows with stride == cols")


def cheap_checks():
    """Checks fast enough to run against every planted-mistake build."""
    return [
        ("golden", check_golden),
        ("round_bf16_sampled", lambda lib: check_round_sampled(lib, BF16, n=1 << 18)),
        ("round_f16_sampled", lambda lib: check_round_sampled(lib, F16, n=1 << 18)),
        ("widen", check_widen_exhaustive),
        ("add", lambda lib: check_add_theorem(lib, n=1 << 14)),
        ("fold_R2", lambda lib: check_fold_bruteforce(lib, 2)),
        ("ordered_sum", check_ordered_sum),
        ("closed_form", check_closed_form),
        ("order", check_order_sensitivity),
        ("broadcast", check_broadcast_and_wire_srcs),
        ("inactive", check_inactive_ranks),
        ("residual", check_residual),
        ("narrow", check_narrow_dst),
        ("rows", check_rows),
    ]
