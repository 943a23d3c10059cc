"""Randomised checks of the host-side validation and planning (no GPU).

``ar_plan_query`` / ``ar_plan_query_add`` run every check ``ar_reduce`` makes
except the memory-kind lookups.  Here they are driven with random rank
counts, sizes, types, mode bits, pointer sets drawn from a few bases (so that
misalignment, exact in-place use, partial overlaps and NULL entries all come
up) and residuals, and compared with a statement of the rules of
``include/ar.h`` written out below with Python's exact integers.  Accepted
calls must also give a consistent plan: the resolved schedule, the number of
destinations, the chunking, per-rank slices that tile the tensor, the active
mask and the algorithmic byte count.
"""
from __future__ import annotations

import pytest
from hypothesis import HealthCheck, event, given, settings
from hypothesis import strategies as st

import mixed_precision_partial_amd as ar

F32, F16, BF16 = ar.AR_F32, ar.AR_F16, ar.AR_BF16
ELEM = {F32: 4, F16: 2, BF16: 2}
WAVE_TILE = 512                 # elements per wave tile: chunk and slice boundaries
MAX_LAUNCH = 1 << 30
SINGLE_SHOT_MAX = 1 << 20       # default AUTO threshold: wire bytes per rank at R = 2
SIZE_MAX = (1 << 64) - 1
MODE_BITS = ar.AR_MODE_MASK | ar.AR_SRC_WIRE | ar.AR_SRC_INACTIVE_NULL

INVALID, UNSUPPORTED = "invalid", "unsupported"


def overlap(a: int, na: int, b: int, nb: int) -> bool:
    return na > 0 and nb > 0 and a < b + nb and b < a + na


def expected(R, n, dst_type, wire_type, mode, dsts, srcs, host, res=None, res_len=0, contiguous=True):
    """(set of reasons the call must be refused, resolved mode or None).

    Each reason is INVALID or UNSUPPORTED, following the rules of include/ar.h.
    `contiguous` False leaves out the overlap checks (row-strided tensors span
    more than n elements; the caller checks them)."""
    why = set()
    if not 2 <= R <= 16:
        return {INVALID}, None
    if dst_type not in ELEM or wire_type not in ELEM:
        return {INVALID}, None
    if mode & ~MODE_BITS:
        return {INVALID}, None
    base = mode & ar.AR_MODE_MASK
    if base > ar.AR_MODE_HOST_STAGED:
        return {INVALID}, None
    if ELEM[wire_type] > ELEM[dst_type]:
        why.add(INVALID)
    if dst_type != F32 and wire_type != dst_type:
        why.add(UNSUPPORTED)
    narrow = dst_type != F32
    src_bytes = ELEM[wire_type] if (mode & ar.AR_SRC_WIRE or narrow) else ELEM[dst_type]
    dst_bytes = ELEM[dst_type]
    res_kind = 0
    if res is not None and n > 0:
        if res_len == 0 or res_len > n or n % res_len:
            why.add(INVALID)
        else:
            res_kind = 1 if res_len == n else 2
            if res_kind == 2 and (res_len % 8 or res_len > MAX_LAUNCH):
                why.add(UNSUPPORTED)
        if res % 16:
            why.add(INVALID)
    if base == ar.AR_MODE_AUTO:
        if host:
            resolved = ar.AR_MODE_HOST_STAGED
        elif R * n * ELEM[wire_type] < 2 * SINGLE_SHOT_MAX:
            resolved = ar.AR_MODE_SINGLE_SHOT
        else:
            resolved = ar.AR_MODE_CHUNKED
    else:
        resolved = base
    n_dst = R if resolved == ar.AR_MODE_RS_BCAST else 1
    for d in dsts[:n_dst]:
        if d is None or d % 16:
            why.add(INVALID)
    for s in srcs:
        if s is None:
            if not mode & ar.AR_SRC_INACTIVE_NULL:
                why.add(INVALID)
        elif s % 16:
            why.add(INVALID)
    if n > (SIZE_MAX // 8) // 16:
        why.add(INVALID)
    if n > 0 and not why and contiguous:
        dl, sl = n * dst_bytes, n * src_bytes
        rl = 0 if res_kind == 0 else (n if res_kind == 1 else res_len) * dst_bytes
        live = dsts[:n_dst]
        for i, d in enumerate(live):
            for e in live[i + 1:]:
                if overlap(d, dl, e, dl):
                    why.add(INVALID)
            for s in srcs:
                if s is not None and overlap(d, dl, s, sl) and not (s == d and src_bytes == dst_bytes):
                    why.add(INVALID)
            if res_kind and overlap(d, dl, res, rl) and not (res_kind == 1 and res == d):
                why.add(INVALID)
    return why, resolved


def check_plan(plan, R, n, dst_type, wire_type, mode, srcs, resolved, res_kind, res_len):
    narrow = dst_type != F32
    src_bytes = ELEM[wire_type] if (mode & ar.AR_SRC_WIRE or narrow) else ELEM[dst_type]
    n_dst = R if resolved == ar.AR_MODE_RS_BCAST else 1
    assert plan.mode == resolved
    assert plan.n_dst == n_dst
    assert plan.src_bytes == src_bytes and plan.wire_bytes == ELEM[wire_type]
    assert plan.dst_bytes == ELEM[dst_type]
    assert plan.active_mask == sum(1 << r for r, s in enumerate(srcs) if s is not None)
    assert plan.residual_kind == res_kind
    res_b = 0 if res_kind == 0 else (n if res_kind == 1 else res_len) * ELEM[dst_type]
    n_active = sum(s is not None for s in srcs)      # an inactive rank is not read
    assert plan.algo_bytes == n_active * n * src_bytes + n_dst * n * ELEM[dst_type] + res_b
    if n == 0:
        assert plan.n_chunks == 0
        return
    assert plan.chunk_elems >= 1
    assert plan.n_chunks == -(-n // plan.chunk_elems)
    # the two-rank contiguous kernels: exactly two active binary32 partials (not flagged as
    # wire-typed) into one binary32 destination, with or without a residual (kept stores, the
    # default for that shape), chunked or single-shot
    pair = (resolved in (ar.AR_MODE_CHUNKED, ar.AR_MODE_SINGLE_SHOT) and R == 2 and n_active == 2 and
            not mode & ar.AR_SRC_WIRE and dst_type == F32)
    # and the two-rank 16-bit kernel: two active 16-bit partials into their own type, no residual
    pair16 = (resolved in (ar.AR_MODE_CHUNKED, ar.AR_MODE_SINGLE_SHOT) and R == 2 and n_active == 2 and
              narrow and res_kind == 0)
    assert (plan.stream_kernel == 3) == (pair or pair16)
    # the kernels for a few active partials: two to four active binary32 partials (other than
    # the two-rank case) into one binary32 destination, no residual or an element-wise one,
    # kept stores
    few = (resolved in (ar.AR_MODE_CHUNKED, ar.AR_MODE_SINGLE_SHOT) and 2 <= n_active <= 4 and
           not (R == 2 and n_active == 2) and not mode & ar.AR_SRC_WIRE and dst_type == F32 and
           res_kind <= 1 and not plan.store_nt)
    assert (plan.stream_kernel == 4) == few
    # the default occupancy hold: the binary32 two-rank kernels, 18 waves, 14 with a residual,
    # and the kernels for a few active partials, 18, 14 or 10 for two, three or four (14, 10
    # or 8 with a residual)
    few_hold = ({2: 14, 3: 10, 4: 8} if res_kind else {2: 18, 3: 14, 4: 10}).get(n_active, 0)
    assert plan.hold_waves == ((14 if res_kind else 18) if pair else (few_hold if few else 0))
    if resolved == ar.AR_MODE_SINGLE_SHOT:
        assert plan.chunk_elems == n and plan.stream_kernel == (3 if pair or pair16 else 4 if few else 0)
    else:
        assert plan.chunk_elems % WAVE_TILE == 0 and plan.chunk_elems <= MAX_LAUNCH
        assert plan.stream_kernel in ((3,) if pair or pair16 else (4,) if few else (1, 2))
        if res_kind and not pair and not few:
            # with a residual: LDS-staged for the broadcast schedule, register-staged otherwise
            assert plan.stream_kernel == (2 if resolved == ar.AR_MODE_RS_BCAST else 1)
        if resolved == ar.AR_MODE_RS_BCAST:
            # the broadcast schedule is LDS-staged for every rank count and width
            assert plan.stream_kernel == 2
    if resolved == ar.AR_MODE_RS_BCAST:
        pos = 0
        for r in range(R):
            assert plan.slice_start[r] == pos
            assert pos % WAVE_TILE == 0
            pos += plan.slice_len[r]
        assert pos == n
    assert plan.host_direct == (1 if resolved == ar.AR_MODE_HOST_STAGED else 0)


@st.composite
def pointers(draw, k):
    """k destination and k source addresses: distinct, aligned and far apart,
    except that a third of the calls get one or two perturbations -- a
    misaligned address, a NULL source, or a tensor placed on or inside another
    (exact in-place use or a partial overlap)."""
    out = [(i + 1) << 36 for i in range(2 * k)]
    if draw(st.integers(0, 2)) == 0:
        for _ in range(draw(st.integers(1, 2))):
            i = draw(st.integers(0, 2 * k - 1))
            how = draw(st.integers(0, 3))
            if out[i] is None:
                continue
            if how == 0:
                out[i] += draw(st.sampled_from([4, 8, 2]))
            elif how == 1 and i >= k:
                out[i] = None
            else:
                j = draw(st.integers(0, 2 * k - 1))
                if j != i and out[j] is not None:
                    out[i] = out[j] + draw(st.sampled_from([0, 0, 16, 4096, 1 << 20]))
    return out[:k], out[k:]


@st.composite
def call(draw):
    """Mostly well-formed calls; each field is out of its domain once in ~12 draws."""
    def rare(valid, junk):
        return draw(junk) if draw(st.integers(0, 11)) == 0 else draw(valid)

    R = rare(st.one_of(st.integers(2, 16), st.sampled_from([2, 4, 8])), st.sampled_from([1, 17, 0, -1]))
    n = draw(st.one_of(st.integers(0, 5000), st.integers(0, 1 << 26),
                       st.sampled_from([1 << 18, (1 << 20) + 8, 1 << 30, (1 << 31) + 3, (1 << 40),
                                        SIZE_MAX // 64, SIZE_MAX // 4])))
    dst_type, wire_type = rare(
        st.sampled_from([(F32, F32), (F32, BF16), (F32, F16), (F16, F16), (BF16, BF16)]),
        st.tuples(st.sampled_from([F32, F16, BF16, 3, -1]), st.sampled_from([F32, F16, BF16, 7])))
    base = rare(st.integers(0, 4), st.sampled_from([5, 255]))
    flags = rare(st.sampled_from([0, ar.AR_SRC_WIRE, ar.AR_SRC_INACTIVE_NULL,
                                  ar.AR_SRC_WIRE | ar.AR_SRC_INACTIVE_NULL]),
                 st.sampled_from([0x400, 1 << 31]))
    k = max(R, 1) if R <= 16 else 16
    dsts, srcs = draw(pointers(k))
    host = draw(st.booleans())
    return R, n, dst_type, wire_type, base | flags, dsts, srcs, host


SETTINGS = settings(max_examples=1500, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def run_case(rc, plan, R, n, dst_type, wire_type, mode, srcs, why, resolved, res_kind=0, res_len=0):
    event(f"status {ar.ar_status_str(rc)}" + (f", mode {plan.mode}" if rc == ar.AR_OK else ""))
    if not why:
        assert rc == ar.AR_OK, f"refused a valid call: {ar.ar_status_str(rc)}"
        check_plan(plan, R, n, dst_type, wire_type, mode, srcs, resolved, res_kind, res_len)
    elif why == {UNSUPPORTED}:
        assert rc == ar.AR_ERR_UNSUPPORTED
    elif why == {INVALID}:
        assert rc == ar.AR_ERR_INVALID
    else:
        assert rc in (ar.AR_ERR_INVALID, ar.AR_ERR_UNSUPPORTED)


@SETTINGS
@given(call())
def test_plan_query_matches_rules(args):
    R, n, dst_type, wire_type, mode, dsts, srcs, host = args
    rc, plan = ar.ar_plan_query(dsts, srcs, n, dst_type, wire_type, mode, srcs_on_host=host,
                                R=max(R, 0) if R <= 16 else R)
    why, resolved = expected(R, n, dst_type, wire_type, mode, dsts, srcs[:max(R, 0)], host)
    run_case(rc, plan, R, n, dst_type, wire_type, mode, srcs[:max(R, 0)], why, resolved)


@SETTINGS
@given(call(), st.data())
def test_plan_query_add_matches_rules(args, data):
    R, n, dst_type, wire_type, mode, dsts, srcs, host = args
    # mostly a tensor of its own; sometimes misaligned, the destination itself, or inside it
    res = data.draw(st.sampled_from([40 << 36] * 5 + [(40 << 36) + 8, dsts[0], dsts[0] + 64]))
    choices = [n, n, n, 0, 8, 4096, 12, n + 8]
    if n > 0:
        choices += [n // 2, n // 8]
    res_len = data.draw(st.sampled_from(choices))
    rc, plan = ar.ar_plan_query_add(dsts, srcs, n, dst_type, wire_type, mode, res, res_len,
                                    srcs_on_host=host, R=max(R, 0) if R <= 16 else R)
    why, resolved = expected(R, n, dst_type, wire_type, mode, dsts, srcs[:max(R, 0)], host, res, res_len)
    res_kind = 0 if n == 0 else (1 if res_len == n else 2)
    run_case(rc, plan, R, n, dst_type, wire_type, mode, srcs[:max(R, 0)], why, resolved, res_kind, res_len)


@pytest.mark.parametrize("a,na,b,nb", [
    (SIZE_MAX - 15, 16, 16, 16),           # a range ending at the top of the address space
    (16, 16, SIZE_MAX - 15, 16),
    (SIZE_MAX - 31, 32, SIZE_MAX - 15, 8),
])
def test_overlap_near_the_top_of_the_address_space(a, na, b, nb):
    """Destination / source ranges that reach the top of the 64-bit space: the
    overlap test must not wrap (a wrapped sum would hide a real overlap)."""
    n = na // 4
    rc, _ = ar.ar_plan_query([a], [b, 1 << 33], n, F32, F32, ar.AR_MODE_CHUNKED)
    want = ar.AR_ERR_INVALID if overlap(a, na, b, nb) and a != b else ar.AR_OK
    assert rc == want


def extent(rows: int, cols: int, stride: int) -> int:
    return 0 if rows == 0 or cols == 0 else (rows - 1) * stride + cols


def expected_rows(R, rows, cols, ss, ds, rs, dst_type, wire_type, mode, dsts, srcs, host, res):
    """Refusal reasons for ar_plan_query_rows (row-strided tensors, rules of include/ar.h)."""
    if cols and rows > SIZE_MAX // cols:
        return {INVALID}, None
    if rows > 1 and any(st_ > (SIZE_MAX // 16) // rows for st_ in (ss, ds, rs)):
        return {INVALID}, None
    n = rows * cols
    why, resolved = expected(R, n, dst_type, wire_type, mode, dsts, srcs, host, contiguous=False)
    if resolved is None:
        return why, None
    narrow = dst_type != F32
    src_bytes = ELEM[wire_type] if (mode & ar.AR_SRC_WIRE or narrow) else ELEM[dst_type]
    dst_bytes = ELEM[dst_type]
    if ss < cols or ds < cols or (ss * src_bytes) % 16 or (ds * dst_bytes) % 16:
        why.add(INVALID)
    if cols > MAX_LAUNCH:
        why.add(UNSUPPORTED)
    res_kind = 0
    if res is not None and n > 0:
        if (rs != 0 and rs < cols) or (rs * dst_bytes) % 16 or res % 16:
            why.add(INVALID)
        res_kind = 2 if rs == 0 else 1
    if n > 0 and not why:
        n_dst = R if resolved == ar.AR_MODE_RS_BCAST else 1
        dl, sl = extent(rows, cols, ds) * dst_bytes, extent(rows, cols, ss) * src_bytes
        rl = 0 if res_kind == 0 else (cols if res_kind == 2 else extent(rows, cols, rs)) * dst_bytes
        live = dsts[:n_dst]
        for i, d in enumerate(live):
            for e in live[i + 1:]:
                if overlap(d, dl, e, dl):
                    why.add(INVALID)
            for s in srcs:
                if s is not None and overlap(d, dl, s, sl) and not (s == d and src_bytes == dst_bytes and ss == ds):
                    why.add(INVALID)
            if res_kind and overlap(d, dl, res, rl) and not (res_kind == 1 and res == d and rs == ds):
                why.add(INVALID)
    return why, (resolved, res_kind)


@st.composite
def row_shape(draw):
    rows = draw(st.one_of(st.integers(0, 300), st.sampled_from([1, 2, 65535, 65536, 70000, 1 << 40])))
    cols = draw(st.one_of(st.integers(0, 5000), st.sampled_from([8, 4096, (1 << 30) + 8, 1 << 50])))

    def stride():
        pad = draw(st.one_of(st.integers(0, 64), st.sampled_from([0, 0, 512, 1 << 20])))
        s = cols + pad
        if draw(st.integers(0, 3)):
            s = -(-s // 8) * 8          # usually a 16-byte row pitch for both element widths
        if draw(st.integers(0, 15)) == 0:
            s = max(0, cols - 8)       # rows that would overlap
        return s

    return rows, cols, stride(), stride(), draw(st.sampled_from([0, 0, stride(), stride()]))


@SETTINGS
@given(call(), row_shape(), st.data())
def test_plan_query_rows_matches_rules(args, shape, data):
    R, _, dst_type, wire_type, mode, dsts, srcs, host = args
    rows, cols, ss, ds, rs = shape
    res = data.draw(st.sampled_from([None, None, 40 << 36, 40 << 36, (40 << 36) + 8, dsts[0]]))
    rc, plan = ar.ar_plan_query_rows(dsts, srcs, rows, cols, ss, ds, dst_type, wire_type, mode, residual=res,
                                     res_stride=rs, srcs_on_host=host, R=max(R, 0) if R <= 16 else R)
    live_srcs = srcs[:max(R, 0)]
    why, out = expected_rows(R, rows, cols, ss, ds, rs, dst_type, wire_type, mode, dsts, live_srcs, host, res)
    event(f"status {ar.ar_status_str(rc)}")
    if why:
        if why == {UNSUPPORTED}:
            assert rc == ar.AR_ERR_UNSUPPORTED
        elif why == {INVALID}:
            assert rc == ar.AR_ERR_INVALID
        else:
            assert rc in (ar.AR_ERR_INVALID, ar.AR_ERR_UNSUPPORTED)
        return
    assert rc == ar.AR_OK, f"refused a valid call: {ar.ar_status_str(rc)}"
    resolved, res_kind = out
    n = rows * cols
    narrow = dst_type != F32
    src_bytes = ELEM[wire_type] if (mode & ar.AR_SRC_WIRE or narrow) else ELEM[dst_type]
    n_dst = R if resolved == ar.AR_MODE_RS_BCAST else 1
    assert plan.mode == resolved and plan.n_dst == n_dst
    assert plan.residual_kind == (res_kind if n > 0 else 0)
    res_b = 0 if n == 0 or res_kind == 0 else (n if res_kind == 1 else cols) * ELEM[dst_type]
    n_active = sum(s is not None for s in live_srcs)
    assert plan.algo_bytes == n_active * n * src_bytes + n_dst * n * ELEM[dst_type] + res_b
    assert all(plan.slice_start[r] == 0 and plan.slice_len[r] == 0 for r in range(16))
    if n == 0:
        assert plan.n_chunks == 0
        return
    # the two-rank row-strided kernels: two active binary32 partials into one binary32
    # destination, rows of whole wave tiles, strides below 2^32 elements
    pair = (resolved in (ar.AR_MODE_CHUNKED, ar.AR_MODE_SINGLE_SHOT) and R == 2 and n_active == 2 and
            not mode & ar.AR_SRC_WIRE and dst_type == F32 and cols % WAVE_TILE == 0 and
            max(ss, ds, rs) < (1 << 32))
    assert (plan.stream_kernel == 3) == pair
    assert plan.hold_waves == ((14 if res_kind else 18) if pair else 0)
    # device schedules: one range per row; host-staged copies move whole rows
    assert plan.chunk_elems % cols == 0
    chunk_rows = plan.chunk_elems // cols
    assert chunk_rows >= 1 and plan.chunk_elems <= max(MAX_LAUNCH, cols)
    if resolved != ar.AR_MODE_HOST_STAGED:
        assert chunk_rows == 1
    assert plan.n_chunks == -(-rows // chunk_rows)
