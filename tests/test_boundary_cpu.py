"""C-ABI boundary checks that need no GPU: the library loads, exports every
declared entry point, and its host-side validation / planning behaves as
``include/ar.h`` states.  No compute call is made here."""
import ctypes
import os
import re

import pytest

import mixed_precision_partial_amd as ar

MiB = 1 << 20
# Well separated fake addresses: validation never dereferences them.
A = [0x10_0000_0000 + i * 0x1_0000_0000 for i in range(40)]


def declared_functions():
    text = open(ar.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ar_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = ar.load_library()
    names = declared_functions()
    assert {"ar_init", "ar_reduce", "ar_reduce_add", "ar_reduce_rows", "ar_free", "ar_status_str",
            "ar_plan_query", "ar_plan_query_add", "ar_plan_query_rows"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in ar.h but not exported"


def test_exports_nothing_else():
    out = os.popen(f"nm -D --defined-only {ar.LIB_PATH}").read()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions())


def test_status_strings():
    assert ar.ar_status_str(ar.AR_OK) == "AR_OK"
    assert ar.ar_status_str(ar.AR_ERR_INVALID) == "AR_ERR_INVALID"
    assert ar.ar_status_str(ar.AR_ERR_UNSUPPORTED) == "AR_ERR_UNSUPPORTED"
    assert ar.ar_status_str(ar.AR_ERR_NOMEM) == "AR_ERR_NOMEM"
    assert ar.ar_status_str(ar.AR_ERR_RUNTIME) == "AR_ERR_RUNTIME"
    assert ar.ar_status_str(1234) == "AR_ERR_UNKNOWN"


def test_struct_layouts_match_header():
    # six ints, xcd_run_elems, then occupancy_hold padded to 8
    assert ctypes.sizeof(ar.ArConfig) == 3 * 8 + 6 * 4 + 8 + 8
    assert ctypes.sizeof(ar.ArPlan) == 4 * 4 + 2 * 8 + 2 * 16 * 8 + 8 + 4 * 4 + 3 * 4 + 4


def q(n, R=2, mode=ar.AR_MODE_AUTO, wire=ar.AR_BF16, dst_type=ar.AR_F32, dsts=None, srcs=None,
      host=False, config=None):
    srcs = A[1:1 + R] if srcs is None else srcs
    dsts = [A[20 + d] for d in range(R)] if dsts is None else dsts
    return ar.ar_plan_query(dsts, srcs, n, dst_type, wire, mode, host, config, R=len(srcs))


def test_rank_count_bounds():
    assert q(4096, R=2)[0] == ar.AR_OK
    assert q(4096, R=16)[0] == ar.AR_OK
    assert q(4096, srcs=A[1:2])[0] == ar.AR_ERR_INVALID
    assert q(4096, srcs=A[1:18])[0] == ar.AR_ERR_INVALID


def test_type_checks():
    assert q(64, wire=7)[0] == ar.AR_ERR_INVALID
    assert q(64, dst_type=9)[0] == ar.AR_ERR_INVALID
    # a wire wider than the destination is invalid; a narrow destination needs its own wire type
    assert q(64, dst_type=ar.AR_F16, wire=ar.AR_F32)[0] == ar.AR_ERR_INVALID
    assert q(64, dst_type=ar.AR_F16, wire=ar.AR_BF16)[0] == ar.AR_ERR_UNSUPPORTED
    assert q(64, dst_type=ar.AR_BF16, wire=ar.AR_F16)[0] == ar.AR_ERR_UNSUPPORTED
    assert q(64, dst_type=ar.AR_F16, wire=ar.AR_F16)[0] == ar.AR_OK
    assert q(64, dst_type=ar.AR_BF16, wire=ar.AR_BF16)[0] == ar.AR_OK


def test_mode_and_flag_checks():
    assert q(64, mode=5)[0] == ar.AR_ERR_INVALID
    assert q(64, mode=ar.AR_MODE_CHUNKED | 0x400)[0] == ar.AR_ERR_INVALID
    assert q(64, mode=ar.AR_MODE_CHUNKED | 0x10000)[0] == ar.AR_ERR_INVALID
    assert q(64, mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_WIRE)[0] == ar.AR_OK


def test_null_and_alignment():
    assert ar.ar_plan_query(None, A[1:3], 64, R=2)[0] == ar.AR_ERR_INVALID
    assert ar.ar_plan_query([A[20]], None, 64, R=2)[0] == ar.AR_ERR_INVALID
    assert q(64, srcs=[A[1], 0])[0] == ar.AR_ERR_INVALID
    assert q(64, dsts=[0])[0] == ar.AR_ERR_INVALID
    assert q(64, srcs=[A[1], A[2] + 8])[0] == ar.AR_ERR_INVALID
    assert q(64, dsts=[A[20] + 4])[0] == ar.AR_ERR_INVALID
    assert q(64, srcs=[A[1], A[2] + 16])[0] == ar.AR_OK


def test_overlap_rules():
    n = 1 << 20
    # exactly in place with fp32 sources: allowed
    assert q(n, mode=ar.AR_MODE_CHUNKED, dsts=[A[1]], srcs=[A[1], A[2]])[0] == ar.AR_OK
    assert q(n, mode=ar.AR_MODE_CHUNKED, dsts=[A[2]], srcs=[A[1], A[2]])[0] == ar.AR_OK
    # partial overlap: invalid
    assert q(n, mode=ar.AR_MODE_CHUNKED, dsts=[A[1] + 4096], srcs=[A[1], A[2]])[0] == ar.AR_ERR_INVALID
    # in place with wire-typed sources (different widths): invalid
    assert q(n, mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_WIRE, dsts=[A[1]], srcs=[A[1], A[2]])[0] == ar.AR_ERR_INVALID
    # destinations overlapping each other (broadcast schedule): invalid
    d = [A[20], A[20] + 4 * n - 16]
    assert q(n, mode=ar.AR_MODE_RS_BCAST, dsts=d)[0] == ar.AR_ERR_INVALID
    # sources may alias each other (read only)
    assert q(n, mode=ar.AR_MODE_CHUNKED, srcs=[A[1], A[1]])[0] == ar.AR_OK
    # n = 0: nothing overlaps
    assert q(0, mode=ar.AR_MODE_CHUNKED, dsts=[A[1] + 16], srcs=[A[1], A[2]])[0] == ar.AR_OK


def test_auto_mode_threshold():
    # below 1 MiB of wire bytes per rank -> single shot, else chunked
    rc, p = q(4096, wire=ar.AR_F32)
    assert rc == ar.AR_OK and p.mode == ar.AR_MODE_SINGLE_SHOT and p.n_chunks == 1
    rc, p = q((1 * MiB) // 2 - 1, wire=ar.AR_BF16)
    assert p.mode == ar.AR_MODE_SINGLE_SHOT
    rc, p = q((1 * MiB) // 2, wire=ar.AR_BF16)
    assert p.mode == ar.AR_MODE_CHUNKED
    rc, p = q(4096, host=True)
    assert p.mode == ar.AR_MODE_HOST_STAGED
    rc, p = q(4096, config={"single_shot_max_bytes": 1024})
    assert p.mode == ar.AR_MODE_CHUNKED
    # more ranks: the limit applies to the wire bytes of all ranks (2 MiB at the default)
    rc, p = q((2 * MiB) // (8 * 2) - 1, R=8, wire=ar.AR_BF16)
    assert p.mode == ar.AR_MODE_SINGLE_SHOT
    rc, p = q((2 * MiB) // (8 * 2), R=8, wire=ar.AR_BF16)
    assert p.mode == ar.AR_MODE_CHUNKED


def test_prefill_chunk_plan():
    # 2048 x 4096 with a bf16 wire in 4 MiB chunks of wire bytes per rank -> 4 chunks of 2 Mi elements
    n = 2048 * 4096
    rc, p = q(n, mode=ar.AR_MODE_CHUNKED, wire=ar.AR_BF16)
    assert rc == ar.AR_OK
    assert p.chunk_elems == 2 * MiB and p.n_chunks == 4
    assert p.algo_bytes == 2 * n * 4 + n * 4 == 100_663_296
    rc, p = q(n, mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_WIRE, wire=ar.AR_BF16)
    assert p.src_bytes == 2 and p.algo_bytes == 2 * n * 2 + n * 4


def test_slice_plan_partitions_range():
    for n, R in [(2048 * 8192, 4), (100_003, 3), (1000, 8), (7, 2), (513 * 16 + 5, 16)]:
        rc, p = q(n, R=R, mode=ar.AR_MODE_RS_BCAST)
        assert rc == ar.AR_OK and p.n_dst == R
        pos = 0
        for r in range(R):
            assert p.slice_start[r] == pos
            assert p.slice_start[r] % 512 == 0
            pos += p.slice_len[r]
        assert pos == n
    rc, p = q(2048 * 8192, R=4, mode=ar.AR_MODE_RS_BCAST, wire=ar.AR_F16)
    assert [p.slice_len[r] for r in range(4)] == [2048 * 8192 // 4] * 4
    assert p.algo_bytes == 4 * 2048 * 8192 * 4 * 2 == 536_870_912


def test_host_chunk_heuristic():
    # clamp(bytes / 2, 512 KiB, 64 MiB) of source bytes per rank
    n = 8192 * 8192
    rc, p = q(n, R=8, mode=ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE, wire=ar.AR_BF16)
    assert p.chunk_elems == (n * 2 // 2) // 2 and p.n_chunks == 2
    rc, p = q(4 * n, R=8, mode=ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE, wire=ar.AR_BF16)
    assert p.chunk_elems == (64 * MiB) // 2
    rc, p = q(100_000, mode=ar.AR_MODE_HOST_STAGED)
    assert p.chunk_elems == (512 * 1024) // 4
    rc, p = q(n, mode=ar.AR_MODE_HOST_STAGED, config={"host_chunk_bytes": 1 << 16})
    assert p.chunk_elems == (1 << 16) // 4
    # direct reads of the pinned buffers by default; the copy-engine pipeline on request
    assert q(n, R=8, mode=ar.AR_MODE_HOST_STAGED)[1].host_direct == 1
    assert q(n, R=8, mode=ar.AR_MODE_HOST_STAGED, config={"host_path": 2})[1].host_direct == 1
    assert q(n, R=8, mode=ar.AR_MODE_HOST_STAGED, config={"host_path": 1})[1].host_direct == 0
    assert q(n, R=8, mode=ar.AR_MODE_CHUNKED)[1].host_direct == 0


def test_bad_config_rejected():
    assert q(64, config={"host_slots": -1})[0] == ar.AR_ERR_INVALID
    assert q(64, config={"stream_kernel": 3})[0] == ar.AR_ERR_INVALID
    assert q(64, config={"grid_wgs": -2})[0] == ar.AR_ERR_INVALID


def test_zero_elements_is_ok():
    rc, p = q(0, mode=ar.AR_MODE_CHUNKED)
    assert rc == ar.AR_OK and p.n_chunks == 0 and p.algo_bytes == 0


def test_ar_free_null_and_init_errors():
    assert ar.load_library().ar_free(None) == ar.AR_OK
    out = ctypes.c_void_p()
    assert ar.load_library().ar_init(None, 0, None) == ar.AR_ERR_INVALID
    bad = ar.ArConfig(host_slots=-3)
    assert ar.load_library().ar_init(ctypes.byref(out), 0, ctypes.byref(bad)) == ar.AR_ERR_INVALID
    assert out.value is None


@pytest.mark.parametrize("rank", [2, 5, 16])
def test_reduce_rejects_before_runtime(rank):
    # a NULL context is rejected without touching the GPU
    lib = ar.load_library()
    srcs = (ctypes.c_void_p * rank)(*A[1:1 + rank])
    dsts = (ctypes.c_void_p * 1)(A[30])
    assert lib.ar_reduce(None, dsts, srcs, rank, 64, ar.AR_F32, ar.AR_BF16, 0, None) == ar.AR_ERR_INVALID


def test_store_policy_rule():
    n = 2048 * 4096
    # fp32 sources, R=2, one destination: reads dominate -> cached stores
    assert q(n, mode=ar.AR_MODE_CHUNKED)[1].store_nt == 0
    # 16-bit sources, R=2: as many bytes written as read -> streaming stores
    assert q(n, mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_WIRE)[1].store_nt == 1
    # broadcast to every rank -> streaming stores
    assert q(n, R=4, mode=ar.AR_MODE_RS_BCAST, wire=ar.AR_F16)[1].store_nt == 1
    # explicit policies win
    assert q(n, mode=ar.AR_MODE_CHUNKED, config={"store_policy": 2})[1].store_nt == 1
    assert q(n, R=4, mode=ar.AR_MODE_RS_BCAST, config={"store_policy": 1})[1].store_nt == 0
    assert q(64, config={"store_policy": 3})[0] == ar.AR_ERR_INVALID


def test_stream_kernel_choice():
    """The automatic family follows the measured table: CHUNKED fp32 sources register-staged;
    16-bit sources LDS-staged at R = 2 and 5..8 into binary32, at R = 2 and 6..8 into a narrow
    destination; the broadcast schedule LDS-staged; with a residual LDS-staged only for the
    broadcast schedule; host-staged calls
    LDS-staged for two 16-bit sources only; two active fp32 sources into one contiguous fp32
    destination, with or without a residual, kept stores and no forced grid take the two-rank
    contiguous kernels (3), chunked or single-shot; two to four active fp32 sources otherwise
    (three or four ranks, or inactive ones among more), no residual, contiguous, the same
    conditions, take the kernels for a few active partials (4)."""
    n = 2048 * 4096
    CH, BC, HS, SW = ar.AR_MODE_CHUNKED, ar.AR_MODE_RS_BCAST, ar.AR_MODE_HOST_STAGED, ar.AR_SRC_WIRE
    # single-shot: the two-rank kernel for its case, the single-shot kernel otherwise
    assert q(4096, mode=ar.AR_MODE_SINGLE_SHOT)[1].stream_kernel == 3
    assert q(4096, mode=ar.AR_MODE_AUTO)[1].stream_kernel == 3          # AUTO resolves to SINGLE_SHOT
    assert q(4096, R=3, mode=ar.AR_MODE_SINGLE_SHOT)[1].stream_kernel == 4
    assert q(4096, R=5, mode=ar.AR_MODE_SINGLE_SHOT)[1].stream_kernel == 0
    assert q(4096, mode=ar.AR_MODE_SINGLE_SHOT | ar.AR_SRC_WIRE)[1].stream_kernel == 0
    assert q(4096, mode=ar.AR_MODE_SINGLE_SHOT, config={"stream_kernel": 1})[1].stream_kernel == 0
    assert q(4096, mode=ar.AR_MODE_SINGLE_SHOT, config={"grid_wgs": 3})[1].stream_kernel == 0
    for R in (2, 3, 4, 5, 8, 16):
        assert q(n, R=R, mode=CH)[1].stream_kernel == {2: 3, 3: 4, 4: 4}.get(R, 1), R
    # the two-rank kernel only for its exact case: every wire type, automatic choice only
    for wire in (ar.AR_F32, ar.AR_F16, ar.AR_BF16):
        assert q(n, mode=CH, wire=wire)[1].stream_kernel == 3
        assert q(n, mode=ar.AR_MODE_AUTO, wire=wire)[1].stream_kernel == 3   # AUTO resolves to CHUNKED
    assert q(4097, mode=CH)[1].stream_kernel == 3
    assert q(n, mode=CH, config={"stream_kernel": 1})[1].stream_kernel == 1
    assert q(n, mode=CH, config={"grid_wgs": 7})[1].stream_kernel == 1
    assert q(n, mode=CH, config={"store_policy": 2})[1].stream_kernel == 1
    assert q(n, srcs=[A[1], 0], mode=CH | ar.AR_SRC_INACTIVE_NULL)[1].stream_kernel == 1
    # two to four active fp32 partials among any rank count, automatic choice only, held
    IN = CH | ar.AR_SRC_INACTIVE_NULL
    for srcs in ([A[1], A[2], 0, A[4]], [0, A[2], A[3]], [A[1], 0, 0, 0, 0, 0, 0, A[8]],
                 [0, A[2], 0, A[4], A[5], 0, A[7], 0], [A[i] for i in range(1, 5)]):
        rc, p = q(n, srcs=srcs, mode=IN)
        held = {2: 18, 3: 14, 4: 10}[sum(1 for x in srcs if x)]
        assert rc == ar.AR_OK and p.stream_kernel == 4 and p.hold_waves == held, srcs
        assert q(n, srcs=srcs, mode=IN, config={"stream_kernel": 1})[1].stream_kernel == 1
        assert q(n, srcs=srcs, mode=IN, config={"grid_wgs": 7})[1].stream_kernel == 1
        assert q(n, srcs=srcs, mode=IN, config={"store_policy": 2})[1].stream_kernel == 1
        assert q(n, srcs=srcs, mode=IN, config={"occupancy_hold": -1})[1].hold_waves == 0
    for srcs in ([A[1], 0, 0, 0], [0, A[2], A[3], A[4], A[5], A[6]], [A[i] for i in range(1, 6)]):
        assert q(n, srcs=srcs, mode=IN)[1].stream_kernel == 1, srcs
    assert q(n, R=3, mode=CH | ar.AR_SRC_WIRE)[1].stream_kernel == 1
    assert q(n, R=3, mode=CH, wire=ar.AR_BF16, dst_type=ar.AR_BF16)[1].stream_kernel != 4
    assert q(n, R=3, mode=ar.AR_MODE_SINGLE_SHOT)[1].stream_kernel == 4
    # with a residual (element-wise or a broadcast row): the two-rank kernels for R = 2
    # CHUNKED; for R = 3 the kernel for a few active partials with an element-wise one (held
    # to 10 waves), the general kernels with a row
    res = [0x7_0000_0000]
    for res_len in (n, 4096):
        rc, p = ar.ar_plan_query_add(A[20:21], A[1:3], n, ar.AR_F32, ar.AR_BF16, CH, res[0], res_len)
        assert rc == ar.AR_OK and p.stream_kernel == 3 and p.residual_kind == (1 if res_len == n else 2)
        rc, p = ar.ar_plan_query_add(A[20:21], A[1:4], n, ar.AR_F32, ar.AR_BF16, CH, res[0], res_len)
        assert rc == ar.AR_OK and p.stream_kernel == (4 if res_len == n else 1)
        assert p.hold_waves == (10 if res_len == n else 0)
        rc, p = ar.ar_plan_query_add(A[20:22], A[1:3], n, ar.AR_F32, ar.AR_BF16, BC, res[0], res_len)
        assert rc == ar.AR_OK and p.stream_kernel == 2
    # row-strided: the two-rank kernels when every row is whole wave tiles
    rc, p = ar.ar_plan_query_rows(A[20:21], A[1:3], 2048, 4096, 4608, 4352, ar.AR_F32, ar.AR_BF16, CH,
                                  residual=res[0], res_stride=0)
    assert rc == ar.AR_OK and p.stream_kernel == 3
    rc, p = ar.ar_plan_query_rows(A[20:21], A[1:3], 2048, 4100, 4608, 4352, ar.AR_F32, ar.AR_BF16, CH,
                                  residual=res[0], res_stride=0)
    assert rc == ar.AR_OK and p.stream_kernel == 1
    rc, p = ar.ar_plan_query_rows(A[20:21], A[1:4], 2048, 4096, 4608, 4352, ar.AR_F32, ar.AR_BF16, CH)
    assert rc == ar.AR_OK and p.stream_kernel == 1
    # two 16-bit partials into their own type, no residual: the two-rank 16-bit kernel,
    # contiguous and unheld; with a residual the register-staged kernel (the residual rule),
    # row-strided the LDS-staged one (R = 2 in the table)
    for wire in (ar.AR_BF16, ar.AR_F16):
        for mode in (CH, ar.AR_MODE_SINGLE_SHOT):
            rc, p = q(n if mode == CH else 4097, mode=mode, wire=wire, dst_type=wire)
            assert rc == ar.AR_OK and p.stream_kernel == 3 and p.hold_waves == 0, (wire, mode)
        rc, p = ar.ar_plan_query_add(A[20:21], A[1:3], n, wire, wire, CH, res[0], n)
        assert rc == ar.AR_OK and p.stream_kernel == 1
        rc, p = ar.ar_plan_query_rows(A[20:21], A[1:3], 2048, 4096, 4608, 4352, wire, wire, CH)
        assert rc == ar.AR_OK and p.stream_kernel == 2
        assert q(n, mode=CH, wire=wire, dst_type=wire, config={"occupancy_hold": 12})[1].hold_waves == 12
    for R in range(2, 17):
        want16 = 2 if R in (2, 5, 6, 7, 8) else 1
        wantn = 3 if R == 2 else (2 if R in (6, 7, 8) else 1)
        assert q(n, R=R, mode=CH | SW)[1].stream_kernel == want16, R
        assert q(n, R=R, mode=CH, wire=ar.AR_BF16, dst_type=ar.AR_BF16)[1].stream_kernel == wantn, R
        assert q(n, R=R, mode=BC, wire=ar.AR_F16)[1].stream_kernel == 2, R
        assert q(n, R=R, mode=BC | SW, wire=ar.AR_F16)[1].stream_kernel == 2, R
        assert q(n, R=R, mode=BC, wire=ar.AR_F16, dst_type=ar.AR_F16)[1].stream_kernel == 2, R
        assert q(n, R=R, mode=HS | SW, host=True)[1].stream_kernel == (2 if R == 2 else 1), R
        assert q(n, R=R, mode=HS, host=True)[1].stream_kernel == 1, R
    # an explicit choice wins
    assert q(n, mode=CH | SW, config={"stream_kernel": 1})[1].stream_kernel == 1
    assert q(n, mode=CH, config={"stream_kernel": 2})[1].stream_kernel == 2


def test_inactive_ranks_flag():
    n = 1 << 20
    srcs = [A[1], 0, A[3]]
    # NULL is invalid without the flag
    assert q(n, srcs=srcs, mode=ar.AR_MODE_CHUNKED)[0] == ar.AR_ERR_INVALID
    rc, p = q(n, srcs=srcs, mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_INACTIVE_NULL)
    assert rc == ar.AR_OK and p.active_mask == 0b101
    # inactive ranks are not read: two sources' bytes plus the destination's
    assert p.algo_bytes == 2 * n * 4 + n * 4
    # the store policy weighs the call's shape (3 ranks against 1 destination): kept
    assert p.store_nt == 0
    rc, p = q(n, srcs=[A[1], 0], mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_INACTIVE_NULL)
    assert rc == ar.AR_OK and p.algo_bytes == n * 4 + n * 4 and p.store_nt == 0
    rc, p = q(n, srcs=[0, 0], mode=ar.AR_MODE_RS_BCAST | ar.AR_SRC_INACTIVE_NULL)
    assert rc == ar.AR_OK and p.active_mask == 0 and p.n_dst == 2 and p.algo_bytes == 2 * n * 4
    rc, p = q(n, mode=ar.AR_MODE_CHUNKED)
    assert p.active_mask == 0b11
    # a NULL destination stays invalid
    assert q(n, dsts=[0], srcs=srcs, mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_INACTIVE_NULL)[0] == ar.AR_ERR_INVALID


def test_narrow_destination_plan():
    n = 2048 * 4096
    for t in (ar.AR_F16, ar.AR_BF16):
        # sources hold the destination type with or without AR_SRC_WIRE
        for flags in (0, ar.AR_SRC_WIRE):
            rc, p = q(n, mode=ar.AR_MODE_CHUNKED | flags, wire=t, dst_type=t)
            assert rc == ar.AR_OK
            assert p.src_bytes == 2 and p.dst_bytes == 2 and p.algo_bytes == 2 * n * 2 + n * 2
        rc, p = q(n, R=4, mode=ar.AR_MODE_RS_BCAST, wire=t, dst_type=t)
        assert p.n_dst == 4 and p.algo_bytes == 4 * n * 2 + 4 * n * 2
    rc, p = q(n, mode=ar.AR_MODE_CHUNKED)
    assert p.dst_bytes == 4
    # in place is allowed for equal widths
    assert q(n, mode=ar.AR_MODE_CHUNKED, wire=ar.AR_F16, dst_type=ar.AR_F16, dsts=[A[1]],
             srcs=[A[1], A[2]])[0] == ar.AR_OK
    # the destination is n * 2 bytes long: a destination just past the end of a source is fine
    assert q(n, mode=ar.AR_MODE_CHUNKED, wire=ar.AR_F16, dst_type=ar.AR_F16, dsts=[A[1] + 2 * n],
             srcs=[A[1], A[2]])[0] == ar.AR_OK
    assert q(n, mode=ar.AR_MODE_CHUNKED, wire=ar.AR_F16, dst_type=ar.AR_F16, dsts=[A[1] + 2 * n - 16],
             srcs=[A[1], A[2]])[0] == ar.AR_ERR_INVALID


def qa(n, res, res_len, R=2, mode=ar.AR_MODE_CHUNKED, wire=ar.AR_BF16, dst_type=ar.AR_F32, dsts=None,
       srcs=None, config=None):
    srcs = A[1:1 + R] if srcs is None else srcs
    dsts = [A[20 + d] for d in range(R)] if dsts is None else dsts
    return ar.ar_plan_query_add(dsts, srcs, n, dst_type, wire, mode, res, res_len, False, config,
                                R=len(srcs))


def test_residual_rules():
    n = 2048 * 4096
    rc, p = qa(n, A[35], n)
    assert rc == ar.AR_OK and p.residual_kind == 1 and p.algo_bytes == 2 * n * 4 + n * 4 + n * 4
    rc, p = qa(n, A[35], 4096)
    assert rc == ar.AR_OK and p.residual_kind == 2 and p.algo_bytes == 2 * n * 4 + n * 4 + 4096 * 4
    # NULL residual, zero length, a length that does not divide n, or longer than n
    assert qa(n, 0, n)[0] == ar.AR_ERR_INVALID
    assert qa(n, A[35], 0)[0] == ar.AR_ERR_INVALID
    assert qa(n, A[35], 4095)[0] == ar.AR_ERR_INVALID
    assert qa(n, A[35], 2 * n)[0] == ar.AR_ERR_INVALID
    # a broadcast row must be a multiple of 8 elements
    assert qa(4 * 12, A[35], 12)[0] == ar.AR_ERR_UNSUPPORTED
    assert qa(4 * 16, A[35], 16)[0] == ar.AR_OK
    # misaligned residual
    assert qa(n, A[35] + 8, n)[0] == ar.AR_ERR_INVALID
    # element-wise residual may be the destination itself (x += reduce); a row may not
    assert qa(n, A[20], n)[0] == ar.AR_OK
    assert qa(n, A[20] + 16, n)[0] == ar.AR_ERR_INVALID
    assert qa(n, A[20], 4096)[0] == ar.AR_ERR_INVALID
    # and it may overlap the sources (read only)
    assert qa(n, A[1], n)[0] == ar.AR_OK
    # with a residual: register-staged automatically (even for two 16-bit sources), LDS-staged
    # for the broadcast schedule, and an explicit choice is honoured
    rc, p = qa(n, A[35], n, mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_WIRE)
    assert p.stream_kernel == 1
    rc, p = qa(n, A[35], n, mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_WIRE, config={"stream_kernel": 2})
    assert p.stream_kernel == 2
    rc, p = qa(n, A[35], n, mode=ar.AR_MODE_RS_BCAST)
    assert rc == ar.AR_OK and p.stream_kernel == 2
    # narrow destination: the residual has the destination type
    rc, p = qa(n, A[35], n, wire=ar.AR_F16, dst_type=ar.AR_F16)
    assert rc == ar.AR_OK and p.algo_bytes == 2 * n * 2 + n * 2 + n * 2
    # n = 0 is a no-op
    assert qa(0, A[35], 0)[0] == ar.AR_OK
    # a NULL context is rejected by ar_reduce_add before anything else
    lib = ar.load_library()
    srcs = (ctypes.c_void_p * 2)(*A[1:3])
    dsts = (ctypes.c_void_p * 1)(A[30])
    assert lib.ar_reduce_add(None, dsts, srcs, 2, 64, ar.AR_F32, ar.AR_BF16, 0, A[35], 64, None) == \
        ar.AR_ERR_INVALID


def qr(rows, cols, ss, ds, R=2, mode=ar.AR_MODE_CHUNKED, wire=ar.AR_BF16, dst_type=ar.AR_F32, res=None, rs=0,
       dsts=None, srcs=None, host=False, config=None):
    srcs = A[1:1 + R] if srcs is None else srcs
    dsts = [A[20 + d] for d in range(R)] if dsts is None else dsts
    return ar.ar_plan_query_rows(dsts, srcs, rows, cols, ss, ds, dst_type, wire, mode, res, rs, host, config,
                                 R=len(srcs))


def test_row_strided_rules():
    assert ctypes.sizeof(ar.ArRows) == 5 * 8
    # a 2048 x 4096 block inside rows of 4608: the algorithmic bytes count the block only
    rc, p = qr(2048, 4096, 4608, 4608)
    assert rc == ar.AR_OK and p.chunk_elems == 4096 and p.n_chunks == 2048
    assert p.algo_bytes == 2 * 2048 * 4096 * 4 + 2048 * 4096 * 4
    # strides shorter than a row, or row starts off 16 bytes
    assert qr(4, 64, 60, 64)[0] == ar.AR_ERR_INVALID
    assert qr(4, 64, 64, 60)[0] == ar.AR_ERR_INVALID
    assert qr(4, 64, 66, 64)[0] == ar.AR_ERR_INVALID            # 66 * 4 B is not a multiple of 16
    assert qr(4, 64, 68, 64)[0] == ar.AR_OK
    assert qr(4, 64, 68, 68, mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_WIRE)[0] == ar.AR_ERR_INVALID  # 68 * 2 B
    assert qr(4, 64, 72, 68, mode=ar.AR_MODE_CHUNKED | ar.AR_SRC_WIRE)[0] == ar.AR_OK
    # residual: element-wise stride or one broadcast row
    rc, p = qr(16, 4096, 4096, 4096, res=A[35], rs=4096)
    assert rc == ar.AR_OK and p.residual_kind == 1 and p.stream_kernel == 3     # two-rank rows kernel
    rc, p = qr(16, 4000, 4096, 4096, res=A[35], rs=4096)
    assert rc == ar.AR_OK and p.residual_kind == 1 and p.stream_kernel == 1     # rows not whole tiles
    rc, p = qr(16, 4096, 4096, 4096, res=A[35], rs=0)
    assert rc == ar.AR_OK and p.residual_kind == 2
    assert p.algo_bytes == 2 * 16 * 4096 * 4 + 16 * 4096 * 4 + 4096 * 4
    assert qr(16, 4096, 4096, 4096, res=A[35], rs=100)[0] == ar.AR_ERR_INVALID
    # overlaps judged on spans: interleaved rows of a source and the destination
    n_span = 3 * 128 + 64
    assert qr(4, 64, 128, 128, dsts=[A[1] + 64 * 4])[0] == ar.AR_ERR_INVALID
    assert qr(4, 64, 128, 128, dsts=[A[1] + n_span * 4])[0] == ar.AR_OK
    # exactly in place needs equal strides
    assert qr(4, 64, 128, 128, dsts=[A[1]])[0] == ar.AR_OK
    assert qr(4, 64, 128, 64, dsts=[A[1]])[0] == ar.AR_ERR_INVALID
    # broadcast schedule: every row to all R destinations, no per-rank slices
    rc, p = qr(8, 4096, 4096, 4096, R=4, mode=ar.AR_MODE_RS_BCAST, wire=ar.AR_F16)
    assert rc == ar.AR_OK and p.n_dst == 4 and all(p.slice_len[r] == 0 for r in range(4))
    # host-staged: chunks of whole rows
    rc, p = qr(8192, 8192, 8192, 8192, R=8, mode=ar.AR_MODE_HOST_STAGED | ar.AR_SRC_WIRE)
    assert rc == ar.AR_OK and p.chunk_elems % 8192 == 0 and p.chunk_elems // 8192 == (64 * MiB) // (8192 * 2)
    # a row longer than one launch covers
    assert qr(1, (1 << 30) + 8, (1 << 30) + 8, (1 << 30) + 8)[0] == ar.AR_ERR_UNSUPPORTED
    # empty shapes are no-ops
    assert qr(0, 64, 64, 64)[0] == ar.AR_OK
    assert qr(5, 0, 0, 0)[0] == ar.AR_OK
    # a NULL shape
    lib = ar.load_library()
    srcs = (ctypes.c_void_p * 2)(*A[1:3])
    dsts = (ctypes.c_void_p * 1)(A[30])
    assert lib.ar_plan_query_rows(None, dsts, srcs, 2, None, 0, 2, 2, None, 0, None) == ar.AR_ERR_INVALID
    assert lib.ar_reduce_rows(None, dsts, srcs, 2, None, 0, 2, 2, None, None) == ar.AR_ERR_INVALID


def test_bound_calls_reach_the_library():
    """ar.bind_reduce converts the arguments once; each invocation is a plain call of
    ar_reduce / ar_reduce_add, whose validation still runs (a NULL context is refused
    before any runtime call, so this runs without a GPU)."""
    fake = [1 << 33, (1 << 33) + (1 << 20)]
    f = ar.bind_reduce(None, [1 << 34], fake, 4096, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_SINGLE_SHOT)
    assert f() == ar.AR_ERR_INVALID and f() == ar.AR_ERR_INVALID
    g = ar.bind_reduce(None, [1 << 34], fake, 4096, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                       residual=1 << 35, residual_len=512)
    assert g() == ar.AR_ERR_INVALID
    h = ar.bind_reduce_rows(None, [1 << 34], fake, 4, 512, 640, 576, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED,
                            residual=1 << 35)
    assert h() == ar.AR_ERR_INVALID and h() == ar.AR_ERR_INVALID


def test_binding_checks_tensor_sizes_before_the_call():
    """The library sees pointers only; the binding checks each tensor argument's byte
    span (and contiguity for the 1-D calls) before calling it.  Host tensors stand in
    for device ones: the check runs before the call, and with a NULL context the call
    itself is refused without touching the GPU."""
    import torch
    n = 1000
    f32 = [torch.empty(n) for _ in range(3)]
    F, B, C = ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED
    assert ar.ar_reduce(None, f32[:1], f32[1:], n, F, B, C, check=False) == ar.AR_ERR_INVALID
    with pytest.raises(ValueError, match="srcs"):
        ar.ar_reduce(None, f32[:1], [f32[1], torch.empty(n - 1)], n, F, B, C)
    with pytest.raises(ValueError, match="dsts"):
        ar.ar_reduce(None, [torch.empty(n // 2)], f32[1:], n, F, B, C)
    with pytest.raises(ValueError, match="not contiguous"):
        ar.ar_reduce(None, f32[:1], [torch.empty(2 * n)[::2], f32[2]], n, F, B, C)
    # sources in the wire type are read at 2 bytes per element
    half = [torch.empty(n, dtype=torch.int16) for _ in range(2)]
    assert ar.ar_reduce(None, f32[:1], half, n, F, B, C | ar.AR_SRC_WIRE, check=False) == ar.AR_ERR_INVALID
    with pytest.raises(ValueError, match="srcs"):
        ar.ar_reduce(None, f32[:1], half, n, F, B, C, check=False)
    # addresses and inactive (None) ranks are not checked; validate=False skips the check
    assert ar.ar_reduce(None, f32[:1], [1 << 33, None], n, F, B, C | ar.AR_SRC_INACTIVE_NULL,
                        check=False) == ar.AR_ERR_INVALID
    assert ar.ar_reduce(None, [torch.empty(1)], f32[1:], n, F, B, C, check=False,
                        validate=False) == ar.AR_ERR_INVALID
    # residuals: element-wise and one row
    with pytest.raises(ValueError, match="residual"):
        ar.ar_reduce_add(None, f32[:1], f32[1:], n, F, B, C, torch.empty(100), n)
    assert ar.ar_reduce_add(None, f32[:1], f32[1:], n, F, B, C, torch.empty(100), check=False) == ar.AR_ERR_INVALID
    with pytest.raises(TypeError, match="residual_len"):
        ar.ar_reduce_add(None, f32[:1], f32[1:], n, F, B, C, 1 << 35)
    with pytest.raises(ValueError, match="residual"):
        ar.bind_reduce(None, f32[:1], f32[1:], n, F, B, C, residual=torch.empty(10), residual_len=100)
    with pytest.raises(ValueError, match="srcs"):
        ar.bind_reduce(None, f32[:1], [f32[1], torch.empty(10)], n, F, B, C)
    # row-strided: a view of rows inside a wider buffer is fine; its span decides
    rows, cols, ss, ds = 4, 16, 24, 20
    srcs = [torch.empty(rows, ss)[:, :cols] for _ in range(2)]
    dst = torch.empty((rows - 1) * ds + cols)
    assert ar.ar_reduce_rows(None, [dst], srcs, rows, cols, ss, ds, F, B, C, check=False) == ar.AR_ERR_INVALID
    with pytest.raises(ValueError, match="dsts"):
        ar.ar_reduce_rows(None, [dst[1:]], srcs, rows, cols, ss, ds, F, B, C)
    with pytest.raises(ValueError, match="srcs"):
        ar.ar_reduce_rows(None, [dst], [srcs[0], torch.empty(rows, ss)[1:, :cols]], rows, cols, ss, ds, F, B, C)
    with pytest.raises(ValueError, match="residual"):
        ar.ar_reduce_rows(None, [dst], srcs, rows, cols, ss, ds, F, B, C, residual=torch.empty(cols - 1))
    assert ar.ar_reduce_rows(None, [dst], srcs, rows, cols, ss, ds, F, B, C, residual=torch.empty(cols),
                             check=False) == ar.AR_ERR_INVALID
    with pytest.raises(ValueError, match="srcs"):
        ar.bind_reduce_rows(None, [dst], [srcs[0], torch.empty(rows, ss)[1:, :cols]], rows, cols, ss, ds, F, B, C)


def test_bound_calls_use_the_compiled_call_type():
    """With the fast-call module built (build() builds it), bound calls are instances of
    its C type, which takes no arguments; without it the binding falls back to ctypes."""
    fast = ar._fast_module()
    if fast is None:
        pytest.skip("fast-call module not built")
    f = ar.bind_reduce(None, [1 << 34], [1 << 33, (1 << 33) + (1 << 20)], 4096)
    assert isinstance(f, fast.BoundCall)
    assert f() == ar.AR_ERR_INVALID
    with pytest.raises(TypeError):
        f(1)


def test_header_is_c_and_matches_the_binding(tmp_path):
    """tests/c_abi/ar_layout.c, built as C99 with gcc against include/ar.h and
    linked with libmpp_ar.so, prints the layouts the C compiler chose; every field
    offset and size must equal the binding's ctypes structures, and a plan computed
    from C must equal the one the binding returns."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "mixed_precision_partial_amd")
    exe = str(tmp_path / "ar_layout")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(root, "include"),
           os.path.join(root, "tests", "c_abi", "ar_layout.c"), "-o", exe, "-L", pkg, "-lmpp_ar",
           f"-Wl,-rpath,{pkg}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.splitlines()
    structs = {"ar_config": ar.ArConfig, "ar_plan": ar.ArPlan, "ar_rows": ar.ArRows}
    seen = set()
    for line in out:
        parts = line.split()
        if parts[0] == "sizeof":
            assert ctypes.sizeof(structs[parts[1]]) == int(parts[2]), line
        elif "." in parts[0] and parts[0].split(".")[0] in structs:
            sname, field = parts[0].split(".")
            desc = getattr(structs[sname], field)
            assert (desc.offset, desc.size) == (int(parts[1]), int(parts[2])), line
            seen.add((sname, field))
    for sname, cls in structs.items():
        assert {f for f, _ in cls._fields_} == {f for s, f in seen if s == sname}, sname
    status = {int(l.split()[1]): l.split()[2] for l in out if l.startswith("status ")}
    assert all(status[s] == ar.ar_status_str(s) for s in status)
    kv = dict(l.split(" ", 1) for l in out if l.startswith(("free_null", "init_null")))
    assert int(kv["free_null"]) == ar.AR_OK and int(kv["init_null"]) == ar.AR_ERR_INVALID
    plan_line = next(l for l in out if l.startswith("plan "))
    vals = plan_line.split()
    got = {vals[i]: int(vals[i + 1]) for i in range(1, len(vals) - 3, 2)}
    got["slice1"] = (int(vals[-2]), int(vals[-1]))
    srcs = [(r + 1) << 36 for r in range(4)]
    dsts = [(r + 9) << 36 for r in range(4)]
    rc, p = ar.ar_plan_query(dsts, srcs, 2048 * 8192, ar.AR_F32, ar.AR_F16, ar.AR_MODE_RS_BCAST)
    assert got["rc"] == rc == ar.AR_OK
    for k in ("mode", "n_dst", "src_bytes", "wire_bytes", "chunk_elems", "n_chunks", "algo_bytes", "store_nt",
              "stream_kernel", "active_mask"):
        assert got[k] == getattr(p, k), k
    assert got["slice1"] == (p.slice_start[1], p.slice_len[1])


def test_xcd_placement_map_is_a_permutation(tmp_path):
    """tests/c_abi/xcd_map_check.cpp, built with hipcc as host code against the
    library's internal header: the workgroup renumbering of the streaming kernels
    is a permutation of the grid for every size and exponent tried, the identity
    at exponent 0, walks runs of consecutive tiles per XCD, and the exponent the
    launcher picks never exceeds the requested run or one round per range."""
    import subprocess

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "xcd_map_check")
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, "-O1", "-std=c++17", "-I", os.path.join(root, "include"),
           "-I", os.path.join(root, "mixed_precision_partial_amd", "csrc"),
           os.path.join(root, "tests", "c_abi", "xcd_map_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.startswith("OK"), out.stdout + out.stderr


def test_occupancy_hold_in_plans(monkeypatch):
    """The plan reports the occupancy hold its launches take: by default the binary32
    two-rank kernels (18 waves, 14 with a residual) and the kernels for a few active
    partials (18, 14 or 10 for two, three or four) only; an explicit ar_config.occupancy_hold
    (or AR_OCCUPANCY_HOLD) holds every streaming launch but never a single-shot one; -1
    holds none; values outside -1..32 are refused."""
    monkeypatch.delenv("AR_OCCUPANCY_HOLD", raising=False)
    n = 2048 * 4096
    two = dict(dsts=[A[20]], srcs=A[1:3], mode=ar.AR_MODE_CHUNKED)
    assert q(n, **two)[1].hold_waves == 18
    rc, p = ar.ar_plan_query_add([A[20]], A[1:3], n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, A[30], n)
    assert rc == ar.AR_OK and p.stream_kernel == 3 and p.hold_waves == 14
    rc, p = ar.ar_plan_query_add([A[20]], A[1:3], n, ar.AR_F32, ar.AR_BF16, ar.AR_MODE_CHUNKED, A[30], 4096)
    assert rc == ar.AR_OK and p.hold_waves == 14
    rc, p = ar.ar_plan_query_rows([A[20]], A[1:3], 2048, 4096, 4608, 4352, ar.AR_F32, ar.AR_BF16,
                                  ar.AR_MODE_CHUNKED)
    assert rc == ar.AR_OK and p.stream_kernel == 3 and p.hold_waves == 18
    three = dict(dsts=[A[20]], srcs=A[1:4], mode=ar.AR_MODE_CHUNKED)
    assert q(n, **three)[1].stream_kernel == 4 and q(n, **three)[1].hold_waves == 14
    five = dict(dsts=[A[20]], srcs=A[1:6], mode=ar.AR_MODE_CHUNKED)
    assert q(n, **five)[1].stream_kernel in (1, 2) and q(n, **five)[1].hold_waves == 0
    assert q(n, **five, config={"occupancy_hold": 12})[1].hold_waves == 12
    assert q(n, **two, config={"occupancy_hold": -1})[1].hold_waves == 0
    assert q(n, **two, config={"occupancy_hold": 12})[1].hold_waves == 12
    assert q(n, **three, config={"occupancy_hold": 12})[1].hold_waves == 12
    ss = dict(dsts=[A[20]], srcs=A[1:6], mode=ar.AR_MODE_SINGLE_SHOT)
    assert q(4096, **ss, config={"occupancy_hold": 12})[1].stream_kernel == 0
    assert q(4096, **ss, config={"occupancy_hold": 12})[1].hold_waves == 0
    for bad in (-2, 33):
        assert q(n, **two, config={"occupancy_hold": bad})[0] == ar.AR_ERR_INVALID
    monkeypatch.setenv("AR_OCCUPANCY_HOLD", "-1")
    assert q(n, **two)[1].hold_waves == 0
    monkeypatch.setenv("AR_OCCUPANCY_HOLD", "20")
    assert q(n, **three)[1].hold_waves == 20
    assert q(n, **two, config={"occupancy_hold": 16})[1].hold_waves == 16   # the field wins
    monkeypatch.setenv("AR_OCCUPANCY_HOLD", "40")
    assert q(n, **two)[0] == ar.AR_ERR_INVALID


def test_occupancy_hold_bytes(tmp_path):
    """tests/c_abi/hold_check.cpp, built with hipcc as host code against the
    library's internal header: the dynamic LDS that holds a CU to N one-wave
    workgroups is the smallest multiple of 512 bytes giving exactly N per CU,
    and no hold is asked for when the grid would not fill the CUs to N."""
    import subprocess

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "hold_check")
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, "-O1", "-std=c++17", "-I", os.path.join(root, "include"),
           "-I", os.path.join(root, "mixed_precision_partial_amd", "csrc"),
           os.path.join(root, "tests", "c_abi", "hold_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.startswith("OK"), out.stdout + out.stderr


def test_few_partial_gaps():
    """tests/c_abi/few_check.cpp, built with hipcc as host code against the library's
    internal header: for every placement of 2 to 4 active ranks among 2 to 16, the
    compacted fold with +0.0 at the gaps that hold inactive ranks gives the bits of the
    fold over every rank with +0.0 for the inactive ones, signed zeros included."""
    import subprocess

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(__import__("tempfile").mkdtemp()) + "/few_check"
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, "-O1", "-std=c++17", "-ffp-contract=off", "-I", os.path.join(root, "include"),
           "-I", os.path.join(root, "mixed_precision_partial_amd", "csrc"),
           os.path.join(root, "tests", "c_abi", "few_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.startswith("OK"), out.stdout + out.stderr


def test_binding_refuses_short_pointer_lists():
    """The library reads R destination pointers in the broadcast schedule (and R
    source pointers always): the binding refuses shorter lists before the call,
    instead of letting the library read past the end of the array it built."""
    srcs = [0x10000, 0x20000, 0x30000, 0x40000]
    dsts = [0x50000, 0x60000]
    bcast = ar.AR_MODE_RS_BCAST
    with pytest.raises(ValueError, match="destinations"):
        ar.ar_plan_query(dsts, srcs, 4096, ar.AR_F32, ar.AR_F16, bcast)
    with pytest.raises(ValueError, match="destinations"):
        ar.ar_plan_query_add(dsts, srcs, 4096, ar.AR_F32, ar.AR_F16, bcast, 0x70000, 4096)
    with pytest.raises(ValueError, match="destinations"):
        ar.ar_plan_query_rows(dsts, srcs, 4, 1024, 1024, 1024, ar.AR_F32, ar.AR_F16, bcast)
    with pytest.raises(ValueError, match="destinations"):
        ar.ar_reduce(None, dsts, srcs, 4096, ar.AR_F32, ar.AR_F16, bcast, validate=False)
    with pytest.raises(ValueError, match="destinations"):
        ar.ar_reduce_rows(None, dsts, srcs, 4, 1024, 1024, 1024, ar.AR_F32, ar.AR_F16, bcast, validate=False)
    with pytest.raises(ValueError, match="srcs has"):
        ar.ar_plan_query([0x50000], srcs[:2], 4096, ar.AR_F32, ar.AR_F16, ar.AR_MODE_CHUNKED, R=4)
    # enough destinations: the library plans the call (made-up addresses, never dereferenced)
    rc, plan = ar.ar_plan_query(dsts + [0x80000, 0x90000], srcs, 4096, ar.AR_F32, ar.AR_F16, bcast)
    assert rc == ar.AR_OK and plan.n_dst == 4
    # one destination is enough outside the broadcast schedule
    rc, _ = ar.ar_plan_query([0x50000], srcs, 4096, ar.AR_F32, ar.AR_F16, ar.AR_MODE_CHUNKED)
    assert rc == ar.AR_OK
    # ctypes arrays pass through as given, as in C; out-of-range R is the library's to reject
    rc, _ = ar.ar_plan_query([0x50000], srcs * 5, 4096, ar.AR_F32, ar.AR_F16, bcast)
    assert rc == ar.AR_ERR_INVALID
