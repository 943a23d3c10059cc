"""Host logic of bench.py (no GPU): the one-GPU guard, the byte counts its
roofline and profile summaries use, and the counter scaling.

The byte formula of every profile configuration is checked against the
library's own plan of the same call (``ar_plan_query*``), so the bench and
the library cannot disagree on what a call must move.
"""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import mixed_precision_partial_amd as ar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASE = [0x20_0000_0000 + i * 0x4_0000_0000 for i in range(40)]   # aligned, 16 GiB apart


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def plan_of(case: dict):
    """The library's plan for the call a profile configuration makes."""
    wire = {"bf16": ar.AR_BF16, "f16": ar.AR_F16}[case["wire"]]
    mode = {"chunked": ar.AR_MODE_CHUNKED, "rs_bcast": ar.AR_MODE_RS_BCAST,
            "host_staged": ar.AR_MODE_HOST_STAGED}[case["mode"]]
    narrow = case.get("dst_bytes", 4) == 2
    dst_type = wire if narrow else ar.AR_F32
    if case["src_bytes"] == 2 and not narrow:
        mode |= ar.AR_SRC_WIRE
    inactive = set(case.get("inactive", ()))
    if inactive:
        mode |= ar.AR_SRC_INACTIVE_NULL
    R = case["R"]
    srcs = [0 if r in inactive else BASE[1 + r] for r in range(R)]
    dsts = [BASE[20 + d] for d in range(R)]
    res = case.get("res")
    if case.get("rows") is not None:
        rows, cols, ss, ds = case["rows"]
        return ar.ar_plan_query_rows(dsts, srcs, rows, cols, ss, ds, dst_type, wire, mode,
                                     residual=None if res is None else BASE[39], res_stride=0,
                                     srcs_on_host=case["host"])
    if res is None:
        return ar.ar_plan_query(dsts, srcs, case["n"], dst_type, wire, mode, case["host"])
    res_len = case["n"] if res == "elementwise" else res
    return ar.ar_plan_query_add(dsts, srcs, case["n"], dst_type, wire, mode, BASE[39], res_len, case["host"])


@pytest.mark.parametrize("name", sorted(bench.PROFILE_CASES))
def test_profile_case_bytes_match_the_plan(name):
    case = bench.PROFILE_CASES[name]
    rc, plan = plan_of(case)
    assert rc == ar.AR_OK, ar.ar_status_str(rc)
    assert plan.n_dst == case["n_dst"]
    assert plan.algo_bytes == bench.case_algo_bytes(case)


def test_headline_bytes():
    # 2 fp32 partials of 2048 x 4096 read, one fp32 destination written
    assert bench.case_algo_bytes(bench.PROFILE_CASES["prefill_bf16"]) == 100_663_296
    assert bench.case_algo_bytes(bench.PROFILE_CASES["slice_bcast_f16"]) == 536_870_912


def write_counters(directory, counter, rows):
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, f"x_{counter}_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    wl = "prefill_bf16_dst"     # bf16 partials into a bf16 destination: 32 MiB read, 16 MiB written
    kernel = "void mpp::(anonymous namespace)::k_stream_lds<Cfg<2, true, true, 2, false, false> >(...)"
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"
    # the calibration copy reads 64 MiB that FETCH_SIZE reports as half (scale 2) and
    # writes 64 MiB that WRITE_SIZE reports whole (scale 1)
    write_counters(tmp_path / "f", "FETCH_SIZE", [(kernel, 16384.0), (kernel, 16384.0), (neg, 32768.0)])
    write_counters(tmp_path / "w", "WRITE_SIZE", [(kernel, 16384.0), (kernel, 16384.0), (neg, 65536.0)])
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), wl)
    with open(tmp_path / "profiles" / f"traffic_{wl}.json") as fh:
        t = json.load(fh)
    assert t["calibration"]["fetch_scale"] == 2.0 and t["calibration"]["write_scale"] == 1.0
    assert t["hbm_bytes_per_launch"] == 32 * 2**20 + 16 * 2**20
    assert t["algo_bytes_per_launch"] == bench.case_algo_bytes(bench.PROFILE_CASES[wl]) == 48 * 2**20
    assert t["traffic_over_algo"] == 1.0 and t["fetch_dispatches"] == 2
    assert t["kernel_source_sha256_16"] == bench.kernel_source_hash()
    assert (tmp_path / "profiles" / f"traffic_{wl}.md").exists()


def test_counters_missing_a_dispatch_are_refused(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    kernel = "void mpp::(anonymous namespace)::k_pair<2>(unsigned int, unsigned int, float*, float const*, float const*, unsigned int)"
    write_counters(tmp_path / "f", "FETCH_SIZE", [(kernel, 1.0)])     # no calibration launch
    write_counters(tmp_path / "w", "WRITE_SIZE", [(kernel, 1.0)])
    with pytest.raises(RuntimeError, match="missing dispatches"):
        bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "prefill_residual")


def test_traffic_is_reported_only_for_the_kernel_it_was_counted_on(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(path))
    assert bench.measured_traffic(1) is None                     # no counter run
    path.write_text(json.dumps({"kernel_source_sha256_16": bench.kernel_source_hash(),
                                "hbm_bytes_per_launch": 100_698_770}))
    assert bench.measured_traffic(1) == 100_698_770
    path.write_text(json.dumps({"kernel_source_sha256_16": "0" * 16, "hbm_bytes_per_launch": 5}))
    assert bench.measured_traffic(1) is None                     # kernels changed since


def test_committed_headline_traffic_summary_is_consistent():
    # (whether it was counted on the current kernels is decided at run time:
    # the bench reports traffic null otherwise)
    with open(os.path.join(ROOT, "profiles", "traffic_prefill_bf16.json")) as fh:
        t = json.load(fh)
    assert len(t["kernel_source_sha256_16"]) == 16
    assert t["algo_bytes_per_launch"] == 100_663_296
    assert 0.99 < t["traffic_over_algo"] < 1.01


def test_kernel_name_matchers():
    assert bench.is_reduce_kernel("void mpp::(anonymous namespace)::k_pair<2>(unsigned int, unsigned int, float*, "
                                  "float const*, float const*, unsigned int)")
    assert not bench.is_reduce_kernel("void mpp::(anonymous namespace)::k_pair<0>(unsigned int, unsigned int, ...)")
    assert not bench.is_reduce_kernel("void k_stream_reg<Cfg<2, false, false, 2, false, false> >(...)")
    assert bench.is_library_kernel("void mpp::(anonymous namespace)::k_pair<1>(unsigned int, ...)")
    assert bench.is_library_kernel("void mpp::(anonymous namespace)::k_pair_res<2, 2>(unsigned int, ...)")
    assert not bench.is_reduce_kernel("void mpp::(anonymous namespace)::k_pair_res<2, 2>(unsigned int, ...)")
    assert bench.is_library_kernel("void k_single_shot<Cfg<0, false, false, 2, false, false> >(...)")
    assert bench.is_library_kernel("void mpp::(anonymous namespace)::k_few<2, 3>(unsigned int, ...)")
    assert not bench.is_reduce_kernel("void mpp::(anonymous namespace)::k_few<2, 3>(unsigned int, ...)")
    assert not bench.is_library_kernel("void at::native::vectorized_elementwise_kernel<4, neg_kernel_cuda>")


def test_kernel_hash_ignores_comments_not_code():
    src = 'int f(int a) { // add one\n  return a + 1; /* done */ }\nconst char *s = "a // b /* c */";\n'
    same = 'int f(int a) {\n\n  return a + 1;  }   // other words\nconst char *s = "a // b /* c */";'
    other = 'int f(int a) { return a + 2; }\nconst char *s = "a // b /* c */";'
    assert bench.code_tokens(src) == bench.code_tokens(same)
    assert bench.code_tokens(src) != bench.code_tokens(other)
    assert '"a // b /* c */"' in bench.code_tokens(src)
    assert bench.code_tokens("char c = '/'; // x") == "char c = '/';"


def test_headline_trace_takes_the_prefill_grid_only(tmp_path, monkeypatch):
    """The default run launches the prefill's kernel for decode-sized and 768 MiB calls too:
    the headline average comes from the dispatches at the prefill call's grid."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    d = tmp_path / "trace"
    os.makedirs(d)
    name = "void mpp::(anonymous namespace)::k_pair<2>(unsigned int, unsigned int, float*, float const*, float const*, unsigned int)"
    with open(d / "trace_kernel_stats.csv", "w") as fh:
        fh.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        fh.write(f'"{name}",5,100000,20000,100.0,2000,60000,1\n')
    grid = bench.prefill_grid_items(2048 * 4096)
    assert grid == 1048576
    rows = [(grid, 15_000), (grid, 16_000), (512, 2_000), (grid * 8, 60_000), (grid, 17_000)]
    with open(d / "trace_kernel_trace.csv", "w") as fh:
        fh.write('"Kernel_Name","Start_Timestamp","End_Timestamp","Workgroup_Size_X","Grid_Size_X"\n')
        t = 1_000_000
        for g, dur in rows:
            fh.write(f'"{name}",{t},{t + dur},64,{g}\n')
            t += 100_000
    bench.summarize_trace(str(d), "prefill_bf16")
    text = (tmp_path / "profiles" / "kernel_trace_prefill_bf16.md").read_text()
    assert "3 dispatches, average 16.000 us" in text
    # a traced profile pass of the same call is summarised under its own name, from the
    # kernel statistics (every dispatch there is the prefill call), without touching the above
    bench.summarize_trace(str(d), "prefill_bf16", bench_run=False)
    pass_text = (tmp_path / "profiles" / "kernel_trace_prefill_bf16_profile_pass.md").read_text()
    assert "profile pass of" in pass_text and "--profile-workload prefill_bf16" in pass_text
    assert "average 20.000 us per launch" in pass_text
    assert (tmp_path / "profiles" / "kernel_trace_prefill_bf16.md").read_text() == text


def test_footprint_summary_compares_the_two_footprints(tmp_path, monkeypatch):
    """The footprint summary averages the prefill kernel's counters per footprint (other
    kernels ignored) and its traced durations, and writes both beside their ratio."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    root = tmp_path / "fp"
    pair = "void mpp::(anonymous namespace)::k_pair<2>(unsigned int, unsigned int, float*, float const*, float const*, unsigned int)"
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"
    for sets, scale in ((8, 1.0), (16, 1.5)):
        for tag in bench.FOOTPRINT_PASSES:
            write_counters(root / f"{tag}{sets}", "TCP_UTCL1_TRANSLATION_MISS_sum" if tag == "utcl" else f"X_{tag}",
                           [(pair, 100.0 * scale), (pair, 300.0 * scale), (neg, 1e6)])
        d = root / f"trace{sets}"
        os.makedirs(d)
        with open(d / "trace_kernel_trace.csv", "w") as fh:
            fh.write('"Kernel_Name","Start_Timestamp","End_Timestamp","Workgroup_Size_X","Grid_Size_X"\n')
            fh.write(f'"{pair}",1000,{1000 + int(15_000 * scale)},64,1048576\n')
            fh.write(f'"{neg}",90000,190000,256,1048576\n')
    text = open(bench.summarize_footprint(str(root))).read()
    assert "| traced duration, us (1 / 1 dispatches) | 15.000 | 22.500 | 1.500 |" in text
    assert "| TCP_UTCL1_TRANSLATION_MISS_sum | 200.0 | 300.0 | 1.500 |" in text
    assert "--profile-workload <workload> --sets {sets}" in text and bench.kernel_source_hash() in text
