"""bench.py's counter records (no GPU): the matrix-core record computed from a rocprofv3-style
counter CSV, and a record taken on other kernel sources being ignored."""
import argparse
import csv

import pytest

import bench

HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
NS = "(anonymous namespace)::"


def write_csvs(tmp_path):
    # one dense call: main kernel 190 ms, split kernel 5 ms, merge 0.02 ms; counters split over
    # 8 rows per dispatch (as per-XCD rows would be); one unrelated kernel that must be ignored
    calls = [(1, NS + "attn_fwd_dense_kernel(" + NS + "DenseArgs)", 0, 190_000_000, 8.0e9),
             (2, NS + "attn_fwd_dense_split_kernel(" + NS + "DenseArgs, " + NS + "SplitArgs)",
              190_000_000, 195_000_000, 0.2e9),
             (3, NS + "merge_kernel(" + NS + "DenseArgs, " + NS + "SplitArgs)", 195_000_000, 195_020_000, 0.0),
             (4, "void " + NS + "qk_prologue_kernel<4>(" + NS + "PrologueArgs)", 196_000_000, 197_000_000, 5.0e9)]
    clock_ghz, busy = 1.6, 0.8
    rows = []
    for d, name, s, e, mfma in calls:
        cycles_per_xcd = (e - s) * clock_ghz
        for _ in range(8):
            rows.append([d, d, "Agent 1", 1, 1, 1, 1, 1, name, 256, 0, 0, 0, 0, 0, "SQ_INSTS_MFMA", mfma / 8, s, e])
            rows.append([d, d, "Agent 1", 1, 1, 1, 1, 1, name, 256, 0, 0, 0, 0, 0, "SQ_VALU_MFMA_BUSY_CYCLES",
                         busy * cycles_per_xcd * 1024 / 8, s, e])
            rows.append([d, d, "Agent 1", 1, 1, 1, 1, 1, name, 256, 0, 0, 0, 0, 0, "GRBM_GUI_ACTIVE",
                         cycles_per_xcd, s, e])
    c = tmp_path / "counters.csv"
    with open(c, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEADER)
        w.writerows(rows)
    a = tmp_path / "agents.csv"
    with open(a, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Simd_Count", "Num_Xcc"])
        w.writerow(["gfx950", "1024", "8"])
    return str(c), str(a)


def test_mfma_record_from_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    c, a = write_csvs(tmp_path)
    args = argparse.Namespace(write_mfma_profile=(c, a), traffic_kind="dense", workload="video_720p",
                              profile_command="")
    assert bench.write_mfma_profile(args) == 0
    got = bench.measured_mfma("video_720p", "attn_fwd_dense_kernel", True, "dense")
    flops = 8.2e9 * 32768
    ms = 195.02
    assert got["kernel_ms"] == pytest.approx(ms, rel=1e-6)
    assert got["counter_tflops"] == pytest.approx(flops / (ms * 1e-3) / 1e12, abs=0.06)
    assert got["util_of_peak"] == pytest.approx(flops / (ms * 1e-3) / 1e12 / 2500.0, abs=1e-4)
    assert got["counter_over_algorithmic_flops"] == pytest.approx(flops / (4.0 * 16 * 180320 ** 2 * 128), abs=1e-4)
    assert got["busy_of_clocked_cycles"] == pytest.approx(0.8, abs=1e-4)
    assert got["avg_shader_clock_ghz"] == pytest.approx(1.6, abs=1e-3)
    # a record without split pieces does not describe a split call, and vice versa
    assert bench.measured_mfma("video_720p", "attn_fwd_dense_kernel", False, "dense") is None


def test_record_of_other_sources_is_ignored(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    c, a = write_csvs(tmp_path)
    args = argparse.Namespace(write_mfma_profile=(c, a), traffic_kind="dense", workload="video_720p",
                              profile_command="")
    bench.write_mfma_profile(args)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kind="dense": "0" * 64)
    assert bench.measured_mfma("video_720p", "attn_fwd_dense_kernel", True, "dense") is None


PACKED_RUN = ["build_varlen_schedule", "varlen_split_plan", "attn_fwd_varlen_kernel", "attn_fwd_varlen_split_kernel",
              "varlen_merge_kernel",                                   # one packed attention call
              "tile_offsets_kernel", "pool_varlen_kernel", "route_varlen_kernel", "lpt_order_kernel",
              "build_varlen_schedule", "attn_fwd_block_sparse_varlen_kernel",   # routing, then the sparse pass
              "qk_norm_packed_kernel", "__amd_rocclr_copyBuffer"]


def test_shared_kernels_go_to_the_call_they_precede():
    order = list(enumerate(PACKED_RUN, start=1))
    assert bench._of_call(order, bench.CALL_KERNELS["varlen"]) == {1, 2, 3, 4, 5}
    assert bench._of_call(order, bench.CALL_KERNELS["block_sparse_varlen"]) == {6, 7, 8, 9, 10, 11}
    assert bench._of_call(order, bench.CALL_KERNELS["packed_prologue"]) == {12}


def test_traffic_record_of_a_packed_run(tmp_path, monkeypatch):
    """FETCH/WRITE of the packed call's five kernels only, scaled by the calibration copy."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    last = len(PACKED_RUN)                              # the calibration copy's dispatch
    fetch = {d: 100.0 * d for d in range(1, last)}
    fetch[last] = 512.0                                 # a 1 MiB copy reads as 512 KiB: scale x2
    write = {d: 10.0 * d for d in range(1, last)}
    write[last] = 1024.0
    paths = []
    for counter, vals in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        p = tmp_path / f"{counter}.csv"
        with open(p, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(HEADER)
            for d, n in enumerate(PACKED_RUN, start=1):
                name = n if n.startswith("__") else NS + n + "(" + NS + "Args)"
                w.writerow([d, d, "Agent 1", 1, 1, 1, 1, 1, name, 256, 0, 0, 0, 0, 0, counter, vals[d], 0, 1])
        paths.append(str(p))
    args = argparse.Namespace(write_traffic_profile=tuple(paths), traffic_kind="varlen", workload="packed_varlen",
                              calibrate_copy_mib=1, profile_command="")
    assert bench.write_traffic_profile(args) == 0
    copy_mib = 1 << 20
    f_scale = copy_mib / (512.0 * 1024)
    w_scale = copy_mib / (1024.0 * 1024)
    want = (100 + 200 + 300 + 400 + 500) * 1024 * f_scale + (10 + 20 + 30 + 40 + 50) * 1024 * w_scale
    assert bench.measured_traffic("packed_varlen", "attn_fwd_varlen_kernel", True, "varlen") == pytest.approx(want)


def test_kernel_names_as_the_profiler_writes_them():
    assert bench._base_name("void (anonymous namespace)::pool_kernel<64>(bool _Accum const*, float, int, int)") == \
        "pool_kernel"
    assert bench._base_name("(anonymous namespace)::merge_kernel((anonymous namespace)::DenseArgs)") == "merge_kernel"
    assert bench._base_name("_ZN12_GLOBAL__N_118pool_varlen_kernelILi256EEEvPKDF16bPfPKiS5_iii") == "pool_varlen_kernel"
    assert bench._base_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_default_warmup_lasts_about_half_a_second():
    assert bench.default_warmup(0.19) == 3          # the 720p call: three calls, ~0.6 s
    assert bench.default_warmup(0.00085) == 589     # the stress call: ~0.5 s of calls
    assert bench.default_warmup(0.0) == 500000      # no measurable duration: bounded
    n = bench.default_warmup(0.0064)
    assert 0.5 <= n * 0.0064 < 0.5 + 0.0064
