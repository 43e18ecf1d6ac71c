"""CPU tests of profile_kernels.py's parsing of rocprofv3 CSV output and bench
lines (no GPU, no profiler): the counter figures bench.py reports as
`roofline.traffic` come through these functions."""
import csv
import json
import os

import pytest

import profile_kernels as P

COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id",
                "Thread_Id", "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size",
                "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count",
                "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "t_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_COLS)
        w.writeheader()
        for disp, name, counter, value in rows:
            r = {c: "0" for c in COUNTER_COLS}
            r.update(Dispatch_Id=str(disp), Kernel_Name=name, Counter_Name=counter,
                     Counter_Value=str(value))
            w.writerow(r)


def test_per_dispatch_sums_instances_and_filters_kernel(tmp_path):
    d = str(tmp_path / "fetch")
    k = "void pkv::decode_partitions_kernel<1, 128, 4, 3, true, 0>(pkv::DecodeArgs)"
    write_counters(d, [(1, k, "FETCH_SIZE", 100.0), (1, k, "FETCH_SIZE", 50.0),   # two instances
                       (2, k, "FETCH_SIZE", 160.0), (3, "copyBuffer", "FETCH_SIZE", 7.0),
                       (2, k, "WRITE_SIZE", 9.0)])
    assert sorted(P.per_dispatch(d, "FETCH_SIZE", "decode_partitions")) == [150.0, 160.0]
    assert P.per_dispatch(d, "FETCH_SIZE", "copyBuffer") == [7.0]
    assert P.metric_means(d, ("FETCH_SIZE",), "decode_partitions") == {"FETCH_SIZE": 155.0}
    with pytest.raises(SystemExit):
        P.per_dispatch(d, "FETCH_SIZE", "prefill_kernel")


def test_unexpected_columns_are_refused(tmp_path):
    d = tmp_path / "bad"
    d.mkdir()
    (d / "t_counter_collection.csv").write_text("Kernel,Value\nx,1\n")
    with pytest.raises(SystemExit):
        P.per_dispatch(str(d), "FETCH_SIZE", "x")


def test_stats_rows_sorted_by_total_time(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "t_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow(["small", 10, 1000, 100, 1.0, 90, 110, 1])
        w.writerow(["big", 2, 9000, 4500, 9.0, 4000, 5000, 1])
    rows = P.stats_rows(str(d))
    assert [r["Name"] for r in rows] == ["big", "small"]


def test_stats_rows_keep_the_library_kernels_past_the_top(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "t_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        for i in range(10):
            w.writerow([f"other{i}", 1, 1000 * (20 - i), 1, 1.0, 1, 1, 0])
        w.writerow(["void pkv::cache_write_kernel<1, 1>(pkv::CacheWriteArgs)", 5, 50, 10, 0.1, 9,
                    11, 0])
        w.writerow(["tiny", 1, 10, 10, 0.0, 10, 10, 0])
    names = [r["Name"] for r in P.stats_rows(str(d), top=3)]
    assert names == ["other0", "other1", "other2",
                     "void pkv::cache_write_kernel<1, 1>(pkv::CacheWriteArgs)"]


def test_bench_line_is_the_last_metric_json_line():
    line = {"metric": "m", "value": 1.0}
    text = "noise\n" + json.dumps({"metric": "old", "value": 0}) + "\n" + json.dumps(line) + "\nbye\n"
    assert P.bench_line(text) == line
    with pytest.raises(SystemExit):
        P.bench_line("no json here\n")


def test_short_names_drop_the_anonymous_namespace():
    n = "void pkv::(anonymous namespace)::decode_merge_rows_kernel<1, 128>(pkv::DecodeArgs)"
    assert P.short(n) == "void pkv::decode_merge_rows_kernel<1, 128>(pkv::DecodeArgs)"
    assert P.short("x" * 200).endswith("...") and len(P.short("x" * 200)) == 91


TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Kernel_Id", "Kernel_Name", "Correlation_Id",
              "Start_Timestamp", "End_Timestamp", "Grid_Size", "Workgroup_Size"]


def test_dispatch_times_separates_launches_after_the_flush(tmp_path):
    """Pass-1 dispatches with the flush's reduction among the four kernels
    before them are the timed (flushed) launches; the trace lists kernels out
    of start order, which the parser sorts."""
    d = tmp_path / "trace"
    d.mkdir()
    p1 = "void pkv::decode_partitions_kernel<2, 128, 4, 3, true, 0>(pkv::DecodeArgs)"
    seq = [("merge", 0, 10), ("cache_write_kernel", 10, 20), (p1, 20, 1020),      # warm
           ("reduce_kernel<512>", 1100, 1300), ("add", 1300, 1301),
           ("cache_write_kernel", 1310, 1320), (p1, 1320, 2420),                  # flushed
           ("merge", 2420, 2430), ("cache_write_kernel", 2440, 2450), (p1, 2450, 3450)]
    with open(d / "t_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_COLS)
        w.writeheader()
        for name, a, b in reversed(seq):
            r = {c: "0" for c in TRACE_COLS}
            r.update(Kernel_Name=name, Start_Timestamp=str(a * 1000), End_Timestamp=str(b * 1000))
            w.writerow(r)
    every, flushed = P.dispatch_times(str(d), "decode_partitions_kernel<2, 128")
    assert every == [1000.0, 1100.0, 1000.0]
    assert flushed == [1100.0]
