"""rocprofv3 evidence for the decode pass-1 kernel and the chunked-prefill kernel.

For each workload this runs `bench.py` under rocprofv3: one kernel trace with
statistics, one FETCH_SIZE pass and one WRITE_SIZE pass (one counter per pass),
then one pass each for the derived metrics LDSBankConflict (percent of GPU time
the LDS stalls on bank conflicts), MeanOccupancyPerCU (resident waves per CU)
and VALUBusy + MfmaUtil (percent of time the vector ALU / the matrix cores are
busy); once, a plain 1 GiB device copy under each byte counter calibrates them.
It writes one summary per workload under profiles/ and, for decode,
pass1_hbm_counters.json, which bench.py reads for `roofline.traffic` while the
decode sources still hash to the value recorded there.

Usage (on a machine with the GPU, from the repository root):
    python profile_kernels.py [--decode 4:0,2:0,3:0,5:512] [--prefill 2:512,4:512]
                              [--out DIR]
and, where only the --out folder comes back from that machine, again with
--from-output (and the same --out) to write the summaries from it.  rocprofv3 is started as a child
process with the Python interpreter right after `--`.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
COUNTERS = os.path.join(PROFILES, "pass1_hbm_counters.json")
KERNEL = "decode_partitions"
PREFILL_KERNEL = "prefill_kernel"
# derived-metric passes (each small enough for one hardware pass)
METRIC_PASSES = (("lds", ("LDSBankConflict",)), ("occ", ("MeanOccupancyPerCU",)),
                 ("busy", ("VALUBusy", "MfmaUtil")))
SLUG = {2: "llama3_8b_bf16", 3: "llama31_70b_shared_prefix_bf16", 4: "llama31_70b_fp8_kv",
        5: "llama31_405b_long_context_bf16"}
COPY_MIB = 1024


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


FROM_OUTPUT = False  # set by --from-output: read the logs of an earlier run


def run(cmd, out_file, limit):
    """Run cmd with a time limit, its output into out_file; return the output."""
    if FROM_OUTPUT:
        with open(out_file) as f:
            return f.read()
    log("run: " + " ".join(cmd))
    with open(out_file, "w") as f:
        p = subprocess.run(["timeout", "-s", "KILL", str(limit)] + cmd, stdout=f,
                           stderr=subprocess.STDOUT, cwd=ROOT)
    with open(out_file) as f:
        text = f.read()
    if p.returncode != 0:
        sys.stdout.write(text[-3000:])
        raise SystemExit(f"command failed with status {p.returncode}: {' '.join(cmd)}")
    return text


def bench_line(text):
    for line in reversed(text.splitlines()):
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    raise SystemExit("no bench line in the output")


def one_csv(d, suffix):
    found = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not found:
        raise SystemExit(f"no *{suffix} under {d}")
    return found[0]


def per_dispatch(d, counter, name_part):
    """Counter value (KiB) per dispatch of the kernels whose name holds name_part."""
    vals = {}
    with open(one_csv(d, "counter_collection.csv")) as f:
        reader = csv.DictReader(f)
        need = {"Counter_Name", "Counter_Value", "Kernel_Name", "Dispatch_Id"}
        if not need <= set(reader.fieldnames or ()):
            raise SystemExit(f"unexpected counter columns: {reader.fieldnames}")
        for row in reader:
            if row["Counter_Name"] != counter or name_part not in row["Kernel_Name"]:
                continue
            k = row["Dispatch_Id"]
            vals[k] = vals.get(k, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for {name_part} under {d}")
    return list(vals.values())


def metric_means(d, names, name_part):
    """Mean over the dispatches of kernel name_part of each derived metric."""
    return {m: sum(v) / len(v) for m in names for v in [per_dispatch(d, m, name_part)]}


def metric_runs(a, tag, base, kernel, py):
    """The derived-metric passes of one workload: (commands, {metric: mean})."""
    cmds, vals = [], {}
    for ptag, names in METRIC_PASSES:
        d = f"{a.out}/{tag}/{ptag}"
        cmd = ["rocprofv3", "--pmc", *names, "--kernel-include-regex", kernel,
               "--output-format", "csv", "-d", d, "-o", "t"] + base
        cmds.append(cmd)
        run(cmd, f"{a.out}/{tag}_{ptag}.log", 120)
        vals.update(metric_means(d, names, kernel))
    return cmds, vals


def metric_lines(vals, waves_cap):
    return [
        "## Occupancy, LDS and ALU counters",
        "",
        f"- LDSBankConflict {vals['LDSBankConflict']:.2f}% of GPU time the LDS is stalled on bank conflicts",
        f"- MeanOccupancyPerCU {vals['MeanOccupancyPerCU']:.2f} resident waves per CU "
        f"(the launch allows {waves_cap})",
        f"- VALUBusy {vals['VALUBusy']:.1f}%, MfmaUtil {vals['MfmaUtil']:.1f}% of GPU time",
        "",
    ]


def short(name, n=88):
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= n else name[:n] + "..."


def stats_rows(d, top=8):
    """The `top` kernels by total time, then every other kernel of this
    library (the step's small kernels: cache write, merge), by total time."""
    with open(one_csv(d, "kernel_stats.csv")) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    return rows[:top] + [r for r in rows[top:] if "pkv::" in r["Name"]]


def dispatch_times(d, name_part, flush_part="reduce_kernel", window=4):
    """Durations (us) of the dispatches of kernels whose name holds name_part,
    from the kernel trace, in dispatch order: (all, after_flush) -- the
    second holds the dispatches with a flush kernel (name holding
    flush_part) among the `window` dispatches before them (the flush's reduction and add, the
    metadata copy, the cache write)."""
    with open(one_csv(d, "kernel_trace.csv")) as f:
        rows = list(csv.DictReader(f))
    need = {"Kernel_Name", "Start_Timestamp", "End_Timestamp"}
    if not rows or not need <= set(rows[0]):
        raise SystemExit(f"unexpected kernel trace columns under {d}")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    every, flushed = [], []
    for i, r in enumerate(rows):
        if name_part not in r["Kernel_Name"]:
            continue
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        every.append(us)
        if any(flush_part in rows[j]["Kernel_Name"] for j in range(max(0, i - window), i)):
            flushed.append(us)
    return every, flushed


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--decode", default="4:0,2:0,3:0,5:512",
                    help="decode workloads, config:partition_tokens (4:0, the default bench "
                         "workload, is traced under the default bench command)")
    ap.add_argument("--prefill", default="2:512,4:512",
                    help="prefill workloads, config:chunk_tokens ('' for none)")
    ap.add_argument("--out", default="prof_out",
                    help="folder for the rocprofv3 output and logs")
    ap.add_argument("--from-output", action="store_true",
                    help="run nothing: write the summaries from the rocprofv3 output and logs "
                         "already under --out (made by an earlier run on the GPU machine)")
    a = ap.parse_args()
    global FROM_OUTPUT
    FROM_OUTPUT = a.from_output
    import bench  # noqa: E402  (hash of the decode sources; imports no GPU code)

    os.makedirs(a.out, exist_ok=True)
    py = sys.executable
    cmds = {}

    # calibration: what each counter reads for a copy of known size
    cal = {}
    for counter, tag in (("FETCH_SIZE", "copy_fetch"), ("WRITE_SIZE", "copy_write")):
        cmd = ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d",
               f"{a.out}/{tag}", "-o", "cp", "--", py, "-u", "bench.py", "--copy-probe-mib",
               str(COPY_MIB)]
        cmds[tag] = cmd
        run(cmd, f"{a.out}/{tag}.log", 120)
        v = per_dispatch(f"{a.out}/{tag}", counter, "copyBuffer")
        big = [x for x in v if x > 0.5 * max(v)]
        cal[counter] = sum(big) / len(big)
        log(f"calibration {counter}: {cal[counter]:.0f} KiB per 1 GiB copy")
    copy_bytes = COPY_MIB << 20
    scale = {c: copy_bytes / (cal[c] * 1024.0) for c in cal}

    try:
        with open(COUNTERS) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        doc = {}
    sha = bench.decode_sources_sha256()
    if doc.get("decode_sources_sha256") != sha:
        doc["workloads"] = {}
    doc.update({
        "kernel": "decode_partitions_kernel",
        "decode_sources_sha256": sha,
        "decode_sources": [os.path.relpath(p, ROOT) for p in bench.DECODE_SRCS],
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib": cal["FETCH_SIZE"],
                             "write_kib": cal["WRITE_SIZE"], "fetch_scale": scale["FETCH_SIZE"],
                             "write_scale": scale["WRITE_SIZE"]},
        "decode_sources_hash": "sha256 of kernels.hip, decode_plan.h, device_common.h and "
                               "pkv_launch.h concatenated, comments and white space removed",
    })
    doc.setdefault("workloads", {})

    for wl in [w for w in a.decode.split(",") if w]:
        cfg, part = (int(x) for x in wl.split(":"))
        tag = f"c{cfg}" + (f"p{part}" if part else "")
        base = ["--", py, "-u", "bench.py", "--config", str(cfg), "--partition", str(part),
                "--others", "none", "--no-probe"]
        # the default workload is traced under exactly the default bench command
        default = cfg == 4 and part == 0
        trace_cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                     f"{a.out}/{tag}/trace", "-o", "t"] + (
                     ["--", py, "-u", "bench.py"] if default else base + [
                         "--steps", "20", "--warmup", "3", "--no-cpu-baseline"])
        line = bench_line(run(trace_cmd, f"{a.out}/{tag}_trace.log", 300))
        rows = stats_rows(f"{a.out}/{tag}/trace")
        # the pass-1 instance of this workload's cache dtype (the default
        # command also runs the other workloads, in other instances)
        inst = {2: "decode_partitions_kernel<1, 128", 3: "decode_partitions_kernel<1, 128",
                4: "decode_partitions_kernel<2, 128", 5: "decode_partitions_kernel<1, 128"}[cfg]
        every, flushed = dispatch_times(f"{a.out}/{tag}/trace", inst)
        got = {}
        pmc_cmds = []
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            d = f"{a.out}/{tag}/{counter.split('_')[0].lower()}"
            cmd = ["rocprofv3", "--pmc", counter, "--kernel-include-regex", KERNEL,
                   "--output-format", "csv", "-d", d, "-o", "t"] + base + [
                   "--steps", "5", "--warmup", "1", "--no-cpu-baseline", "--no-parity"]
            pmc_cmds.append(cmd)
            pl = bench_line(run(cmd, f"{a.out}/{tag}_{counter}.log", 300))
            v = per_dispatch(d, counter, KERNEL)
            got[counter] = (sum(v) / len(v), len(v), pl["roofline"]["bytes_per_launch"])
        mbase = base + ["--steps", "5", "--warmup", "1", "--no-cpu-baseline", "--no-parity"]
        mcmds, mvals = metric_runs(a, tag, mbase, KERNEL, py)
        fetch_kib, nd, alg = got["FETCH_SIZE"]
        write_kib = got["WRITE_SIZE"][0]
        rd = fetch_kib * 1024 * scale["FETCH_SIZE"]
        wr = write_kib * 1024 * scale["WRITE_SIZE"]
        hbm = rd + wr
        name = line["config"]["workload"]
        fname = f"decode_partitions_{SLUG[cfg]}" + (f"_p{part}" if part else "") + ".md"
        key = bench.workload_key(cfg, part)
        doc["workloads"][key] = {"workload": name, "hbm_bytes_per_launch": int(hbm),
                                 "fetch_kib": fetch_kib, "write_kib": write_kib,
                                 "summary": f"profiles/{fname}",
                                 "algorithmic_bytes_per_launch": int(alg)}
        p1 = [r for r in rows if inst in r["Name"]]
        p1_us = float(p1[0]["AverageNs"]) / 1e3 if p1 else float("nan")
        fl_us = sum(flushed) / len(flushed) if flushed else float("nan")
        r = line["roofline"]
        lines = [
            f"# Pass-1 kernel on {name}" + (f", split-KV partitions of {part} tokens" if part else ""),
            "",
            "Kernel statistics (rocprofv3), run from the repository root on one MI355X:",
            "",
            "```",
            " ".join(trace_cmd).replace(py, "python"),
            "```",
            "",
            "| kernel | calls | avg us | min us | max us | % of GPU time |",
            "|---|---|---|---|---|---|",
        ]
        for row in rows:
            lines.append(f"| `{short(row['Name'])}` | {row['Calls']} | {float(row['AverageNs']) / 1e3:.1f} | "
                         f"{float(row['MinNs']) / 1e3:.1f} | {float(row['MaxNs']) / 1e3:.1f} | "
                         f"{float(row['Percentage']):.1f} |")
        lines += [
            "",
            f"Under the profiler the bench line of this run read pass 1 at {r['avg_launch_us']} us "
            f"(mean of its {r['timed_launches']} timed launches, each after a 1 GiB read that "
            f"evicts L2 and MALL; HIP events on the launch stream), against {fl_us:.1f} us mean "
            f"kernel time of the {len(flushed)} pass-1 dispatches the trace shows right after that "
            f"read, and {p1_us:.1f} us over all {len(every)} dispatches of this instance (warm "
            f"steps included); algorithmic bytes per launch {r['bytes_per_launch'] / 1e9:.4f} GB "
            f"-> {r['achieved']} GB/s, {100 * r['frac']:.1f}% of 8 TB/s; whole step "
            f"{line['ms_per_step']} ms.",
            "",
            "## HBM traffic of the pass-1 kernel",
            "",
            "One counter per run:",
            "",
            "```",
            *[" ".join(c).replace(py, "python") for c in pmc_cmds],
            " ".join(cmds["copy_fetch"]).replace(py, "python"),
            " ".join(cmds["copy_write"]).replace(py, "python"),
            "```",
            "",
            f"- calibration: a {COPY_MIB} MiB device copy (`__amd_rocclr_copyBuffer`) reads FETCH_SIZE "
            f"{cal['FETCH_SIZE']:.0f} KiB and writes WRITE_SIZE {cal['WRITE_SIZE']:.0f} KiB per "
            f"dispatch, so the scale factors are fetch x{scale['FETCH_SIZE']:.3f}, write "
            f"x{scale['WRITE_SIZE']:.3f}",
            f"- pass 1, mean over {nd} dispatches: FETCH_SIZE {fetch_kib:.0f} KiB -> {rd / 1e9:.4f} GB "
            f"read; WRITE_SIZE {write_kib:.0f} KiB -> {wr / 1e6:.2f} MB written",
            f"- HBM bytes per launch {hbm / 1e9:.4f} GB against {alg / 1e9:.4f} GB algorithmic "
            f"({hbm / alg:.3f}x)",
            f"- pass-1 sources hash at measurement (sha256 of kernels.hip, decode_plan.h, "
            f"device_common.h, pkv_launch.h with comments and white space removed): `{sha}`",
            "",
            *metric_lines(mvals, 8),
            "```",
            *[" ".join(c).replace(py, "python") for c in mcmds],
            "```",
            "",
        ]
        with open(os.path.join(PROFILES, fname), "w") as f:
            f.write("\n".join(lines))
        log(f"{key}: pass 1 {p1_us:.1f} us (after the flush {fl_us:.1f} us), HBM {hbm / 1e9:.4f} GB vs algorithmic "
            f"{alg / 1e9:.4f} GB ({hbm / alg:.3f}x) -> profiles/{fname}")
        with open(COUNTERS, "w") as f:
            json.dump(doc, f, indent=1)
            f.write("\n")
    for wl in [w for w in a.prefill.split(",") if w]:
        cfg, chunk = (int(x) for x in wl.split(":"))
        tag = f"pf{cfg}c{chunk}"
        base = ["--", py, "-u", "bench.py", "--op", "prefill", "--config", str(cfg), "--chunk",
                str(chunk)]
        trace_cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                     f"{a.out}/{tag}/trace", "-o", "t"] + base + [
                     "--steps", "10", "--warmup", "2", "--no-cpu-baseline"]
        line = bench_line(run(trace_cmd, f"{a.out}/{tag}_trace.log", 300))
        rows = stats_rows(f"{a.out}/{tag}/trace")
        mbase = base + ["--steps", "3", "--warmup", "1", "--no-cpu-baseline"]
        got, pmc_cmds = {}, []
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            d = f"{a.out}/{tag}/{counter.split('_')[0].lower()}"
            cmd = ["rocprofv3", "--pmc", counter, "--kernel-include-regex", PREFILL_KERNEL,
                   "--output-format", "csv", "-d", d, "-o", "t"] + mbase
            pmc_cmds.append(cmd)
            run(cmd, f"{a.out}/{tag}_{counter}.log", 300)
            v = per_dispatch(d, counter, PREFILL_KERNEL)
            got[counter] = sum(v) / len(v)
        mcmds, mvals = metric_runs(a, tag, mbase, PREFILL_KERNEL, py)
        rd = got["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"]
        wr = got["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
        r = line["roofline"]
        pk = [x for x in rows if PREFILL_KERNEL in x["Name"]]
        k_us = float(pk[0]["AverageNs"]) / 1e3 if pk else float("nan")
        name = line["config"]["workload"]
        fname = f"prefill_kernel_{SLUG[cfg]}_chunk{chunk}.md"
        lines = [
            f"# Chunked-prefill kernel on {name}, chunk {chunk}",
            "",
            f"Every sequence attends its last {chunk} cached tokens causally over its whole paged "
            f"context ({line['config']['query_tokens']} query tokens in all).",
            "",
            "Kernel statistics (rocprofv3), run from the repository root on one MI355X:",
            "",
            "```",
            " ".join(trace_cmd).replace(py, "python"),
            "```",
            "",
            "| kernel | calls | avg us | min us | max us | % of GPU time |",
            "|---|---|---|---|---|---|",
        ]
        for row in rows:
            lines.append(f"| `{short(row['Name'])}` | {row['Calls']} | {float(row['AverageNs']) / 1e3:.1f} | "
                         f"{float(row['MinNs']) / 1e3:.1f} | {float(row['MaxNs']) / 1e3:.1f} | "
                         f"{float(row['Percentage']):.1f} |")
        lines += [
            "",
            f"Under the profiler the bench line read the kernel at {r['avg_launch_us']} us (HIP "
            f"events on the launch stream) against {k_us:.1f} us average kernel time above; "
            f"algorithmic work per launch {r['flops_per_launch'] / 1e12:.4f} TFLOP (4 * D per "
            f"visible (row, head, token)) -> {r['achieved']} TFLOP/s, {100 * r['frac']:.1f}% of the "
            f"{r['peak']:.0f} TFLOP/s dense MFMA peak of its compute dtype.",
            "",
            "## Fabric traffic of the prefill kernel",
            "",
            "```",
            *[" ".join(c).replace(py, "python") for c in pmc_cmds],
            "```",
            "",
            f"FETCH_SIZE {got['FETCH_SIZE']:.0f} KiB and WRITE_SIZE {got['WRITE_SIZE']:.0f} KiB per "
            f"dispatch, scaled by the copy calibration (x{scale['FETCH_SIZE']:.3f}, "
            f"x{scale['WRITE_SIZE']:.3f}): {rd / 1e9:.3f} GB read and {wr / 1e9:.3f} GB written per "
            f"launch, against {line['kv_bytes'] / 1e9:.3f} GB of unique K/V bytes the chunks see "
            f"(every query item of a (head, sequence) pair re-reads the context, mostly from L2).",
            "",
            *metric_lines(mvals, 8),
            "```",
            *[" ".join(c).replace(py, "python") for c in mcmds],
            "```",
            "",
        ]
        with open(os.path.join(PROFILES, fname), "w") as f:
            f.write("\n".join(lines))
        log(f"prefill {cfg}:{chunk}: {k_us:.1f} us, {r['achieved']} TFLOP/s, "
            f"MfmaUtil {mvals['MfmaUtil']:.1f}% VALUBusy {mvals['VALUBusy']:.1f}% -> profiles/{fname}")
    log("done")


if __name__ == "__main__":
    main()
