"""Benchmark of the paged decode-attention hot path on one MI355X.

One step = one decode step of one attention layer over a batch of resident
sequences, i.e. the whole hot path:
  a1  host block manager appends one token per sequence (a block is taken
      only at a block boundary); the slots and lengths are copied to the
      device (pinned, double-buffered, async);
  a2  the decode append writes each new token's K and V into its slot and
      sets the sequence's device table entry for the new position;
  a3-a8  decode attention: pass 1 (per-partition attention over the block
      table) and pass 2 (log-sum-exp merge of split-KV partials).
Inputs are resident in HBM before the timed region; each step decodes the
next token, so contexts grow by one per step.

Prints one JSON line.  `value` is KV GB/s over the whole step (algorithmic
KV bytes / step time); `roofline` is the pass-1 kernel's algorithmic bytes
per launch over its HIP-event-timed average duration, against 8 TB/s.  The
events bracket pass 1 on every fifth timed step (at least ten launches): an
event pair costs ~6 us of step time, which the other steps do not pay.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import re
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV GB/s and % of HBM peak; seq-tokens/s per layer"
HBM_PEAK_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "pass1_hbm_counters.json")
# the sources the pass-1 kernel is built from (the merge and prefill live apart)
DECODE_SRCS = [os.path.join(ROOT, "paged_kv_cache_189_amd", "csrc", n)
               for n in ("kernels.hip", "decode_plan.h", "device_common.h", "pkv_launch.h")]


def decode_sources_sha256():
    """Hash of the decode sources with comments and white space removed, so
    an edit of a comment keeps the counter figures measured on that code."""
    h = hashlib.sha256()
    for p in DECODE_SRCS:
        with open(p) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update(re.sub(r"\s+", "", src).encode())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload index (1-5)")
    ap.add_argument("--partition", type=int, default=-1,
                    help="tokens per split-KV partition (-1: the workload's choice)")
    ap.add_argument("--block-size", type=int, default=16, choices=(16, 32),
                    help="tokens per physical KV block")
    ap.add_argument("--op", default="decode", choices=("decode", "prefill", "sim"),
                    help="decode step (default), chunked-prefill attention, or the host-only "
                         "continuous-batching simulation")
    ap.add_argument("--chunk", type=int, default=512,
                    help="query tokens per sequence for --op prefill (the last ones of each context)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=0,
                    help="sequences in the oracle sample (0: the default for the workload)")
    ap.add_argument("--cold-launches", type=int, default=5,
                    help="after the timed steps, pass-1 launches each preceded by a 1 GiB read "
                         "(more than L2 + MALL), reported as roofline.cold_cache")
    ap.add_argument("--kernel-launches", type=int, default=10,
                    help="after the timed steps, steps with events around each kernel (append, "
                         "pass 1, merge), reported as step_kernels")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


# Split-KV partition size per workload (tokens); 0 = balanced ranges only.
# The 405B-shaped long-context workload is specified with 512-token partitions.
PARTITION = {1: 0, 2: 0, 3: 0, 4: 0, 5: 512}
CPU_SEQS = {1: 4, 2: 64, 3: 32, 4: 8, 5: 1}


def kv_bytes(spec, tables, lens):
    """Algorithmic KV bytes: tokens used in each UNIQUE physical block, times
    2 (K and V) * kv heads * head dim * bytes per element; and the logical
    figure that counts shared blocks once per sequence."""
    import workloads
    per_tok = 2 * spec.num_kv_heads * spec.head_dim * workloads.ELEM_BYTES[spec.cache_dtype]
    BS = spec.block_size
    lens = np.asarray(lens, dtype=np.int64)
    n = (lens + BS - 1) // BS
    cols = np.arange(tables.shape[1])[None, :]
    mask = cols < n[:, None]
    blocks = tables[mask].astype(np.int64)
    used = np.minimum(BS, (lens[:, None] - cols * BS))[mask]
    fill = np.zeros(int(blocks.max()) + 1 if blocks.size else 1, dtype=np.int64)
    np.maximum.at(fill, blocks, used)
    return int(fill.sum()) * per_tok, int(lens.sum()) * per_tok


def other_bytes(spec, lens):
    import workloads
    S = len(lens)
    qb = workloads.ELEM_BYTES[spec.q_dtype]
    ob = workloads.ELEM_BYTES[spec.out_dtype]
    tables = 4 * int(sum(-(-int(L) // spec.block_size) for L in lens))
    return S * spec.num_q_heads * spec.head_dim * (qb + ob) + tables + 4 * S


def copy_probe(mib):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "launches": 3}), flush=True)


def workload_key(config, partition, block_size=16):
    key = f"{config}:{partition}"
    return key if block_size == 16 else f"{key}:b{block_size}"


def traffic_from_counters(key):
    """HBM bytes per pass-1 launch of workload `key` from the committed
    rocprofv3 counter runs, or None when the kernel source changed since they
    were taken or the workload was not measured."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
        if c.get("decode_sources_sha256") != decode_sources_sha256():
            return None
        return c.get("workloads", {}).get(key)
    except (OSError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path is "
              "not sharded across GPUs in this library.", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_189_amd as pkv
    import workloads

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.op == "sim":
        sim_bench(args)
        return
    if args.op == "prefill":
        prefill_bench(args)
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pkv.lib()
    dev = torch.device("cuda:0")
    spec = dataclasses.replace(workloads.SPECS[args.config], block_size=args.block_size)
    BS = spec.block_size
    part = PARTITION[args.config] if args.partition < 0 else args.partition
    total_steps = args.warmup + args.steps
    lens0 = workloads.lengths(spec)
    S = len(lens0)
    t_build = time.perf_counter()
    w = workloads.make(spec, device=dev, lens=lens0)
    # table wide enough for the tokens this run appends
    width = w.max_blocks * BS + total_steps + BS
    max_blocks = -(-width // BS)
    nb_extra = S * (-(-total_steps // BS) + 1)
    # grow the pool for the appended tokens (fresh blocks hold N(0,1)-free garbage;
    # they are written by the cache write before they are read)
    if nb_extra:
        ks, vs = workloads.pool_shapes(nb_extra, spec.num_kv_heads, spec.head_dim, spec.cache_dtype,
                                       BS)
        w.k_cache = torch.cat([w.k_cache, torch.zeros(ks, dtype=w.k_cache.dtype, device=dev)])
        w.v_cache = torch.cat([w.v_cache, torch.zeros(vs, dtype=w.v_cache.dtype, device=dev)])
    num_blocks = w.num_blocks + nb_extra
    order = np.concatenate([w.free_order, np.arange(w.num_blocks, num_blocks, dtype=np.int32)])
    bm = pkv.BlockManager(num_blocks, BS, max_blocks, order)
    slots0 = workloads.allocate_context(bm, spec, lens0)  # context + first decode token
    ids = np.arange(S, dtype=np.int64)
    _, tables0, blens = bm.export(ids)
    workloads.poison_unused(w, tables0[:, : w.max_blocks], lens0 - 1)

    out_dtype = torch.float32 if spec.out_dtype == workloads.F32 else torch.bfloat16
    # Device block tables are copied once; afterwards a step sends its slots
    # and lengths in one small packed buffer, and the decode append that
    # writes the new tokens' K/V also sets each sequence's table entry for
    # its new position (a fresh block at a block boundary).
    d_tables = torch.from_numpy(tables0).to(dev)
    meta_bytes = 8 * S + 4 * S

    def views(buf):
        return buf[:8 * S].view(torch.int64), buf[8 * S:12 * S].view(torch.int32)

    d_meta = torch.empty(meta_bytes, dtype=torch.uint8, device=dev)
    d_slots, d_lens = views(d_meta)
    params = pkv.make_decode_params(w.q, w.k_cache, d_tables, max_blocks * BS, w.scale, w.k_scale,
                                    w.v_scale, out_dtype, part)
    ws = torch.empty(max(pkv.pkv_decode_workspace_bytes(params), 256), dtype=torch.uint8, device=dev)
    out = torch.empty(w.q.shape, dtype=out_dtype, device=dev)
    lse = torch.empty((S, spec.num_q_heads), dtype=torch.float32, device=dev)
    # two pinned host buffers for the per-step metadata
    pin = []
    for _ in range(2):
        hb = torch.empty(meta_bytes, dtype=torch.uint8, pin_memory=True)
        hs, hl = views(hb)
        pin.append(dict(raw=hb, slots=hs, lens=hl))
    host_lens = blens.astype(np.int32).copy()
    copied = [torch.cuda.Event(), torch.cuda.Event()]
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    build_s = time.perf_counter() - t_build

    lens_per_step = []  # every timed step
    ev, ev_lens = [], []  # the event-timed pass-1 launches and their lengths

    # pass 1 is bracketed by events on every EVENT_EVERY-th timed step
    event_every = max(1, min(5, args.steps // 10))

    def step(i, timed):
        sampled = timed and (i - args.warmup) % event_every == 0
        buf = pin[i % 2]
        copied[i % 2].synchronize()  # the copy that last read this buffer is done
        sl, ln = buf["slots"].numpy(), buf["lens"].numpy()
        if i == 0:
            sl[:], ln[:] = slots0, host_lens
        else:
            rc, _ = bm.append_slots(ids, out=sl)                       # a1
            assert rc == 0, rc
            host_lens[:] += 1
            ln[:] = host_lens
        d_meta.copy_(buf["raw"], non_blocking=True)
        copied[i % 2].record(stream)
        pkv.pkv_append_decode_tokens(w.k_new, w.v_new, w.k_cache, w.v_cache, d_slots,  # a2
                                     d_lens, d_tables, w.k_scale, w.v_scale)
        if sampled:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        pkv.pkv_decode_attention_partitions(params, out, w.q, w.k_cache, w.v_cache, d_tables,
                                            d_lens, ws, lse)                     # a3-a6, a8
        if sampled:
            e1.record(stream)
            ev.append((e0, e1))
            ev_lens.append(ln.copy())
        if timed:
            lens_per_step.append(ln.copy())
        pkv.pkv_decode_attention_merge(params, out, d_lens, ws, lse)             # a7

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, total_steps):
        step(i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    pass1_ms = [a.elapsed_time(b) for a, b in ev]
    pass1_avg_ms = float(np.mean(pass1_ms))
    # Each kernel of the step on its own, events around every launch, after
    # the timed steps so their clocks stay untouched.  The append repeats the
    # last step's (same tokens, slots and table entries: it rewrites what is
    # there), so the state checked below is unchanged.
    kev = []
    for _ in range(args.kernel_launches):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        pkv.pkv_append_decode_tokens(w.k_new, w.v_new, w.k_cache, w.v_cache, d_slots, d_lens,
                                     d_tables, w.k_scale, w.v_scale)
        e[1].record(stream)
        pkv.pkv_decode_attention_partitions(params, out, w.q, w.k_cache, w.v_cache, d_tables,
                                            d_lens, ws, lse)
        e[2].record(stream)
        pkv.pkv_decode_attention_merge(params, out, d_lens, ws, lse)
        e[3].record(stream)
        kev.append(e)
    torch.cuda.synchronize()
    step_kernels = None
    if kev:
        us = np.array([[e[k].elapsed_time(e[k + 1]) * 1e3 for k in range(3)] for e in kev])
        step_kernels = {"append_a2_us": round(float(us[:, 0].mean()), 2),
                        "pass1_us": round(float(us[:, 1].mean()), 2),
                        "merge_a7_us": round(float(us[:, 2].mean()), 2),
                        "launches": len(kev),
                        "how": "HIP events around each kernel, after the timed steps"}

    # Cold caches: back-to-back steps of one layer re-read the same blocks, and
    # lines kept by the default-policy loads survive in the 256 MB MALL into
    # the next step, which a model's other layers would evict.  These launches
    # repeat pass 1 on the final state, each after reading 1 GiB (which evicts
    # L2 and MALL without leaving dirty lines to drain during pass 1).
    cold = None
    if args.cold_launches > 0:
        flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.zeros((), dtype=torch.float32, device=dev)
        sink.add_(flush.sum())  # the zero fill's dirty lines drain here
        cev = []
        for _ in range(args.cold_launches):
            sink.add_(flush.sum())
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            pkv.pkv_decode_attention_partitions(params, out, w.q, w.k_cache, w.v_cache, d_tables,
                                                d_lens, ws, lse)
            c1.record(stream)
            pkv.pkv_decode_attention_merge(params, out, d_lens, ws, lse)
            cev.append((c0, c1))
        torch.cuda.synchronize()
        cold_ms = float(np.mean([a.elapsed_time(b) for a, b in cev]))
        del flush

    # algorithmic bytes, step by step (contexts grow by one token per step)
    _, tables_now, lens_now = bm.export(ids)
    # the device tables kept by the decode append must equal the manager's
    assert np.array_equal(d_tables.cpu().numpy(), tables_now), "device block tables drifted"
    assert np.array_equal(lens_now, host_lens), "context lengths drifted"
    kv_u, kv_l = [], []
    for ln in lens_per_step:
        u, l = kv_bytes(spec, tables_now, ln)
        kv_u.append(u)
        kv_l.append(l)
    kv_step = float(np.mean(kv_u))
    pass1_bytes = float(np.mean([kv_bytes(spec, tables_now, ln)[0] + other_bytes(spec, ln)
                                 for ln in ev_lens]))
    achieved = pass1_bytes / (pass1_avg_ms * 1e-3) / 1e9
    value = kv_step / (ms_per_step * 1e-3) / 1e9
    seq_tok_s = S / (ms_per_step * 1e-3)

    if cold is None and args.cold_launches > 0:
        cold_bytes = kv_bytes(spec, tables_now, host_lens)[0] + other_bytes(spec, host_lens)
        cold_gbs = cold_bytes / (cold_ms * 1e-3) / 1e9
        cold = {"achieved": round(cold_gbs, 1), "frac": round(cold_gbs / HBM_PEAK_GBS, 4),
                "avg_launch_us": round(cold_ms * 1e3, 2), "launches": args.cold_launches,
                "before_each": "1 GiB read (evicts L2 and MALL)"}

    counters = traffic_from_counters(workload_key(args.config, part, BS))
    traffic = counters.get("hbm_bytes_per_launch") if counters else None

    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {workloads.F32: "f32", workloads.BF16: "bf16",
                  workloads.E4M3: "fp8-e4m3 kv, bf16 q/out"}[spec.cache_dtype],
        "data": "synthetic (seeded N(0,1) values, shuffled block tables)",
        "config": {"workload": spec.name, "seqs": S, "q_heads": spec.num_q_heads,
                   "kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim, "block_size": BS,
                   "partition_tokens": pkv.pkv_decode_partition_size(params),
                   "mean_context": float(np.mean(lens_per_step[0])), "parallelism": "1 GPU"},
        "seq_tokens_per_s_per_layer": round(seq_tok_s, 1),
        "kv_bytes_per_step": int(kv_step),
        "kv_bytes_per_step_logical": int(np.mean(kv_l)),
        "roofline": {"bound": "hbm", "kernel": "decode_partitions_kernel (pass 1)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": int(pass1_bytes), "avg_launch_us": round(pass1_avg_ms * 1e3, 2),
                     "timed_launches": len(ev), "cold_cache": cold},
        "step_kernels": step_kernels,
        "setup_s": round(build_s, 1),
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, w, bm, ids, args, pkv, torch)
    print(json.dumps(res), flush=True)


MFMA_PEAK_TFLOPS = {0: 157.3, 1: 2500.0, 2: 2500.0}  # fp32 MFMA; bf16 MFMA (fp8 KV is widened to bf16)


def sim_bench(args):
    """Host-only: the block manager under continuous batching on a synthetic
    request trace, paging versus a static reservation of max_model_len, and
    paging with the prefix cache.  Shape: Llama-3-8B on a 40 GB GPU with 90%
    of its memory for the engine (16 GB of weights, 128 KiB of KV per token),
    max-model-len 8192, max-num-seqs 256, 16-token blocks; 2000 requests with
    log-normal prompt (median 600) and output (median 250) lengths, 60% of
    them opening with one of four 512-token system prompts."""
    import paged_kv_cache_189_amd as pkv
    rng = np.random.default_rng(2024)
    R, BS, ML, MNS = 2000, 16, 8192, 256
    kv_per_token = 2 * 32 * 8 * 128 * 2
    nb = int((40e9 * 0.90 - 16.06e9) // (kv_per_token * BS))
    systems = [list(rng.integers(0, 32000, 512)) for _ in range(4)]
    prompts, outs = [], []
    for r in range(R):
        n = int(np.clip(np.rint(rng.lognormal(np.log(600), 0.8)), 1, 6000))
        o = int(np.clip(np.rint(rng.lognormal(np.log(250), 0.8)), 1, 2000))
        p = list(rng.integers(0, 32000, n))
        if rng.random() < 0.6:
            p = systems[int(rng.integers(0, 4))] + p
        prompts.append(p[: ML - o])
        outs.append(o)
    pl = np.array([len(p) for p in prompts], dtype=np.int32)
    ol = np.array(outs, dtype=np.int32)
    ids = np.concatenate(prompts).astype(np.int32)
    runs = {}
    for name, pol, cache in (("static_reservation", pkv.PKV_SIM_STATIC, False),
                             ("paged", pkv.PKV_SIM_PAGED, False),
                             ("paged_prefix_cache", pkv.PKV_SIM_PAGED, True)):
        t0 = time.perf_counter()
        rc, res, _ = pkv.pkv_sim_run(nb, BS, ML, MNS, pol, pl, ol, ids, cache)
        secs = time.perf_counter() - t0
        assert rc == pkv.PKV_OK, pkv.lib().pkv_last_error().decode()
        res["tokens_per_iteration"] = round(res["generated_tokens"] / res["iterations"], 2)
        res["host_us_per_iteration"] = round(secs * 1e6 / res["iterations"], 2)
        res["mean_running"] = round(res["mean_running"], 2)
        res["mean_kv_utilization"] = round(res["mean_kv_utilization"], 4)
        runs[name] = res
    ratio = runs["paged"]["tokens_per_iteration"] / runs["static_reservation"]["tokens_per_iteration"]
    print(json.dumps({"metric": "continuous-batching simulation: generated tokens per iteration",
                      "value": runs["paged"]["tokens_per_iteration"], "unit": "tokens/iteration",
                      "higher_is_better": True, "data": "synthetic request trace (seeded)",
                      "config": {"requests": R, "num_blocks": nb, "block_size": BS,
                                 "max_model_len": ML, "max_num_seqs": MNS},
                      "paged_over_static": round(ratio, 3), "runs": runs}), flush=True)


def prefill_bench(args):
    """Chunked-prefill attention: every sequence of the workload attends its
    last `chunk` tokens causally over its whole paged context (K/V already in
    the cache).  Roofline against the dense MFMA peak of the compute dtype:
    algorithmic FLOPs = sum over query rows and heads of 4 * D * (p + 1)."""
    import torch

    import paged_kv_cache_189_amd as pkv
    import workloads
    dev = torch.device("cuda:0")
    spec = dataclasses.replace(workloads.SPECS[args.config], block_size=args.block_size)
    BS = spec.block_size
    lens = workloads.lengths(spec)
    S = len(lens)
    w = workloads.make(spec, device=dev, lens=lens)
    bm = pkv.BlockManager(w.num_blocks, BS, w.max_blocks, w.free_order)
    workloads.allocate_context(bm, spec, lens)
    ids = np.arange(S, dtype=np.int64)
    _, tables, blens = bm.export(ids)
    workloads.poison_unused(w, tables, blens)
    chunks = np.minimum(blens, args.chunk).astype(np.int64)
    qstart = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    R = int(qstart[-1])
    gen = torch.Generator(device=dev).manual_seed(7000 + spec.index)
    qdt = torch.float32 if spec.q_dtype == workloads.F32 else torch.bfloat16
    q = torch.randn((R, spec.num_q_heads, spec.head_dim), generator=gen, device=dev).to(qdt)
    out = torch.empty_like(q)
    lse = torch.empty((R, spec.num_q_heads), dtype=torch.float32, device=dev)
    d_tables = torch.from_numpy(tables).to(dev)
    d_lens = torch.from_numpy(blens).to(dev)
    d_qs = torch.from_numpy(qstart).to(dev)
    p = pkv.make_prefill_params(q, w.k_cache, d_tables, S, w.max_blocks * BS, w.scale, w.k_scale,
                                w.v_scale, qdt)
    run = lambda: pkv.pkv_prefill_attention(p, out, q, w.k_cache, w.v_cache, d_tables, d_lens,
                                            d_qs, lse)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # causal work: row j of sequence s sees L_s - C_s + j + 1 tokens
    seen = sum(int(c) * (int(L) - int(c)) + int(c) * (int(c) + 1) // 2 for L, c in zip(blens, chunks))
    flops = 4.0 * spec.num_q_heads * spec.head_dim * seen
    kvb, _ = kv_bytes(spec, tables, blens)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[spec.cache_dtype]
    res = {"metric": "chunked prefill attention: TFLOP/s", "value": round(tflops, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 4), "higher_is_better": True, "vs_baseline": None,
           "dtype": {0: "f32", 1: "bf16", 2: "fp8-e4m3 kv, bf16 q/out"}[spec.cache_dtype],
           "data": "synthetic (seeded N(0,1) values, shuffled block tables)",
           "config": {"workload": spec.name, "seqs": S, "query_tokens": R, "chunk": args.chunk,
                      "block_size": BS, "parallelism": "1 GPU"},
           "kv_bytes": int(kvb), "kv_gbs": round(kvb / (ms * 1e-3) / 1e9, 1),
           "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(tflops, 2),
                        "peak": peak, "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                        "traffic": None, "flops_per_launch": flops,
                        "avg_launch_us": round(ms * 1e3, 2)}}
    print(json.dumps(res), flush=True)


def cpu_baseline(spec, w, bm, ids, args, pkv, torch):
    """The fp64 oracle, untuned, on a bounded sample of the same workload:
    its cache write stores each sampled sequence's decode token and its
    attention runs over the sampled sequences.  Host copies of the sampled
    sequences' blocks are made before the clock starts."""
    from oracle import oracle as O
    import workloads
    BS = spec.block_size
    k = min(args.cpu_seqs or CPU_SEQS[spec.index], len(ids))
    seqs = np.arange(k)
    _, tables, lens = bm.export(ids[:k])
    n = [-(-int(L) // BS) for L in lens]
    blocks = np.unique(np.concatenate([tables[i, :n[i]] for i in range(k)]))
    remap = np.full(int(tables.max()) + 1, -1, dtype=np.int64)
    remap[blocks] = np.arange(len(blocks))
    t = np.full(tables.shape, -1, dtype=np.int32)
    for i in range(k):
        t[i, :n[i]] = remap[tables[i, :n[i]]]
    idx = torch.from_numpy(blocks.astype(np.int64)).to(w.k_cache.device)

    def host(x):
        x = x.cpu()
        return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()

    kc, vc = host(w.k_cache.index_select(0, idx)), host(w.v_cache.index_select(0, idx))
    q = np.ascontiguousarray(host(w.q[:k]))
    kn = np.ascontiguousarray(host(w.k_new[:k]))
    vn = np.ascontiguousarray(host(w.v_new[:k]))
    pos = np.maximum(lens - 1, 0)  # the decode token of each sampled sequence
    slots = np.array([t[i, pos[i] // BS] * BS + pos[i] % BS for i in range(k)], dtype=np.int64)
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():  # the share this job was given
        cores = max(1, min(cores, int(os.environ["OMP_NUM_THREADS"])))
    reps = 0
    t0 = time.perf_counter()
    while True:  # repeat the sampled step until about 10 s of CPU work
        O.reshape_and_cache(kn, vn, spec.q_dtype, kc, vc, spec.cache_dtype, slots, BS, w.k_scale,
                            w.v_scale)
        O.decode_attention(q, spec.q_dtype, kc, vc, spec.cache_dtype, t, lens, spec.num_kv_heads,
                           BS, w.scale, w.k_scale, w.v_scale, threads=cores)
        reps += 1
        secs = time.perf_counter() - t0
        if secs >= 10.0 or reps >= 50:
            break
    per_tok = 2 * spec.num_kv_heads * spec.head_dim * workloads.ELEM_BYTES[spec.cache_dtype]
    kvb = int(np.sum(lens)) * per_tok * reps
    return {"value": round(kvb / secs / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seq_tokens_per_s_per_layer": round(k * reps / secs, 2), "seconds": round(secs, 2),
            "sample": f"{k} of {len(ids)} sequences of one step (all {spec.num_q_heads} query heads, "
                      f"{int(np.sum(lens))} tokens), cache write + fp64 attention, repeated {reps}x"}


if __name__ == "__main__":
    main()
