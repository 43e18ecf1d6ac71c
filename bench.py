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

Default workload: the 70B-shaped layer with an fp8 E4M3 KV cache (256
sequences, the largest of the five), with the other full-size workloads
(Llama-3-8B-shaped, 70B with a shared prefix, 405B long context with 512-token
partitions) measured the same way and reported in the same line.

Timing protocol per workload: W untimed warm-up steps; then K timed steps,
each preceded by a 1 GiB read that evicts L2 and the 256 MB MALL (a model's
other layers would have evicted them between two steps of one layer), each
bracketed by HIP events on the launch stream (step: from the metadata copy
to the end of the merge; pass 1 alone; pass 1 + pass 2); then K warm steps
back to back, timed by the wall clock; then a few steps with events around
every kernel.  `value`, `ms_per_step` and `roofline` are the flushed figures;
the warm ones sit beside them.  The timed region (the K flushed steps,
flushes included) is bracketed by synchronizations; its wall time is reported
too.

After the timed steps the state of each workload's last step is checked
against the fp64 oracle on a sample of sequences: the oracle gets the
generated pool as it was before any library write, its own allocator's
tables, and its own cache write of every token the steps appended.  On the
default workload the same oracle run, repeated, is the CPU baseline.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
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
FLUSH_BYTES = 1 << 30
TOL = {0: None, 1: 1e-2, 2: 3e-2}  # by cache dtype: fp32 is 1e-5 of each row's largest |value|


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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, help="headline workload (1-5)")
    ap.add_argument("--others", default="2,3,5",
                    help="further workloads measured and reported in the same line ('none' for none)")
    ap.add_argument("--partition", type=int, default=-1,
                    help="tokens per split-KV partition of the headline workload (-1: its own)")
    ap.add_argument("--block-size", type=int, default=16, choices=(16, 32),
                    help="tokens per physical KV block")
    ap.add_argument("--op", default="decode", choices=("decode", "prefill", "sim"),
                    help="decode step (default), chunked-prefill attention, or the host-only "
                         "continuous-batching simulation")
    ap.add_argument("--chunk", type=int, default=512,
                    help="query tokens per sequence for --op prefill (the last ones of each context)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle check of the final state")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU work of the repeated oracle run behind cpu_baseline")
    ap.add_argument("--kernel-launches", type=int, default=10,
                    help="after the timed steps, steps with events around each kernel (append, "
                         "pass 1, merge), reported as step_kernels")
    ap.add_argument("--no-probe", action="store_true", help="skip the read-bandwidth probe")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


# Split-KV partition size per workload (tokens); 0 = balanced ranges only.
# The 405B-shaped long-context workload is specified with 512-token partitions.
PARTITION = {1: 0, 2: 0, 3: 0, 4: 0, 5: 512}
# sequences of each workload checked against the oracle (and, for the
# headline, timed as the CPU baseline)
PARITY_SEQS = {1: 4, 2: 8, 3: 8, 4: 8, 5: 1}


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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def job_cores():
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():  # the share this job was given
        cores = max(1, min(cores, int(os.environ["OMP_NUM_THREADS"])))
    return cores


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ read ceiling
def read_ceiling(pkv, torch, gib=4):
    """The read-bandwidth probe over `gib` GiB (more than L2 + MALL): a
    contiguous sweep (default policy, non-temporal) and 4 KiB tiles in a
    shuffled order (non-temporal), three timed launches each; GB/s of each
    and the best."""
    dev = torch.device("cuda:0")
    nbytes = gib << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    buf.random_(0, 1 << 30)
    grid = 256 * 32
    sink = torch.zeros(grid * 256, dtype=torch.int32, device=dev)
    tile = 4096
    gen = torch.Generator(device=dev).manual_seed(1234)
    order = torch.randperm(nbytes // tile, device=dev, generator=gen).to(torch.int32)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, mode in (("sweep_default", 0), ("sweep_nontemporal", 1), ("tiles_4k_shuffled_nt", 2)):
        kw = dict(order=order, tile_bytes=tile) if mode == 2 else {}
        pkv.pkv_read_probe(buf, mode, sink, grid=grid, **kw)  # warm-up
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pkv.pkv_read_probe(buf, mode, sink, grid=grid, **kw)
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        ms = min(a.elapsed_time(b) for a, b in ts)
        res[name] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf, order, sink
    torch.cuda.empty_cache()
    res["best_gbs"] = max(res.values())
    res["bytes"] = nbytes
    res["how"] = "pkv_read_probe, best of 3 event-timed launches per form"
    return res


# ------------------------------------------------------------------ one workload
class OracleSample:
    """The oracle's view of a sample of sequences at the final step, made
    before the library writes anything: the generated pool bytes of the
    blocks the sequences will hold, gathered from the device, with tables
    from the oracle's own allocator replaying the run's appends."""

    def __init__(self, spec, w, order, num_blocks, max_blocks, lens0, n_steps, k, torch):
        from oracle import oracle as O
        import workloads
        BS = spec.block_size
        S = len(lens0)
        ob = O.BlockAllocator(num_blocks, BS, max_blocks, order)
        workloads.allocate_context(ob, spec, lens0)
        ids = np.arange(S, dtype=np.int64)
        for _ in range(n_steps - 1):
            rc, _ = ob.append_slots(ids)
            assert rc == 0, rc
        _, tables, lens = ob.export(ids)
        # sequences: evenly spread over the batch, the longest included
        seqs = np.unique(np.concatenate([np.linspace(0, S - 1, min(k, S)).round().astype(np.int64),
                                         [int(np.argmax(lens))]]))
        n = [-(-int(lens[s]) // BS) for s in seqs]
        blocks = np.unique(np.concatenate([tables[s, :n[i]] for i, s in enumerate(seqs)]))
        remap = np.full(int(tables.max()) + 1, -1, dtype=np.int64)
        remap[blocks] = np.arange(len(blocks))
        t = np.full((len(seqs), tables.shape[1]), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            t[i, :n[i]] = remap[tables[s, :n[i]]]
        idx = torch.from_numpy(blocks.astype(np.int64)).to(w.k_cache.device)
        self.kc = self.host(w.k_cache.index_select(0, idx), torch)
        self.vc = self.host(w.v_cache.index_select(0, idx), torch)
        sel = torch.from_numpy(seqs).to(w.q.device)
        self.q = np.ascontiguousarray(self.host(w.q.index_select(0, sel), torch))
        kn = self.host(w.k_new.index_select(0, sel), torch)
        vn = self.host(w.v_new.index_select(0, sel), torch)
        # every token the run appends: positions lens0 - 1 .. lens - 1, each
        # with its sequence's new K and V
        rows, slots = [], []
        for i, s in enumerate(seqs):
            for p in range(int(lens0[s]) - 1, int(lens[s])):
                rows.append(i)
                slots.append(int(t[i, p // BS]) * BS + p % BS)
        rows = np.array(rows)
        self.kn_all = np.ascontiguousarray(kn[rows])
        self.vn_all = np.ascontiguousarray(vn[rows])
        self.slots_all = np.array(slots, dtype=np.int64)
        # the last step's tokens alone (the timed CPU step)
        last = np.cumsum([int(lens[s]) - int(lens0[s]) + 1 for s in seqs]) - 1
        self.kn_last = np.ascontiguousarray(kn)
        self.vn_last = np.ascontiguousarray(vn)
        self.slots_last = self.slots_all[last]
        self.seqs, self.tables, self.lens = seqs, t, lens[seqs].astype(np.int32)
        self.lens_all = lens
        self.spec, self.w = spec, w

    @staticmethod
    def host(x, torch):
        x = x.cpu()
        return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()

    def write_all(self):
        from oracle import oracle as O
        s, w = self.spec, self.w
        O.reshape_and_cache(self.kn_all, self.vn_all, s.q_dtype, self.kc, self.vc, s.cache_dtype,
                            self.slots_all, s.block_size, w.k_scale, w.v_scale)

    def step(self, threads, seqs=None):
        """The oracle's decode step on the sample: cache write of the last
        step's tokens (rewriting what write_all put there) and fp64
        attention.  seqs: indices into the sample (default all)."""
        from oracle import oracle as O
        s, w = self.spec, self.w
        i = np.arange(len(self.seqs)) if seqs is None else np.asarray(seqs)
        O.reshape_and_cache(self.kn_last[i], self.vn_last[i], s.q_dtype, self.kc, self.vc,
                            s.cache_dtype, self.slots_last[i], s.block_size, w.k_scale, w.v_scale)
        return O.decode_attention(self.q[i], s.q_dtype, self.kc, self.vc, s.cache_dtype,
                                  self.tables[i], self.lens[i], s.num_kv_heads, s.block_size,
                                  w.scale, w.k_scale, w.v_scale, threads=threads)


def compare(spec, got, got_lse, ref, ref_lse):
    """Max error of the GPU rows against the oracle's, and whether it meets
    the bar of the cache dtype."""
    got = got.astype(np.float64)
    err = np.abs(got - ref)
    tol = TOL[spec.cache_dtype]
    if tol is None:
        rowmax = np.maximum(np.abs(ref).max(axis=2, keepdims=True), 1e-300)
        metric = float((err / rowmax).max())
        ok = metric <= 1e-5
        kind = "max |err| / row max |ref|"
    else:
        # the bar bounds the computation; a bf16 output adds its own rounding,
        # half a bf16 ulp of the value
        _, e = np.frexp(np.abs(ref))
        half_ulp = np.where(ref == 0, 0.0, np.ldexp(1.0, e - 9))
        metric = float(err.max())
        ok = bool(np.all(err <= tol + half_ulp))
        kind = "max abs err (bar: tol + half a bf16 ulp of the value)"
    fin = np.isfinite(ref_lse)
    lerr = float(np.abs(got_lse[fin] - ref_lse[fin]).max() / max(1.0, np.abs(ref_lse[fin]).max())) \
        if fin.any() else 0.0
    ok = ok and bool(np.all(np.isfinite(got))) and np.array_equal(fin, np.isfinite(got_lse)) \
        and lerr <= 1e-4
    return {"max_err": metric, "kind": kind, "tol": tol if tol is not None else 1e-5,
            "max_abs_ref": float(np.abs(ref).max()), "lse_rel_err": lerr, "ok": bool(ok)}


def run_workload(args, index, part_arg, pkv, torch, flush, sink, headline):
    import workloads
    dev = torch.device("cuda:0")
    spec = dataclasses.replace(workloads.SPECS[index], block_size=args.block_size)
    BS = spec.block_size
    part = PARTITION[index] if part_arg < 0 else part_arg
    W, K = args.warmup, args.steps
    n_steps = W + 2 * K  # warm-up, flushed, warm; the first uses the context's own decode token
    lens0 = workloads.lengths(spec)
    S = len(lens0)
    t_build = time.perf_counter()
    w = workloads.make(spec, device=dev, lens=lens0)
    width = w.max_blocks * BS + n_steps + BS
    max_blocks = -(-width // BS)
    nb_extra = S * (-(-n_steps // BS) + 1)
    if nb_extra:  # room for the appended tokens (written before they are read)
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
    sample = None
    if not args.no_parity or (headline and not args.no_cpu_baseline):
        sample = OracleSample(spec, w, order, num_blocks, max_blocks, lens0, n_steps,
                              PARITY_SEQS[index], torch)

    out_dtype = torch.float32 if spec.out_dtype == workloads.F32 else torch.bfloat16
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

    def do_flush():
        sink.add_(flush.sum())  # a 1 GiB read: evicts L2 and the MALL, leaves no dirty lines

    def step(i, ev=None):
        """One decode step; ev = (u0, e0, p0, p1, e1) events: metadata upload
        start, step start (the metadata in HBM), pass 1 start and end, step
        end."""
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
        lens_now = ln.copy()
        if ev is not None:
            do_flush()
            ev[0].record(stream)
        d_meta.copy_(buf["raw"], non_blocking=True)
        copied[i % 2].record(stream)
        if ev is not None:
            ev[1].record(stream)
        pkv.pkv_append_decode_tokens(w.k_new, w.v_new, w.k_cache, w.v_cache, d_slots,  # a2
                                     d_lens, d_tables, w.k_scale, w.v_scale)
        if ev is not None:
            ev[2].record(stream)
        pkv.pkv_decode_attention_partitions(params, out, w.q, w.k_cache, w.v_cache, d_tables,
                                            d_lens, ws, lse)                     # a3-a6, a8
        if ev is not None:
            ev[3].record(stream)
        pkv.pkv_decode_attention_merge(params, out, d_lens, ws, lse)             # a7
        if ev is not None:
            ev[4].record(stream)
        return lens_now

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    # flushed, event-timed steps (the headline protocol)
    evs, lens_flushed = [], []
    t0 = time.perf_counter()
    for i in range(W, W + K):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        lens_flushed.append(step(i, e))
        evs.append(e)
    torch.cuda.synchronize()
    flushed_wall_s = time.perf_counter() - t0
    step_ms = np.array([e[1].elapsed_time(e[4]) for e in evs])
    upload_step_ms = np.array([e[0].elapsed_time(e[4]) for e in evs])
    pass1_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    attn_ms = np.array([e[2].elapsed_time(e[4]) for e in evs])
    # warm steps back to back, wall clock
    lens_warm = []
    t0 = time.perf_counter()
    for i in range(W + K, n_steps):
        lens_warm.append(step(i))
    torch.cuda.synchronize()
    warm_step_ms = (time.perf_counter() - t0) * 1e3 / K
    # each kernel on its own, warm (the append repeats the last step's tokens
    # and slots, which rewrites what is there)
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
    us = np.array([[e[k].elapsed_time(e[k + 1]) * 1e3 for k in range(3)] for e in kev]) \
        if kev else np.full((1, 3), np.nan)

    # the device tables kept by the decode append must equal the manager's
    _, tables_now, lens_now = bm.export(ids)
    assert np.array_equal(d_tables.cpu().numpy(), tables_now), "device block tables drifted"
    assert np.array_equal(lens_now, host_lens), "context lengths drifted"

    def kv(ln):
        return kv_bytes(spec, tables_now, ln)

    kv_f = np.array([kv(ln)[0] for ln in lens_flushed], dtype=np.float64)
    kv_fl = np.array([kv(ln)[1] for ln in lens_flushed], dtype=np.float64)
    p1_f = kv_f + np.array([other_bytes(spec, ln) for ln in lens_flushed], dtype=np.float64)
    kv_w = np.array([kv(ln)[0] for ln in lens_warm], dtype=np.float64)
    p1_last = kv(host_lens)[0] + other_bytes(spec, host_lens)
    flushed_gbs = float(np.mean(kv_f / (step_ms * 1e-3)) / 1e9)
    p1_gbs = float(np.mean(p1_f / (pass1_ms * 1e-3)) / 1e9)
    warm_p1_gbs = float(p1_last / (np.mean(us[:, 1]) * 1e-6) / 1e9)
    res = {
        "workload": spec.name, "index": index, "seqs": S,
        "partition_tokens": pkv.pkv_decode_partition_size(params), "block_size": BS,
        "pass1_ranges": pkv.pkv_decode_num_ranges(params),
        "mean_context": float(np.mean(lens_flushed[0])),
        "kv_bytes_per_step": int(np.mean(kv_f)), "kv_bytes_per_step_logical": int(np.mean(kv_fl)),
        "pass1_bytes_per_launch": int(np.mean(p1_f)),
        "flushed": {
            "step_ms": round(float(np.mean(step_ms)), 4),
            "step_ms_median": round(float(np.median(step_ms)), 4),
            "step_ms_min": round(float(np.min(step_ms)), 4),
            "kv_gbs": round(flushed_gbs, 1),
            "seq_tokens_per_s_per_layer": round(S / (np.mean(step_ms) * 1e-3), 1),
            "step_ms_incl_metadata_upload": round(float(np.mean(upload_step_ms)), 4),
            "kv_gbs_incl_metadata_upload": round(float(np.mean(kv_f / (upload_step_ms * 1e-3))) / 1e9, 1),
            "attention_us": round(float(np.mean(attn_ms)) * 1e3, 2),
            "attention_us_median": round(float(np.median(attn_ms)) * 1e3, 2),
            "attention_us_min": round(float(np.min(attn_ms)) * 1e3, 2),
            "pass1_us": round(float(np.mean(pass1_ms)) * 1e3, 2),
            "pass1_gbs": round(p1_gbs, 1), "pass1_frac": round(p1_gbs / HBM_PEAK_GBS, 4),
            "steps": K, "wall_s_incl_flushes": round(flushed_wall_s, 4)},
        "warm": {
            "step_ms": round(warm_step_ms, 4),
            "kv_gbs": round(float(np.mean(kv_w)) / (warm_step_ms * 1e-3) / 1e9, 1),
            "seq_tokens_per_s_per_layer": round(S / (warm_step_ms * 1e-3), 1),
            "pass1_us": round(float(np.mean(us[:, 1])), 2),
            "pass1_gbs": round(warm_p1_gbs, 1), "pass1_frac": round(warm_p1_gbs / HBM_PEAK_GBS, 4),
            "steps": K},
        "step_kernels": {"append_a2_us": round(float(us[:, 0].mean()), 2),
                         "pass1_us": round(float(us[:, 1].mean()), 2),
                         "merge_a7_us": round(float(us[:, 2].mean()), 2),
                         "launches": len(kev), "how": "HIP events around each kernel, warm"},
        "setup_s": round(build_s, 1),
    }
    counters = traffic_from_counters(workload_key(index, part, BS))
    res["traffic"] = counters.get("hbm_bytes_per_launch") if counters else None
    res["dtype"] = {workloads.F32: "f32", workloads.BF16: "bf16",
                    workloads.E4M3: "fp8-e4m3 kv, bf16 q/out"}[spec.cache_dtype]
    if sample is not None:
        assert np.array_equal(sample.lens_all, lens_now), "oracle allocator lengths differ"
        sample.write_all()
        cores = job_cores()
        t0 = time.perf_counter()
        ref, ref_lse = sample.step(cores)
        first_s = time.perf_counter() - t0
        sel = torch.from_numpy(sample.seqs).to(dev)
        got = out.index_select(0, sel).float().cpu().numpy()
        got_lse = lse.index_select(0, sel).cpu().numpy().astype(np.float64)
        if not args.no_parity:
            res["parity"] = dict(compare(spec, got, got_lse, ref, ref_lse),
                                 seqs=[int(s) for s in sample.seqs],
                                 what="final step's output and lse vs the fp64 oracle")
        if headline and not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline(spec, sample, cores, first_s, args.cpu_seconds)
    del w, ws, out, lse, d_tables
    torch.cuda.empty_cache()
    return res


def cpu_baseline(spec, sample, cores, first_s, seconds):
    """The fp64 oracle, untuned, on the sample: its cache write of the
    step's tokens and its attention over the sampled sequences, repeated for
    about `seconds`; then once on one thread over the shortest sampled
    sequence."""
    import workloads
    reps, t0 = 0, time.perf_counter()
    while True:
        sample.step(cores)
        reps += 1
        secs = time.perf_counter() - t0
        if secs + first_s >= seconds or reps >= 50:
            break
    per_tok = 2 * spec.num_kv_heads * spec.head_dim * workloads.ELEM_BYTES[spec.cache_dtype]
    k = len(sample.seqs)
    toks = int(np.sum(sample.lens))
    kvb = toks * per_tok * reps
    j = int(np.argmin(sample.lens))  # the shortest sampled sequence
    t1 = time.perf_counter()
    sample.step(1, [j])
    one_s = time.perf_counter() - t1
    one_tok = int(sample.lens[j])
    return {"value": round(kvb / secs / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seq_tokens_per_s_per_layer": round(k * reps / secs, 2), "seconds": round(secs, 2),
            "cpu_model": cpu_model(),
            "sample": f"{k} of {spec.num_seqs} sequences of the final step (all "
                      f"{spec.num_q_heads} query heads, {toks} tokens), cache write + fp64 "
                      f"attention, repeated {reps}x on {cores} threads",
            "one_thread": {"value": round(one_tok * per_tok / one_s / 1e9, 4), "unit": "GB/s",
                           "seconds": round(one_s, 3),
                           "seq_tokens_per_s_per_layer": round(1 / one_s, 3),
                           "sample": f"1 sequence of {one_tok} tokens, one run"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path is "
              "not sharded across GPUs in this library.", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_189_amd as pkv

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
    ceiling = None if args.no_probe else read_ceiling(pkv, torch)
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    sink.add_(flush.sum())  # the zero fill's dirty lines drain here
    log(f"workload {args.config} (headline)")
    head = run_workload(args, args.config, args.partition, pkv, torch, flush, sink, True)
    others = []
    for idx in [int(x) for x in args.others.split(",") if x.strip() and x.strip() != "none"]:
        if idx == args.config:
            continue
        log(f"workload {idx}")
        others.append(run_workload(args, idx, -1, pkv, torch, flush, sink, False))
    f = head["flushed"]
    r = {"bound": "hbm", "kernel": "decode_partitions_kernel (pass 1)",
         "achieved": f["pass1_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": f["pass1_frac"], "traffic": head["traffic"],
         "bytes_per_launch": head["pass1_bytes_per_launch"], "avg_launch_us": f["pass1_us"],
         "timed_launches": f["steps"],
         "protocol": "each launch after a 1 GiB read that evicts L2 and MALL; HIP events on the "
                     "launch stream",
         "warm": {"achieved": head["warm"]["pass1_gbs"], "frac": head["warm"]["pass1_frac"],
                  "avg_launch_us": head["warm"]["pass1_us"]}}
    if ceiling:
        r["ceiling"] = ceiling
        r["ceiling_frac"] = round(f["pass1_gbs"] / ceiling["best_gbs"], 4)
    parity_ok = all(x.get("parity", {}).get("ok", True) for x in [head] + others)
    res = {
        "metric": METRIC, "value": f["kv_gbs"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": f["step_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,1) values, shuffled block tables)",
        "config": {"workload": head["workload"], "seqs": head["seqs"],
                   "q_heads": workloads_spec(head["index"]).num_q_heads,
                   "kv_heads": workloads_spec(head["index"]).num_kv_heads,
                   "head_dim": workloads_spec(head["index"]).head_dim,
                   "block_size": head["block_size"], "partition_tokens": head["partition_tokens"],
                   "mean_context": head["mean_context"], "parallelism": "1 GPU"},
        "timing": "value and ms_per_step: mean over the timed steps of the step's HIP-event time "
                  "(decode append to merge end, the step's slots and lengths already in HBM), "
                  "each step after a 1 GiB read that evicts L2 and MALL; "
                  "flushed.step_ms_incl_metadata_upload adds their copy from pinned host memory "
                  "(PCIe); warm: back-to-back steps, wall clock, host work and upload included",
        "seq_tokens_per_s_per_layer": f["seq_tokens_per_s_per_layer"],
        "kv_bytes_per_step": head["kv_bytes_per_step"],
        "kv_bytes_per_step_logical": head["kv_bytes_per_step_logical"],
        "roofline": r,
        "flushed": f, "warm": head["warm"], "step_kernels": head["step_kernels"],
        "parity_max_err": head.get("parity", {}).get("max_err"),
        "parity": head.get("parity"), "parity_ok_all": parity_ok,
        "workloads": [summary(x) for x in [head] + others],
        "setup_s": head["setup_s"],
    }
    if "cpu_baseline" in head:
        res["cpu_baseline"] = head["cpu_baseline"]
    print(json.dumps(res), flush=True)
    if not parity_ok:
        print("bench.py: the GPU output of a timed state does not match the oracle", file=sys.stderr)
        sys.exit(1)


def workloads_spec(index):
    import workloads
    return workloads.SPECS[index]


def summary(x):
    """The per-workload figures kept in the line."""
    keys = ("workload", "index", "seqs", "partition_tokens", "pass1_ranges", "mean_context",
            "kv_bytes_per_step", "kv_bytes_per_step_logical", "pass1_bytes_per_launch", "traffic",
            "dtype")
    s = {k: x[k] for k in keys}
    s["flushed"] = {k: x["flushed"][k] for k in ("step_ms", "step_ms_median", "step_ms_min",
                                                 "kv_gbs", "seq_tokens_per_s_per_layer",
                                                 "step_ms_incl_metadata_upload", "attention_us",
                                                 "pass1_us", "pass1_gbs", "pass1_frac")}
    s["warm"] = {k: x["warm"][k] for k in ("step_ms", "kv_gbs", "seq_tokens_per_s_per_layer",
                                           "pass1_us", "pass1_frac")}
    s["merge_us"] = x["step_kernels"]["merge_a7_us"]
    s["append_us"] = x["step_kernels"]["append_a2_us"]
    if "parity" in x:
        s["parity"] = {k: x["parity"][k] for k in ("max_err", "kind", "tol", "max_abs_ref",
                                                   "lse_rel_err", "ok")}
        s["parity"]["seqs"] = len(x["parity"]["seqs"])
    return s


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


def prefill_oracle_leg(spec, w, lens, chunks, qstart, q, out, lse, torch, threads):
    """The oracle beside the prefill line: for the shortest and the longest
    sequence, the first and the last (up to) 16 rows of its chunk (positions
    L - C .. L - C + 15 and L - 16 .. L - 1) against the fp64 oracle.  Its
    inputs are the generated pool bytes (prefill writes no pool byte) of the
    sequence's blocks, gathered in table order with the tables of the
    oracle's own allocator, and the generated Q rows.  Returns the parity of
    those rows and the oracle's timing (its FLOP rate on them)."""
    from oracle import oracle as O
    import workloads
    BS = spec.block_size
    S = len(lens)
    ob = O.BlockAllocator(w.num_blocks, BS, w.max_blocks, w.free_order)
    workloads.allocate_context(ob, spec, lens)
    _, tables_o, _ = ob.export(np.arange(S, dtype=np.int64))
    host = OracleSample.host
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens))})
    checks, secs, flops, rows_done = [], 0.0, 0.0, 0
    for s in seqs:
        L, C = int(lens[s]), int(chunks[s])
        if C <= 0:
            continue
        n = -(-L // BS)
        idx = torch.from_numpy(tables_o[s, :n].astype(np.int64)).to(w.k_cache.device)
        kc = host(w.k_cache.index_select(0, idx), torch)
        vc = host(w.v_cache.index_select(0, idx), torch)
        table = np.arange(n, dtype=np.int32)[None, :]
        m = min(16, C)
        q0, q1 = int(qstart[s]), int(qstart[s + 1])
        for ctx, lo in ((L - C + m, q0), (L, q1 - m)):
            qr = np.ascontiguousarray(host(q[lo:lo + m], torch))
            t0 = time.perf_counter()
            ref, rlse = O.prefill_attention(qr, spec.q_dtype, kc, vc, spec.cache_dtype, table,
                                            np.array([ctx], dtype=np.int32),
                                            np.array([0, m], dtype=np.int32), spec.num_kv_heads, BS,
                                            float(np.float32(w.scale)), w.k_scale, w.v_scale,
                                            threads=threads)
            secs += time.perf_counter() - t0
            flops += 4.0 * spec.num_q_heads * spec.head_dim * sum(ctx - m + j + 1 for j in range(m))
            rows_done += m
            got = out[lo:lo + m].float().cpu().numpy()
            checks.append(compare(spec, got, lse[lo:lo + m].cpu().numpy().astype(np.float64), ref,
                                  rlse))
    worst = max(checks, key=lambda r: (r["max_err"], r["lse_rel_err"]))
    parity = dict(worst, lse_rel_err=max(r["lse_rel_err"] for r in checks),
                  ok=all(r["ok"] for r in checks), seqs=len(seqs), rows=rows_done,
                  how="first and last 16 rows of the chunks of the shortest and longest sequence")
    cpu = {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle", "seconds": round(secs, 2), "cpu_model": cpu_model(),
           "sample": f"{rows_done} query rows x {spec.num_q_heads} heads of {len(seqs)} sequences "
                     f"(first and last 16 chunk rows each), fp64 attention on {threads} threads"}
    return parity, cpu


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
    if not args.no_parity or not args.no_cpu_baseline:
        parity, cpu = prefill_oracle_leg(spec, w, blens, chunks, qstart, q, out, lse, torch,
                                         job_cores())
        if not args.no_parity:
            res["parity"] = parity
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)
    if not args.no_parity and not res["parity"]["ok"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
