"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: slot mapping and cache bytes bit-exact; attention within 1e-5 of each
row's largest |value| for fp32, 1e-2 max-abs for bf16 outputs, 3e-2 max-abs
for fp8 KV; the oracle consumes exactly the stored (rounded / quantized)
values the GPU consumed.  Every case prints its name before its GPU work.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_189_amd as pkv
import workloads
from oracle import oracle as O
from tests import gpu_case as G

pytestmark = pytest.mark.gpu

BS = 16
F32, BF16, E4M3 = workloads.F32, workloads.BF16, workloads.E4M3


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.lib()  # fail loudly if the library is missing
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def full_parity(c, seqs=None, label=""):
    """Cache write (bit-exact) and attention (tolerance) on the sampled seqs."""
    seqs = np.arange(len(c.lens)) if seqs is None else np.asarray(seqs)
    before = G.host_copy(c, seqs)
    G.log(f"[{label}] cache write + decode on GPU")
    G.run_cache_write(c)
    G.run_decode(c)
    torch.cuda.synchronize()
    after = G.host_copy(c, seqs)
    G.oracle_cache_write(c, before)
    assert np.array_equal(G.bits(before.k), G.bits(after.k)), f"{label}: K cache bytes differ"
    assert np.array_equal(G.bits(before.v), G.bits(after.v)), f"{label}: V cache bytes differ"
    ref, rlse, secs = G.oracle_decode(c, before)
    err = G.compare_out(c, seqs, ref, rlse, label)
    G.log(f"[{label}] max err {err:.3e} (oracle {secs:.2f}s)")
    return ref, rlse


def small_spec(index, base, S, Hq, Hkv, D, lens, cache=None):
    spec = G.spec_with(index, base=base, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, lengths=G.fixed_lengths(lens), pool_blocks=None,
                       prefix_tokens=0, max_model_len=0)
    if cache is not None:
        qd = F32 if cache == F32 else BF16
        spec = dataclasses.replace(spec, cache_dtype=cache, q_dtype=qd, out_dtype=qd)
    return spec


# ------------------------------------------------------------------- configs at small size
@pytest.mark.parametrize("part", [0, 16, 64])
def test_tiny_fp32_config(part):
    spec = workloads.SPECS[1]
    c = G.build(spec, partition_size=part)
    full_parity(c, label=f"tiny fp32 part={part}")


RAGGED = [1, 15, 16, 17, 100, 511, 512, 513, 1500, 2049]


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
@pytest.mark.parametrize("part", [0, 16, 48, 64])
def test_ragged_lengths(cache, part):
    base = {F32: 1, BF16: 2, E4M3: 4}[cache]
    spec = small_spec(200 + cache, base, len(RAGGED), 32, 8, 128, RAGGED, cache)
    c = G.build(spec, partition_size=part)
    full_parity(c, label=f"ragged dtype={cache} part={part}")


@pytest.mark.parametrize("cache", [BF16, E4M3])
@pytest.mark.parametrize("part", [0, 64])
def test_decode_sharp_softmax(cache, part):
    """Queries 8 times N(0, 1) (exact in bf16): scores spread over ~12 in log2
    units, so a few tokens carry each row and the lazy running max moves more
    often; output and lse against the oracle."""
    base = {BF16: 2, E4M3: 4}[cache]
    spec = small_spec(205 + cache, base, len(RAGGED), 32, 8, 128, RAGGED, cache)
    c = G.build(spec, partition_size=part)
    c.w.q.mul_(8.0)
    full_parity(c, label=f"sharp dtype={cache} part={part}")


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
def test_many_ranges_per_sequence(cache):
    """Enough blocks that every pass-1 range is busy: long sequences span many
    ranges and workgroups, short ones share a range; no partition cuts."""
    rng = np.random.default_rng(17 + cache)
    lens = np.concatenate([rng.integers(1, 200, 12), rng.integers(200, 3000, 12),
                           rng.integers(3000, 12000, 8)])
    base = {F32: 1, BF16: 2, E4M3: 4}[cache]
    spec = small_spec(210 + cache, base, len(lens), 32, 8, 128, lens, cache)
    c = G.build(spec, partition_size=0)
    full_parity(c, label=f"many ranges dtype={cache}")


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
def test_sequence_spanning_more_than_64_ranges(cache):
    """A 100K-token sequence spans about 250 pass-1 ranges per kv head, more
    than the merge wave has lanes: its rows take several rounds of 64 pieces;
    the short sequences beside it finish in pass 1 or merge in one round."""
    lens = [100_000, 1, 700, 3000, 16, 9000]
    base = {F32: 1, BF16: 2, E4M3: 4}[cache]
    spec = small_spec(220 + cache, base, len(lens), 32, 8, 128, lens, cache)
    c = G.build(spec, partition_size=0)
    full_parity(c, label=f"100K tokens dtype={cache}")


@pytest.mark.parametrize("cache", [BF16, E4M3])
@pytest.mark.parametrize("part", [16, 48, 96])
def test_partition_cuts_odd_and_even_tiles(cache, part):
    """Partitions of an odd (1, 3) and an even (6) number of 16-token tiles
    over sequences that span many ranges: the fp8 path takes two blocks per
    stage only where every cut falls between pairs, and the 16-token tile
    loop otherwise."""
    rng = np.random.default_rng(23 + cache + part)
    lens = np.concatenate([rng.integers(1, 200, 8), rng.integers(200, 3000, 8),
                           rng.integers(3000, 9000, 6)])
    base = {BF16: 2, E4M3: 4}[cache]
    spec = small_spec(230 + cache, base, len(lens), 32, 8, 128, lens, cache)
    c = G.build(spec, partition_size=part)
    full_parity(c, label=f"partition cuts dtype={cache} part={part}")


@pytest.mark.parametrize("cache", [BF16, E4M3])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("group", [1, 4, 16])
def test_many_cuts_per_wave(cache, D, group):
    """One-tile partitions over ~20 000 tiles: every pass-1 range holds about
    ten cuts, so each wave stages its partial states in LDS, writes them out
    whenever its staging area is full (every three cuts at D = 128, two at
    D = 64) and once more at its range's end; G = 1 and 4 leave staged rows
    that must not be written."""
    lens = [40_000, 39_001, 20_017, 41_000, 1, 17]
    base = {BF16: 2, E4M3: 4}[cache]
    spec = small_spec(260 + 10 * group + D // 64 + cache, base, len(lens), 2 * group, 2, D,
                      lens, cache)
    c = G.build(spec, partition_size=16)
    full_parity(c, label=f"many cuts dtype={cache} D={D} G={group}")


@pytest.mark.parametrize("cache", [BF16, E4M3])
@pytest.mark.parametrize("part", [0, 64])
def test_more_than_1024_sequences(cache, part):
    """A batch past the in-kernel plan's 1024 sequences: a one-workgroup plan
    kernel runs before pass 1, which then reads the plan from the workspace."""
    rng = np.random.default_rng(41 + cache + part)
    lens = rng.integers(1, 400, 1100)
    lens[[5, 600, 1099]] = [2000, 3000, 1]
    base = {BF16: 2, E4M3: 4}[cache]
    spec = small_spec(250 + cache + part, base, len(lens), 16, 4, 128, lens, cache)
    c = G.build(spec, partition_size=part)
    seqs = np.unique(np.concatenate([[0, 5, 600, 1023, 1024, 1099],
                                     rng.choice(len(lens), 40, replace=False)]))
    full_parity(c, seqs, label=f"1100 seqs dtype={cache} part={part}")


@pytest.mark.parametrize("cache", [BF16, E4M3])
def test_short_contexts_every_row(cache):
    """4096 sequences of 1 to 40 tokens, every output row against the oracle:
    attention over a few tokens gives outputs as large as single V values,
    where the bf16 roundings of P and of the output leave the least room
    under the output bar."""
    rng = np.random.default_rng(53 + cache)
    lens = rng.integers(1, 41, 4096)
    base = {BF16: 2, E4M3: 4}[cache]
    spec = small_spec(270 + cache, base, len(lens), 32, 8, 128, lens, cache)
    c = G.build(spec, partition_size=0)
    full_parity(c, label=f"4096 short sequences dtype={cache}")


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8, 16])
def test_gqa_headdim_dtype_variants(cache, D, group):
    Hkv = 2
    lens = [3, 40, 257, 700]
    spec = small_spec(300 + 10 * group + D // 64 + cache, 2, len(lens), Hkv * group, Hkv, D, lens,
                      cache)
    c = G.build(spec, partition_size=256)
    full_parity(c, label=f"gqa G={group} D={D} dtype={cache}")


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_decode_negative_and_zero_scale(cache, scale):
    """Any finite softmax scale: a negative one flips which keys dominate,
    zero gives uniform weights over the context (with partition cuts, so the
    merge sees the same scale's states)."""
    lens = [1, 17, 300, 2049]
    base = {F32: 1, BF16: 2, E4M3: 4}[cache]
    spec = small_spec(270 + cache, base, len(lens), 16, 4, 128, lens, cache)
    c = G.build(spec, partition_size=64)
    c.w.scale = scale
    c.params.scale = scale
    full_parity(c, label=f"decode scale {scale} dtype={cache}")


def test_empty_sequence_row():
    spec = small_spec(400, 2, 3, 8, 2, 128, [33, 5, 600])
    c = G.build(spec, partition_size=64)
    c.d_lens[1] = 0
    G.log("[empty] decode with one zero-length sequence")
    G.run_cache_write(c)
    G.run_decode(c)
    torch.cuda.synchronize()
    out = c.out.float().cpu().numpy()
    lse = c.lse.cpu().numpy()
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(out[[0, 2]]))


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
@pytest.mark.parametrize("part", [0, 64])
def test_all_sequences_empty(cache, part):
    """No sequence has a token: pass 1 has no blocks to cut into ranges, and
    every row is the empty row (zeros, lse = -inf)."""
    base = {F32: 1, BF16: 2, E4M3: 4}[cache]
    spec = small_spec(410 + cache, base, 3, 8, 2, 128, [33, 5, 600], cache)
    c = G.build(spec, partition_size=part)
    c.d_lens.zero_()
    c.out.fill_(7.0)
    G.log(f"[all empty] dtype={cache} part={part}")
    G.run_decode(c)
    torch.cuda.synchronize()
    assert np.all(c.out.float().cpu().numpy() == 0)
    assert np.all(np.isneginf(c.lse.cpu().numpy()))


@pytest.mark.parametrize("cache", [BF16, E4M3])
@pytest.mark.parametrize("part", [0, 64])
def test_decode_without_lse_output(cache, part):
    """lse_out is optional: without it the output is bit-identical."""
    base = {BF16: 2, E4M3: 4}[cache]
    spec = small_spec(420 + cache, base, len(RAGGED), 32, 8, 128, RAGGED, cache)
    c = G.build(spec, partition_size=part)
    G.log(f"[no lse] dtype={cache} part={part}")
    G.run_cache_write(c)
    G.run_decode(c)
    with_lse = c.out.clone()
    c.out.fill_(7.0)
    w = c.w
    pkv.pkv_decode_attention(c.params, c.out, w.q, w.k_cache, w.v_cache, c.d_tables, c.d_lens,
                             c.workspace, None)
    torch.cuda.synchronize()
    assert torch.equal(c.out.view(torch.int16), with_lse.view(torch.int16))


def test_passes_separately_equal_composed():
    spec = small_spec(401, 2, 4, 16, 4, 128, [700, 1200, 35, 2000])
    c = G.build(spec, partition_size=128)
    G.log("[two passes] composed call")
    G.run_cache_write(c)
    G.run_decode(c)
    torch.cuda.synchronize()
    o1, l1 = c.out.clone(), c.lse.clone()
    c.out.fill_(float("nan"))
    c.lse.fill_(float("nan"))
    w = c.w
    G.log("[two passes] partitions then merge")
    pkv.pkv_decode_attention_partitions(c.params, c.out, w.q, w.k_cache, w.v_cache, c.d_tables,
                                        c.d_lens, c.workspace, c.lse)
    pkv.pkv_decode_attention_merge(c.params, c.out, c.d_lens, c.workspace, c.lse)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), c.out.view(torch.int16)) and torch.equal(l1, c.lse)


# ------------------------------------------------------------------- invariants of paging
@pytest.mark.parametrize("cache", [BF16, E4M3])
def test_block_relabel_bit_identical(cache):
    lens = [70, 300, 1025, 16]
    spec = small_spec(500 + cache, 2, len(lens), 16, 2, 128, lens, cache)
    c = G.build(spec, partition_size=256)
    G.log(f"[relabel dtype={cache}] original placement")
    G.run_cache_write(c)
    G.run_decode(c)
    torch.cuda.synchronize()
    o1, l1 = c.out.clone(), c.lse.clone()
    nb = c.w.num_blocks
    pi = torch.from_numpy(np.random.default_rng(9).permutation(nb)).to(c.out.device)
    k2 = torch.empty_like(c.w.k_cache)
    v2 = torch.empty_like(c.w.v_cache)
    k2[pi] = c.w.k_cache
    v2[pi] = c.w.v_cache
    t2 = c.d_tables.clone()
    m = t2 >= 0
    t2[m] = pi[t2[m].long()].int()
    G.log(f"[relabel dtype={cache}] permuted placement")
    pkv.pkv_decode_attention(c.params, c.out, c.w.q, k2, v2, t2, c.d_lens, c.workspace, c.lse)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), c.out.view(torch.int16))
    assert torch.equal(l1, c.lse)


def test_shared_prefix_equals_copied_bit_identical():
    spec = dataclasses.replace(workloads.SPECS[3], index=600, num_seqs=8)
    lens = workloads.lengths(spec, 8)
    c = G.build(spec, lens=lens, partition_size=512)
    G.log("[prefix] shared prefix blocks")
    G.run_cache_write(c)
    G.run_decode(c)
    torch.cuda.synchronize()
    o1, l1 = c.out.clone(), c.lse.clone()
    # copies of the 64 prefix blocks for sequences 1.., appended past the pool
    pre = spec.prefix_tokens // BS
    S = len(lens)
    w = c.w
    shared = torch.from_numpy(c.tables[0, :pre].astype(np.int64)).to(w.k_cache.device)
    k2 = torch.cat([w.k_cache] + [w.k_cache[shared]] * (S - 1))
    v2 = torch.cat([w.v_cache] + [w.v_cache[shared]] * (S - 1))
    t2 = c.tables.copy()
    for s in range(1, S):
        t2[s, :pre] = w.num_blocks + (s - 1) * pre + np.arange(pre)
    p2 = pkv.make_decode_params(w.q, k2, c.d_tables, c.params.max_context_len, w.scale,
                                w.k_scale, w.v_scale, c.out.dtype, 512)
    G.log("[prefix] copied prefix blocks")
    pkv.pkv_decode_attention(p2, c.out, w.q, k2, v2, torch.from_numpy(t2).to(c.out.device),
                             c.d_lens, c.workspace, c.lse)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), c.out.view(torch.int16))
    assert torch.equal(l1, c.lse)


def test_constant_v_gives_constant_output():
    """V == 1 in every used block: the output is exactly 1 (the weights that
    multiply V are the ones the normaliser sums).  Unused blocks keep NaN."""
    lens = [1, 17, 900, 4000]
    spec = small_spec(700, 2, len(lens), 32, 8, 128, lens)
    c = G.build(spec, partition_size=512)
    G.run_cache_write(c)
    used = np.unique(np.concatenate([c.tables[s, :-(-int(L) // BS)] for s, L in enumerate(c.lens)]))
    c.w.v_cache[torch.from_numpy(used).to(c.out.device)] = 1.0
    G.log("[V==1] decode")
    G.run_decode(c)
    torch.cuda.synchronize()
    assert torch.all(c.out.float() == 1.0)


# ------------------------------------------------------------------- cache write variants
@pytest.mark.parametrize("src,dst", [(F32, F32), (BF16, BF16), (F32, BF16), (BF16, E4M3),
                                     (F32, E4M3)])
@pytest.mark.parametrize("D", [64, 128])
def test_cache_write_bit_exact(src, dst, D):
    rng = np.random.default_rng(800 + 10 * src + dst)
    T, H, nb = 37, 4, 20
    X = 16 // workloads.ELEM_BYTES[dst]
    sdt = torch.float32 if src == F32 else torch.bfloat16
    kn = (torch.from_numpy(rng.standard_normal((T, H, D)).astype(np.float32)) * 3).to(sdt).cuda()
    vn = (torch.from_numpy(rng.standard_normal((T, H, D)).astype(np.float32)) * 3).to(sdt).cuda()
    kn[0, 0, :4] = torch.tensor([1e6, -1e6, 3e-9, 0.0])  # saturation, subnormal, zero
    slots = rng.choice(nb * BS, size=T, replace=False).astype(np.int64)
    slots[3] = -1
    slots[5] = nb * BS + 7  # out of range: skipped
    kshape, vshape = workloads.pool_shapes(nb, H, D, dst)
    sto = workloads.TORCH_STORAGE[dst]
    kc = torch.zeros(kshape, dtype=sto, device="cuda")
    vc = torch.zeros(vshape, dtype=sto, device="cuda")
    ks, vs = (0.0137, 0.0291) if dst == E4M3 else (1.0, 1.0)
    G.log(f"[cache write {src}->{dst} D={D}]")
    pkv.pkv_reshape_and_cache(kn, vn, kc, vc, torch.from_numpy(slots).cuda(), ks, vs)
    torch.cuda.synchronize()
    ko = np.zeros(kshape, dtype=G.np_storage(kc[:1]).dtype)
    vo = np.zeros(vshape, dtype=ko.dtype)
    sl = slots.copy()
    sl[5] = -1  # the oracle would reject it; the library skips it
    O.reshape_and_cache(G.np_storage(kn), G.np_storage(vn), src, ko, vo, dst, sl, BS, ks, vs)
    assert np.array_equal(G.bits(G.np_storage(kc)), G.bits(ko))
    assert np.array_equal(G.bits(G.np_storage(vc)), G.bits(vo))


# ------------------------------------------------------------------- full sizes, sampled
@pytest.mark.parametrize("index,k,part", [(2, 64, None), (3, 32, None), (4, 32, None),
                                          (4, 12, 48), (5, 8, None)])
def test_full_size_config_sampled(index, k, part):
    """Each workload at full size in the launch configuration the benchmark
    times.  The sample is chosen by the CPU model of the work division
    (tests/test_work_division.py) at this device's range count, so that it
    holds sequences meeting each case of it: pieces folded between waves
    (publish, absorb), pairs finished in pass 1 and merged in pass 2, more
    than 64 pieces in one merge, range boundaries at odd tiles (the fp8
    block-pair stages mask half a pair there), partition cuts at range
    starts.  The 70B fp8 workload is also run with 48-token partitions, an
    odd number of tiles, which sends its segments to the 16-token tile loop."""
    from tests import test_work_division as WD
    spec = workloads.SPECS[index]
    G.log(f"[config {index} part={part}] building {spec.name}")
    c = G.build(spec, partition_size=part)
    R = pkv.pkv_decode_num_ranges(c.params)
    pb = pkv.pkv_decode_partition_size(c.params) // BS
    nblocks = [-(-int(L) // BS) for L in c.lens]
    flags = WD.case_flags(nblocks, spec.num_kv_heads, R, pb)
    cases = WD.FULL_SIZE_CASES.get((index, pb), ())
    seqs = WD.targeted_sample(flags, c.lens, k, cases, index)
    for case in cases:
        assert any(case in flags[int(s)] for s in seqs), f"no sampled sequence meets {case} (R={R})"
    G.log(f"[config {index} part={part}] R={R}, {len(seqs)} seqs covering {sorted(cases)}")
    full_parity(c, seqs, label=f"config {index} part={part} full size, {len(seqs)} sampled seqs")
    del c


# ------------------------------------------------------------------- copy-on-write and multi-token append
def _to_device(a: np.ndarray, dtype: int, device="cuda") -> torch.Tensor:
    if dtype == BF16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def _rand_storage(gen, shape, dtype, scale=1.0):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if dtype == F32:
        return x.numpy()
    if dtype == BF16:
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return (x.to(torch.bfloat16).float() / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
@pytest.mark.parametrize("D", [64, 128])
def test_copy_blocks_bit_exact(cache, D):
    gen = torch.Generator().manual_seed(70 + cache + D)
    nb, Hkv = 40, 4
    ks, vs = workloads.pool_shapes(nb, Hkv, D, cache)
    k = _rand_storage(gen, ks, cache, 0.01)
    v = _rand_storage(gen, vs, cache, 0.01)
    src = np.array([3, 7, 7, 0, 39, 12], dtype=np.int32)
    dst = np.array([5, 8, 9, 1, 38, 13], dtype=np.int32)
    dk, dv = _to_device(k, cache), _to_device(v, cache)
    G.log(f"[copy blocks dtype={cache} D={D}]")
    pkv.pkv_copy_blocks(dk, dv, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    O.copy_blocks(k, v, src, dst)
    assert np.array_equal(G.bits(G.np_storage(dk)), G.bits(k))
    assert np.array_equal(G.bits(G.np_storage(dv)), G.bits(v))


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
def test_cow_fork_diverge_and_multi_token_append(cache):
    """Multi-token append (one cache write of 183 tokens for three
    sequences), forks at mid-block and block-aligned positions, then a
    copy-on-write batch: slots and copy pairs equal the oracle allocator's,
    both pools equal the oracle's bit for bit after the device copy and
    cache write, and decode of all seven sequences matches the oracle."""
    gen = torch.Generator().manual_seed(80 + cache)
    Hq, Hkv, D, nb, mb = 16, 4, 128, 96, 24
    qd = F32 if cache == F32 else BF16
    ksc, vsc = (1.0, 1.0) if cache != E4M3 else (0.011, 0.013)
    order = np.random.default_rng(81 + cache).permutation(nb).astype(np.int32)
    bm = pkv.BlockManager(nb, BS, mb, order)
    ob = O.BlockAllocator(nb, BS, mb, order)
    ks, vs = workloads.pool_shapes(nb, Hkv, D, cache)
    k = np.zeros(ks, dtype=O.NP_STORAGE[cache])
    v = np.zeros(vs, dtype=O.NP_STORAGE[cache])
    dk, dv = _to_device(k, cache), _to_device(v, cache)

    def write(ids, with_cow):
        if with_cow:
            r1, s1, a1, b1 = bm.append_slots_cow(ids)
            r2, s2, a2, b2 = ob.append_slots_cow(ids)
            assert r1 == r2 == 0 and np.array_equal(a1, a2) and np.array_equal(b1, b2)
            if len(a1):
                pkv.pkv_copy_blocks(dk, dv, torch.from_numpy(a1).cuda(), torch.from_numpy(b1).cuda())
                O.copy_blocks(k, v, a2, b2)
        else:
            r1, s1 = bm.append_slots(ids)
            r2, s2 = ob.append_slots(ids)
            assert r1 == r2 == 0
        assert np.array_equal(s1, s2)
        kn = _rand_storage(gen, (len(ids), Hkv, D), qd)
        vn = _rand_storage(gen, (len(ids), Hkv, D), qd)
        pkv.pkv_reshape_and_cache(_to_device(kn, qd), _to_device(vn, qd), dk, dv,
                                  torch.from_numpy(s1).cuda(), ksc, vsc)
        O.reshape_and_cache(kn, vn, qd, k, v, cache, s2, BS, ksc, vsc)
        return len(a1) if with_cow else 0

    for s in range(3):
        assert bm.add_seq(s) == 0 and ob.add_seq(s) == 0
    G.log(f"[cow dtype={cache}] multi-token append")
    write(np.array([0] * 37 + [1] * 16 + [2] * 130, dtype=np.int64), False)
    for parent, child in ((0, 3), (0, 4), (2, 5), (1, 6)):
        assert bm.fork_seq(parent, child) == 0 and ob.fork_seq(parent, child) == 0
    G.log(f"[cow dtype={cache}] copy-on-write batch")
    ids = np.array([3] * 5 + [0] * 3 + [4] * 20 + [5] + [2] * 2 + [6] * 17 + [1], dtype=np.int64)
    copies = write(ids, True)
    # 3 then 0 copy the shared block 2 (4, its last holder, keeps it); 5 copies
    # block 8 of 2; 6 and 1 sit at block boundaries
    assert copies == 3
    torch.cuda.synchronize()
    assert np.array_equal(G.bits(G.np_storage(dk)), G.bits(k)), "K pool differs"
    assert np.array_equal(G.bits(G.np_storage(dv)), G.bits(v)), "V pool differs"

    seqs = np.arange(7, dtype=np.int64)
    _, tables, lens = bm.export(seqs)
    q = _rand_storage(gen, (7, Hq, D), qd)
    dq = _to_device(q, qd)
    out_t = torch.float32 if cache == F32 else torch.bfloat16
    d_tables = torch.from_numpy(tables).cuda()
    params = pkv.make_decode_params(dq, dk, d_tables, mb * BS, 1 / math.sqrt(D), ksc, vsc, out_t, 0)
    ws = torch.empty(pkv.pkv_decode_workspace_bytes(params), dtype=torch.uint8, device="cuda")
    out = torch.full((7, Hq, D), float("nan"), dtype=out_t, device="cuda")
    lse = torch.full((7, Hq), float("nan"), dtype=torch.float32, device="cuda")
    G.log(f"[cow dtype={cache}] decode")
    pkv.pkv_decode_attention(params, out, dq, dk, dv, d_tables, torch.from_numpy(lens).cuda(), ws, lse)
    torch.cuda.synchronize()
    ref, rlse = O.decode_attention(q, qd, k, v, cache, tables, lens, Hkv, BS,
                                   float(np.float32(1 / math.sqrt(D))), ksc, vsc)
    got = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    if cache == F32:
        assert np.all(err <= 1e-5 * np.abs(ref).max(axis=2, keepdims=True))
    else:
        assert np.all(err <= G.out_bound(ref, cache)), err.max()
    assert np.allclose(lse.cpu().numpy(), rlse, rtol=1e-4, atol=1e-4)


# ------------------------------------------------------------------- 32-token blocks
@pytest.mark.parametrize("cache,D", [(F32, 128), (BF16, 128), (BF16, 64), (E4M3, 128), (E4M3, 64)])
@pytest.mark.parametrize("part", [0, 64])
def test_block_size_32(cache, D, part):
    """32-token blocks: one multi-token append + cache write (bit-exact
    against the oracle's cache write) and decode against the oracle, for
    lengths around the block and tile boundaries."""
    BS32 = 32
    gen = torch.Generator().manual_seed(90 + cache + D + part)
    Hq, Hkv = 16, 4
    lens = np.array([1, 15, 16, 17, 31, 32, 33, 100, 1000, 3000], dtype=np.int64)
    nb = int(sum(-(-lens // BS32))) + 7
    mb = int(-(-lens.max() // BS32))
    qd = F32 if cache == F32 else BF16
    ksc, vsc = (1.0, 1.0) if cache != E4M3 else (0.011, 0.013)
    order = np.random.default_rng(91 + cache).permutation(nb).astype(np.int32)
    bm = pkv.BlockManager(nb, BS32, mb, order)
    ob = O.BlockAllocator(nb, BS32, mb, order)
    ks, vs = workloads.pool_shapes(nb, Hkv, D, cache, BS32)
    k = _rand_storage(gen, ks, cache, ksc)  # unused slots keep random values
    v = _rand_storage(gen, vs, cache, vsc)
    dk, dv = _to_device(k, cache), _to_device(v, cache)
    S = len(lens)
    for s in range(S):
        assert bm.add_seq(s) == 0 and ob.add_seq(s) == 0
    ids = np.repeat(np.arange(S, dtype=np.int64), lens)
    r1, s1 = bm.append_slots(ids)
    r2, s2 = ob.append_slots(ids)
    assert r1 == r2 == 0 and np.array_equal(s1, s2)
    kn = _rand_storage(gen, (len(ids), Hkv, D), qd)
    vn = _rand_storage(gen, (len(ids), Hkv, D), qd)
    G.log(f"[block 32 dtype={cache} D={D} part={part}] cache write of {len(ids)} tokens")
    pkv.pkv_reshape_and_cache(_to_device(kn, qd), _to_device(vn, qd), dk, dv,
                              torch.from_numpy(s1).cuda(), ksc, vsc)
    O.reshape_and_cache(kn, vn, qd, k, v, cache, s2, BS32, ksc, vsc)
    torch.cuda.synchronize()
    assert np.array_equal(G.bits(G.np_storage(dk)), G.bits(k)), "K pool differs"
    assert np.array_equal(G.bits(G.np_storage(dv)), G.bits(v)), "V pool differs"
    _, tables, blens = bm.export(np.arange(S, dtype=np.int64))
    q = _rand_storage(gen, (S, Hq, D), qd)
    dq = _to_device(q, qd)
    out_t = torch.float32 if cache == F32 else torch.bfloat16
    d_tables = torch.from_numpy(tables).cuda()
    params = pkv.make_decode_params(dq, dk, d_tables, mb * BS32, 1 / math.sqrt(D), ksc, vsc, out_t,
                                    part)
    assert params.block_size == BS32
    ws = torch.empty(pkv.pkv_decode_workspace_bytes(params), dtype=torch.uint8, device="cuda")
    out = torch.full((S, Hq, D), float("nan"), dtype=out_t, device="cuda")
    lse = torch.full((S, Hq), float("nan"), dtype=torch.float32, device="cuda")
    G.log(f"[block 32 dtype={cache} D={D} part={part}] decode")
    pkv.pkv_decode_attention(params, out, dq, dk, dv, d_tables, torch.from_numpy(blens).cuda(), ws,
                             lse)
    torch.cuda.synchronize()
    ref, rlse = O.decode_attention(q, qd, k, v, cache, tables, blens, Hkv, BS32,
                                   float(np.float32(1 / math.sqrt(D))), ksc, vsc)
    got = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    if cache == F32:
        assert np.all(err <= 1e-5 * np.abs(ref).max(axis=2, keepdims=True))
    else:
        assert np.all(err <= G.out_bound(ref, cache)), err.max()
    assert np.allclose(lse.cpu().numpy(), rlse, rtol=1e-4, atol=1e-4)


# ------------------------------------------------------------------- chunked prefill
def _paged_batch(gen, cache, D, Hkv, lens, bs=16, seed=0):
    """Pools filled through one multi-token append + cache write on both sides
    (bit-exact check included); returns device and host views."""
    lens = np.asarray(lens, dtype=np.int64)
    nb = int(sum(-(-lens // bs))) + 5
    mb = int(max(1, -(-lens.max() // bs)))
    qd = F32 if cache == F32 else BF16
    ksc, vsc = (1.0, 1.0) if cache != E4M3 else (0.011, 0.013)
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    bm = pkv.BlockManager(nb, bs, mb, order)
    ob = O.BlockAllocator(nb, bs, mb, order)
    ks, vs = workloads.pool_shapes(nb, Hkv, D, cache, bs)
    k = _rand_storage(gen, ks, cache, ksc)
    v = _rand_storage(gen, vs, cache, vsc)
    dk, dv = _to_device(k, cache), _to_device(v, cache)
    S = len(lens)
    for s in range(S):
        assert bm.add_seq(s) == 0 and ob.add_seq(s) == 0
    ids = np.repeat(np.arange(S, dtype=np.int64), lens)
    r1, s1 = bm.append_slots(ids)
    r2, s2 = ob.append_slots(ids)
    assert r1 == r2 == 0 and np.array_equal(s1, s2)
    kn = _rand_storage(gen, (len(ids), Hkv, D), qd)
    vn = _rand_storage(gen, (len(ids), Hkv, D), qd)
    pkv.pkv_reshape_and_cache(_to_device(kn, qd), _to_device(vn, qd), dk, dv,
                              torch.from_numpy(s1).cuda(), ksc, vsc)
    O.reshape_and_cache(kn, vn, qd, k, v, cache, s2, bs, ksc, vsc)
    torch.cuda.synchronize()
    assert np.array_equal(G.bits(G.np_storage(dk)), G.bits(k)), "K pool differs"
    _, tables, blens = bm.export(np.arange(S, dtype=np.int64))
    return dict(k=k, v=v, dk=dk, dv=dv, tables=tables, lens=blens, mb=mb, qd=qd, ksc=ksc,
                vsc=vsc, bs=bs)


def _prefill_case(cache, D, grp, lens, chunks, bs=16, Hkv=2, label="", scale=None, q_fn=None):
    gen = torch.Generator().manual_seed(1000 + 97 * cache + D + 7 * grp + bs)
    b = _paged_batch(gen, cache, D, Hkv, lens, bs, seed=grp + D)
    Hq = Hkv * grp
    qstart = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    R = int(qstart[-1])
    q = _rand_storage(gen, (R, Hq, D), b["qd"])
    if q_fn is not None:  # reshape the query values (fp32), then store them as the query dtype
        qf = q.astype(np.float32) if b["qd"] == F32 else (q.astype(np.uint32) << 16).view(np.float32)
        qf = torch.from_numpy(np.ascontiguousarray(q_fn(qf), dtype=np.float32))
        q = qf.numpy() if b["qd"] == F32 else qf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    dq = _to_device(q, b["qd"])
    out_t = torch.float32 if cache == F32 else torch.bfloat16
    d_tables = torch.from_numpy(b["tables"]).cuda()
    scale = 1 / math.sqrt(D) if scale is None else scale
    p = pkv.make_prefill_params(dq, b["dk"], d_tables, len(lens), b["mb"] * bs, scale, b["ksc"],
                                b["vsc"], out_t)
    out = torch.full((R, Hq, D), float("nan"), dtype=out_t, device="cuda")
    lse = torch.full((R, Hq), float("nan"), dtype=torch.float32, device="cuda")
    G.log(f"[prefill {label}] dtype={cache} D={D} G={grp} bs={bs} rows={R}")
    pkv.pkv_prefill_attention(p, out, dq, b["dk"], b["dv"], d_tables,
                              torch.from_numpy(b["lens"]).cuda(), torch.from_numpy(qstart).cuda(),
                              lse)
    torch.cuda.synchronize()
    ref, rlse = O.prefill_attention(q, b["qd"], b["k"], b["v"], cache, b["tables"], b["lens"],
                                    qstart, Hkv, bs, float(np.float32(scale)), b["ksc"], b["vsc"])
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    err = np.abs(got - ref)
    if cache == F32:
        bound = 1e-5 * np.abs(ref).max(axis=2, keepdims=True)
        assert np.all(err <= np.maximum(bound, 1e-30)), f"{label}: fp32 err"
    else:
        assert np.all(err <= G.out_bound(ref, cache)), f"{label}: max abs err {err.max()}"
    gl = lse.cpu().numpy()
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(gl)), f"{label}: lse finiteness"
    lerr = np.abs(gl[fin] - rlse[fin]) / (1e-4 + 1e-4 * np.abs(rlse[fin])) if fin.any() else np.zeros(1)
    G.log(f"[prefill {label}] max abs err {err.max():.3e}, lse err / bar {lerr.max():.3f}")
    assert lerr.max() <= 1.0, f"{label}: lse"
    return got, ref


PF_LENS = [1, 17, 100, 700, 2049, 3000]
PF_CHUNKS = [1, 17, 37, 300, 1, 160]


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("group", [1, 3, 4, 8, 16])
def test_prefill_mixed_chunks(cache, D, group):
    _prefill_case(cache, D, group, PF_LENS, PF_CHUNKS, label=f"mixed")


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_block_size_32(cache, D):
    _prefill_case(cache, D, 4, PF_LENS, PF_CHUNKS, bs=32, label="bs32")


@pytest.mark.parametrize("cache", [F32, BF16])
@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_prefill_negative_and_zero_scale(cache, scale):
    """The softmax scale is any finite number: a negative one flips which
    keys dominate, zero gives uniform weights over the causal window."""
    _prefill_case(cache, 64, 4, [40, 300, 77], [40, 33, 9], label=f"scale {scale}", scale=scale)


def test_prefill_full_sequences_and_overlong_chunks():
    """C = L (the whole sequence is the chunk) and C > L (leading rows see
    nothing and are written as zeros with lse = -inf)."""
    got, ref = _prefill_case(BF16, 128, 4, [1000, 3, 64], [1000, 5, 64], label="full/overlong")
    assert np.all(got[1000:1002] == 0)



@pytest.mark.parametrize("cache", [BF16, E4M3])
def test_prefill_empty_chunks_and_contexts(cache):
    """Sequences with no chunk (C = 0: no workgroup item), one with an empty
    context as well, beside chunks that end inside a 32-token step and one
    spanning whole steps; the other rows must be untouched by the empty ones."""
    _prefill_case(cache, 128, 4, [0, 5, 300, 64, 33], [0, 0, 17, 64, 0], label="empty chunks")

@pytest.mark.parametrize("cache", [BF16, E4M3])
def test_prefill_max_sequences(cache):
    """The largest batch a prefill call takes, 1024 sequences: every
    workgroup builds the item prefix sums over four 256-sequence rounds and
    finds its sequence among all of them.  Short ragged contexts, chunks from
    none to the whole context."""
    rng = np.random.default_rng(31 + cache)
    lens = rng.integers(0, 80, 1024)
    chunks = np.minimum(lens, rng.integers(0, 48, 1024))
    _prefill_case(cache, 128, 4, lens, chunks, label="1024 sequences")


@pytest.mark.parametrize("cache", [BF16, E4M3])
@pytest.mark.parametrize("gain", [4.0, 8.0])
def test_prefill_sharp_softmax(cache, gain):
    """Queries 4 and 8 times N(0, 1): scores with a spread of 6 to 12 in log2
    units, so a few tokens carry most of each row's weight and a small score
    error moves the output the most (with an fp8 cache the scores take q as
    two E4M3 terms)."""
    _prefill_case(cache, 128, 4, PF_LENS, PF_CHUNKS, label=f"sharp x{gain}",
                  q_fn=lambda q: q * gain)


@pytest.mark.parametrize("cache", [BF16, E4M3])
def test_prefill_query_rows_of_any_size(cache):
    """Query rows scaled by 2^-24 .. 2^6 and one dim per row 64 times the
    others: the fp8 score path scales each row by its own power of two."""
    def q_fn(q):
        rng = np.random.default_rng(17)
        R, Hq, D = q.shape
        q = q * np.exp2(rng.integers(-24, 7, size=(R, Hq, 1))).astype(np.float32) / 64
        d = rng.integers(0, D, size=(R, Hq, 1))
        np.put_along_axis(q, d, np.take_along_axis(q, d, 2) * 64, 2)
        return q
    _prefill_case(cache, 128, 4, PF_LENS, PF_CHUNKS, label="row sizes", q_fn=q_fn)


# ------------------------------------------------------------------- automatic prefix caching
def test_prefix_cache_reuses_cached_kv_end_to_end():
    """K and V are a fixed function of (token id, position), as a model's
    would be of the token prefix.  Sequence A writes its prompt; after A is
    freed, B shares A's first 40 tokens and C repeats A's prompt: they get
    A's cached blocks back and write only their remaining tokens.  Tables
    equal the oracle allocator's, and decode of B and C over the reused
    blocks equals the oracle over pools where every token was written."""
    from oracle.prefix_cache import PrefixCacheAllocator
    gen = torch.Generator().manual_seed(4242)
    Hq, Hkv, D, bs, nb, mb = 16, 4, 128, 16, 64, 16
    vocab, maxpos = 60, mb * bs
    kv_k = _rand_storage(gen, (vocab, maxpos, Hkv, D), BF16)   # K of token id at position
    kv_v = _rand_storage(gen, (vocab, maxpos, Hkv, D), BF16)
    order = np.random.default_rng(5).permutation(nb).astype(np.int32)
    bm = pkv.BlockManager(nb, bs, mb, order)
    ob = PrefixCacheAllocator(nb, bs, mb, order)
    ks, vs = workloads.pool_shapes(nb, Hkv, D, BF16, bs)
    k_all = np.zeros(ks, np.uint16)   # oracle pools: every token written
    v_all = np.zeros(vs, np.uint16)
    dk, dv = _to_device(k_all.copy(), BF16), _to_device(v_all.copy(), BF16)
    rng = np.random.default_rng(6)
    prompt_a = list(rng.integers(0, vocab, 70))
    prompts = {0: prompt_a, 1: prompt_a[:40] + list(rng.integers(0, vocab, 30)), 2: list(prompt_a)}

    def admit(sid):
        toks = prompts[sid]
        r1, s1, c1 = bm.add_seq_prompt(sid, toks)
        r2, s2, c2 = ob.add_seq_prompt(sid, toks)
        assert r1 == r2 == 0 and list(s1) == s2 and c1 == c2
        pos = np.arange(len(toks))
        tk = np.asarray(toks)
        kn, vn = kv_k[tk, pos], kv_v[tk, pos]
        new = slice(c1, len(toks))   # the device gets only the tokens not cached
        pkv.pkv_reshape_and_cache(_to_device(np.ascontiguousarray(kn[new]), BF16),
                                  _to_device(np.ascontiguousarray(vn[new]), BF16), dk, dv,
                                  torch.from_numpy(np.ascontiguousarray(s1[new])).cuda())
        O.reshape_and_cache(np.ascontiguousarray(kn), np.ascontiguousarray(vn), BF16, k_all,
                            v_all, BF16, np.asarray(s1, np.int64), bs)
        return c1

    G.log("[prefix cache] admit A, free it, admit B and C")
    assert admit(0) == 0
    assert bm.free_seq(0) == ob.free_seq(0) == 0
    assert admit(1) == 32            # two full blocks of the shared 40 tokens
    assert admit(2) == 64            # four full blocks; the fifth holds the last token
    seqs = np.array([1, 2], dtype=np.int64)
    _, tables, lens = bm.export(seqs)
    for i, sid in enumerate(seqs):
        t, L = ob.table(int(sid))
        assert list(tables[i][: len(t)]) == t and lens[i] == L
    q = _rand_storage(gen, (2, Hq, D), BF16)
    dq = _to_device(q, BF16)
    d_tables = torch.from_numpy(tables).cuda()
    params = pkv.make_decode_params(dq, dk, d_tables, mb * bs, 1 / math.sqrt(D), 1.0, 1.0,
                                    torch.bfloat16, 0)
    ws = torch.empty(pkv.pkv_decode_workspace_bytes(params), dtype=torch.uint8, device="cuda")
    out = torch.empty((2, Hq, D), dtype=torch.bfloat16, device="cuda")
    pkv.pkv_decode_attention(params, out, dq, dk, dv, d_tables, torch.from_numpy(lens).cuda(), ws)
    torch.cuda.synchronize()
    ref, _ = O.decode_attention(q, BF16, k_all, v_all, BF16, tables, lens, Hkv, bs,
                                float(np.float32(1 / math.sqrt(D))))
    err = np.abs(out.float().cpu().numpy() - ref)
    assert np.all(err <= G.out_bound(ref, BF16)), err.max()


# ------------------------------------------------------------------- decode append (cache + tables)
@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
def test_append_decode_tokens_sets_tables_and_cache(cache):
    """pkv_append_decode_tokens: the cache bytes equal the oracle's cache
    write, the device table entry of each new position equals the host block
    manager's (poisoned beforehand, so a missed write shows), a skipped slot
    leaves its row alone, and decode over the updated tables matches the oracle."""
    lens = [1, 16, 17, 33, 100, 257, 1000, 1025]
    spec = small_spec(960 + cache, 2, len(lens), 16, 4, 128, lens, cache)
    c = G.build(spec)
    S = len(c.lens)
    seqs = np.arange(S)
    before = G.host_copy(c, seqs)
    pos = c.lens.astype(np.int64) - 1
    col = torch.from_numpy(pos // BS).cuda()
    rows = torch.arange(S, device="cuda")
    c.d_tables[rows, col] = -7
    skip = 3
    slots = c.d_slots.clone()
    slots[skip] = -1
    G.log(f"[append decode tokens dtype={cache}] skipped slot of sequence {skip}")
    w = c.w
    pkv.pkv_append_decode_tokens(w.k_new, w.v_new, w.k_cache, w.v_cache, slots, c.d_lens,
                                 c.d_tables, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    got = c.d_tables.cpu().numpy()
    want = c.tables.copy()
    want[skip, pos[skip] // BS] = -7
    assert np.array_equal(got, want), "device tables differ from the block manager's"
    # the skipped token wrote nothing; then write it and check every byte
    after_skip = G.host_copy(c, seqs)
    c.d_tables.copy_(torch.from_numpy(c.tables).cuda())
    G.log(f"[append decode tokens dtype={cache}] all slots, then decode")
    pkv.pkv_append_decode_tokens(w.k_new, w.v_new, w.k_cache, w.v_cache, c.d_slots, c.d_lens,
                                 c.d_tables, w.k_scale, w.v_scale)
    G.run_decode(c)
    torch.cuda.synchronize()
    assert np.array_equal(c.d_tables.cpu().numpy(), c.tables)
    after = G.host_copy(c, seqs)
    G.oracle_cache_write(c, before)
    assert np.array_equal(G.bits(before.k), G.bits(after.k)), "K cache bytes differ"
    assert np.array_equal(G.bits(before.v), G.bits(after.v)), "V cache bytes differ"
    # the skipped sequence's block held its old bytes after the first call
    b_skip = np.searchsorted(before.blocks, int(c.slots_o[skip]) // BS)
    others = np.ones(len(before.blocks), dtype=bool)
    others[b_skip] = False
    assert np.array_equal(G.bits(after_skip.k[others]), G.bits(before.k[others]))
    assert not np.array_equal(G.bits(after_skip.k[b_skip]), G.bits(before.k[b_skip]))
    ref, rlse, _ = G.oracle_decode(c, before)
    G.compare_out(c, seqs, ref, rlse, f"append decode dtype={cache}")


@pytest.mark.parametrize("cache", [F32, BF16, E4M3])
def test_append_decode_tokens_block_size_32(cache):
    """The decode append over 32-token blocks: contexts are appended on the
    host, then one decode token per sequence goes through
    pkv_append_decode_tokens; the pools equal the oracle's cache write bit
    for bit and the device table equals the block manager's, with entry
    (L - 1) / 32 poisoned beforehand."""
    BS32, D, Hkv = 32, 128, 4
    gen = torch.Generator().manual_seed(130 + cache)
    lens = np.array([1, 31, 32, 33, 64, 65, 100, 1000], dtype=np.int64)  # after the append
    nb = int(sum(-(-lens // BS32))) + 5
    mb = int(-(-lens.max() // BS32)) + 1
    qd = F32 if cache == F32 else BF16
    ksc, vsc = (1.0, 1.0) if cache != E4M3 else (0.017, 0.019)
    order = np.random.default_rng(131 + cache).permutation(nb).astype(np.int32)
    bm = pkv.BlockManager(nb, BS32, mb, order)
    ob = O.BlockAllocator(nb, BS32, mb, order)
    ks, vs = workloads.pool_shapes(nb, Hkv, D, cache, BS32)
    k = _rand_storage(gen, ks, cache, ksc)
    v = _rand_storage(gen, vs, cache, vsc)
    dk, dv = _to_device(k, cache), _to_device(v, cache)
    S = len(lens)
    ids = np.arange(S, dtype=np.int64)
    for s in range(S):
        assert bm.add_seq(s) == 0 and ob.add_seq(s) == 0
    ctx = np.repeat(ids, lens - 1)
    if len(ctx):
        assert bm.append_slots(ctx)[0] == 0 and ob.append_slots(ctx)[0] == 0
    _, before_tables, _ = bm.export(ids)
    r1, s1 = bm.append_slots(ids)   # the decode token of every sequence
    r2, s2 = ob.append_slots(ids)
    assert r1 == r2 == 0 and np.array_equal(s1, s2)
    _, tables, blens = bm.export(ids)
    assert np.array_equal(blens, lens)
    d_tables = torch.from_numpy(before_tables).cuda()
    d_tables[torch.arange(S, device="cuda"), torch.from_numpy((lens - 1) // BS32).cuda()] = -5
    kn = _rand_storage(gen, (S, Hkv, D), qd)
    vn = _rand_storage(gen, (S, Hkv, D), qd)
    G.log(f"[append decode tokens, 32-token blocks, dtype={cache}]")
    pkv.pkv_append_decode_tokens(_to_device(kn, qd), _to_device(vn, qd), dk, dv,
                                 torch.from_numpy(s1).cuda(),
                                 torch.from_numpy(lens.astype(np.int32)).cuda(), d_tables, ksc, vsc)
    O.reshape_and_cache(kn, vn, qd, k, v, cache, s2, BS32, ksc, vsc)
    torch.cuda.synchronize()
    assert np.array_equal(d_tables.cpu().numpy(), tables), "device tables differ"
    assert np.array_equal(G.bits(G.np_storage(dk)), G.bits(k)), "K pool differs"
    assert np.array_equal(G.bits(G.np_storage(dv)), G.bits(v)), "V pool differs"
