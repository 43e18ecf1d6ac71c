"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: torch's
codecs, numpy / torch SDPA dense attention on gathered contiguous K and V,
scalar brute force, closed forms, invariants of paging, and the worked byte
example printed on "vLLM PagedAttention Optimization: Complete Step-by-Step
Tuning Guide for Low-Latency Inference", Step 1.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests import dense_ref

HERE = os.path.dirname(os.path.abspath(__file__))
BS = 16


# ----------------------------------------------------------------- helpers
def rand_storage(rng, shape, dtype, scale=1.0):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    if dtype == O.F32:
        return x.numpy()
    if dtype == O.BF16:
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return (x.to(torch.bfloat16).float() / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_problem(seed, lens, Hq=8, Hkv=2, D=32, cache_dtype=O.BF16, q_dtype=O.BF16, slack=3,
                 k_scale=1.0, v_scale=1.0):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    S = len(lens)
    nblk = [-(-int(L) // BS) for L in lens]
    nb = sum(nblk) + slack
    mb = max(max(nblk), 1) + 1
    X = 16 // {O.F32: 4, O.BF16: 2, O.E4M3: 1}[cache_dtype]
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((S, mb), -1, dtype=np.int32)
    pos = 0
    for s in range(S):
        tables[s, :nblk[s]] = perm[pos:pos + nblk[s]]
        pos += nblk[s]
    k = rand_storage(rng, (nb, Hkv, D // X, BS, X), cache_dtype, k_scale)
    v = rand_storage(rng, (nb, Hkv, D, BS), cache_dtype, v_scale)
    q = rand_storage(rng, (S, Hq, D), q_dtype)
    return dict(q=q, q_dtype=q_dtype, k_cache=k, v_cache=v, cache_dtype=cache_dtype,
                block_tables=tables, context_lens=lens, num_kv_heads=Hkv, block_size=BS,
                scale=float(np.float32(1 / math.sqrt(D))), k_scale=k_scale, v_scale=v_scale)


def dense_args(p):
    return (p["q"], p["q_dtype"], p["k_cache"], p["v_cache"], p["cache_dtype"],
            p["block_tables"], p["context_lens"], p["scale"], p["k_scale"], p["v_scale"])


# ----------------------------------------------------------------- byte accounting
def test_kv_bytes_worked_example():
    vals = {}
    with open(os.path.join(HERE, "golden", "kv_bytes_llama70b.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    b = O.kv_bytes_per_token(vals["layers"], vals["kv_heads"], vals["head_dim"],
                             vals["bytes_per_elem"])
    assert b == vals["bytes_per_token"]
    assert b * vals["context_tokens"] == vals["approx_gib_per_sequence"] * 2**30
    # a dropped factor (K and V) or a wrong operand shows up on other shapes
    assert O.kv_bytes_per_token(1, 1, 1, 1) == 2
    assert O.kv_bytes_per_token(32, 8, 128, 1) == 2 * 32 * 8 * 128


# ----------------------------------------------------------------- e4m3
def test_e4m3_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], got[~nan])
    assert O.e4m3_decode(0x7E) == 448.0 and O.e4m3_decode(0x01) == 2.0**-9
    assert O.e4m3_decode(0x08) == 2.0**-6 and O.e4m3_decode(0x38) == 1.0


def test_e4m3_encode_vs_torch_and_ties():
    finite = [c for c in range(0x7F)]
    vals = np.array([O.e4m3_decode(c) for c in finite])
    mids = (vals[:-1] + vals[1:]) / 2  # exact in fp32: tie points
    rng = np.random.default_rng(7)
    rnd = np.concatenate([rng.uniform(-448, 448, 20000),
                          rng.standard_normal(20000) * 2.0**rng.integers(-12, 8, 20000),
                          vals, -vals, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    x = rnd.astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = O.e4m3_encode_array(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    # ties go to the even code
    for c in range(0x7E):
        m = np.float32(mids[c])
        assert O.e4m3_encode(float(m)) == (c if c % 2 == 0 else c + 1)


def test_e4m3_encode_saturates_and_roundtrips():
    for x in [448.0, 449.0, 463.9, 464.0, 500.0, 1e6, float("inf")]:
        assert O.e4m3_encode(x) == 0x7E
        assert O.e4m3_encode(-x) == 0xFE
    assert O.e4m3_encode(float("nan")) & 0x7F == 0x7F
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert O.e4m3_encode(O.e4m3_decode(c)) == c


# ----------------------------------------------------------------- bf16
def test_bf16_encode_vs_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, 4096, dtype=np.uint32) << 16) | 0x8000
    near_max = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0x7F7F0000], dtype=np.uint32)
    allbits = np.concatenate([bits, ties, near_max, near_max | 0x80000000])
    x = allbits.view(np.float32)
    x = x[np.isfinite(x)]
    got = O.bf16_encode_array(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    assert O.bf16_decode(0x3F80) == 1.0 and O.bf16_decode(0xC000) == -2.0


# ----------------------------------------------------------------- attention
@pytest.mark.parametrize("cache_dtype,q_dtype", [(O.F32, O.F32), (O.BF16, O.BF16), (O.E4M3, O.BF16)])
def test_dense_equivalence(cache_dtype, q_dtype):
    ks, vs = (0.0123, 0.0071) if cache_dtype == O.E4M3 else (1.0, 1.0)
    p = make_problem(11, [1, 17, 33, 50, 16, 130], Hq=8, Hkv=2, D=32, cache_dtype=cache_dtype,
                     q_dtype=q_dtype, k_scale=ks, v_scale=vs)
    out, lse = O.decode_attention(**p)
    ref, rlse = dense_ref.dense_attention(*dense_args(p))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))
    np.testing.assert_allclose(lse, rlse, rtol=1e-13, atol=1e-12)


def test_sdpa_equivalence_gqa():
    p = make_problem(12, [5, 40, 77], Hq=16, Hkv=2, D=64, cache_dtype=O.BF16)
    out, _ = O.decode_attention(**p)
    ref = dense_ref.sdpa_attention(*dense_args(p))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_brute_force_tiny():
    """Scalar Python, fsum, and the max-free form w_t = 1 / sum_u exp(sc_u - sc_t)."""
    p = make_problem(13, [3, 19, 40], Hq=4, Hkv=2, D=8, cache_dtype=O.F32, q_dtype=O.F32)
    out, _ = O.decode_attention(**p)
    K, V = dense_ref.token_major(p["k_cache"], p["v_cache"])
    q = p["q"]
    for s in range(3):
        L = int(p["context_lens"][s])
        for h in range(4):
            g = h // 2
            sc = []
            for t in range(L):
                b = p["block_tables"][s][t // BS]
                sc.append(p["scale"] * math.fsum(float(q[s, h, d]) * float(K[b, g, t % BS, d])
                                                 for d in range(8)))
            w = [1.0 / math.fsum(math.exp(su - st) for su in sc) for st in sc]
            for d in range(8):
                ref = math.fsum(w[t] * float(V[p["block_tables"][s][t // BS], g, t % BS, d])
                                for t in range(L))
                assert abs(out[s, h, d] - ref) <= 1e-13


def permute_blocks(p, seed):
    rng = np.random.default_rng(seed)
    nb = p["k_cache"].shape[0]
    pi = rng.permutation(nb)  # old block b moves to pi[b]
    k2 = np.empty_like(p["k_cache"])
    v2 = np.empty_like(p["v_cache"])
    k2[pi] = p["k_cache"]
    v2[pi] = p["v_cache"]
    t2 = p["block_tables"].copy()
    t2[t2 >= 0] = pi[t2[t2 >= 0]]
    return dict(p, k_cache=k2, v_cache=v2, block_tables=t2)


@pytest.mark.parametrize("cache_dtype", [O.F32, O.BF16, O.E4M3])
def test_block_placement_invariance_bit_identical(cache_dtype):
    p = make_problem(14, [7, 64, 100, 1], cache_dtype=cache_dtype,
                     q_dtype=O.F32 if cache_dtype == O.F32 else O.BF16,
                     k_scale=0.02 if cache_dtype == O.E4M3 else 1.0)
    out, lse = O.decode_attention(**p)
    out2, lse2 = O.decode_attention(**permute_blocks(p, 99))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_shared_prefix_equals_copied_bit_identical():
    rng = np.random.default_rng(15)
    S, Hq, Hkv, D = 4, 8, 2, 32
    pre_blocks = 3
    suffix = [5, 20, 16, 33]
    lens = np.array([pre_blocks * BS + x for x in suffix], dtype=np.int32)
    suf_blocks = [-(-x // BS) for x in suffix]
    nb_shared = pre_blocks + sum(suf_blocks)
    nb_copied = S * pre_blocks + sum(suf_blocks)
    k_pre = rand_storage(rng, (pre_blocks, Hkv, D // 8, BS, 8), O.BF16)
    v_pre = rand_storage(rng, (pre_blocks, Hkv, D, BS), O.BF16)
    k_suf = rand_storage(rng, (sum(suf_blocks), Hkv, D // 8, BS, 8), O.BF16)
    v_suf = rand_storage(rng, (sum(suf_blocks), Hkv, D, BS), O.BF16)
    q = rand_storage(rng, (S, Hq, D), O.BF16)
    mb = pre_blocks + max(suf_blocks)
    # shared: blocks 0..2 are the prefix in every table
    ts = np.full((S, mb), -1, np.int32)
    # copied: each sequence owns a copy of the prefix
    tc = np.full((S, mb), -1, np.int32)
    kc = np.concatenate([k_pre] * S + [k_suf])
    vc = np.concatenate([v_pre] * S + [v_suf])
    ksh = np.concatenate([k_pre, k_suf])
    vsh = np.concatenate([v_pre, v_suf])
    pos = 0
    for s in range(S):
        ts[s, :pre_blocks] = np.arange(pre_blocks)
        tc[s, :pre_blocks] = s * pre_blocks + np.arange(pre_blocks)
        ts[s, pre_blocks:pre_blocks + suf_blocks[s]] = pre_blocks + pos + np.arange(suf_blocks[s])
        tc[s, pre_blocks:pre_blocks + suf_blocks[s]] = S * pre_blocks + pos + np.arange(suf_blocks[s])
        pos += suf_blocks[s]
    assert ksh.shape[0] == nb_shared and kc.shape[0] == nb_copied
    common = dict(q=q, q_dtype=O.BF16, cache_dtype=O.BF16, context_lens=lens, num_kv_heads=Hkv,
                  block_size=BS, scale=0.17677669)
    a = O.decode_attention(k_cache=ksh, v_cache=vsh, block_tables=ts, **common)
    b = O.decode_attention(k_cache=kc, v_cache=vc, block_tables=tc, **common)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_softmax_weights_sum_to_one_and_lse():
    p = make_problem(16, [1, 2, 31, 200], Hq=8, Hkv=2, D=32)
    out, lse, w = O.decode_attention(**p, want_weights=True)
    for s, L in enumerate(p["context_lens"]):
        sums = w[s, :, :L].sum(axis=1)
        np.testing.assert_allclose(sums, 1.0, rtol=0, atol=1e-12)
        assert np.all(w[s, :, :L] >= 0)


def test_closed_forms():
    # L = 1: out = v_0 for any q
    p = make_problem(17, [1, 2, 2], Hq=4, Hkv=1, D=16, cache_dtype=O.F32, q_dtype=O.F32)
    out, lse = O.decode_attention(**p)
    K, V = dense_ref.token_major(p["k_cache"], p["v_cache"])
    b0 = p["block_tables"][0][0]
    for h in range(4):
        assert np.array_equal(out[0, h], V[b0, 0, 0].astype(np.float64))
    # L = 2: w_0 = 1 / (1 + exp(sc_1 - sc_0))
    for s in (1, 2):
        b = p["block_tables"][s][0]
        for h in range(4):
            q = p["q"][s, h].astype(np.float64)
            sc = [p["scale"] * float(q @ K[b, 0, t].astype(np.float64)) for t in (0, 1)]
            w0 = 1.0 / (1.0 + math.exp(sc[1] - sc[0]))
            ref = w0 * V[b, 0, 0].astype(np.float64) + (1 - w0) * V[b, 0, 1].astype(np.float64)
            np.testing.assert_allclose(out[s, h], ref, rtol=0, atol=1e-14)
            assert abs(lse[s, h] - (max(sc) + math.log(sum(math.exp(x - max(sc)) for x in sc)))) < 1e-14
    # K == 0: out is the plain mean of the V rows
    p = make_problem(18, [37, 5], Hq=4, Hkv=2, D=16, cache_dtype=O.F32, q_dtype=O.F32)
    p["k_cache"][:] = 0
    out, _ = O.decode_attention(**p)
    K, V = dense_ref.token_major(p["k_cache"], p["v_cache"])
    for s, L in enumerate(p["context_lens"]):
        _, Vs = dense_ref.gather(p["k_cache"], p["v_cache"], p["block_tables"][s], int(L))
        mean = Vs.astype(np.float64).mean(axis=0)  # [Hkv][D]
        for h in range(4):
            np.testing.assert_allclose(out[s, h], mean[h // 2], rtol=0, atol=1e-14)
    # V == c: out == c; and linearity in V
    p = make_problem(19, [50, 3], Hq=4, Hkv=2, D=16, cache_dtype=O.F32, q_dtype=O.F32)
    p["v_cache"][:] = 0.75
    out, _ = O.decode_attention(**p)
    np.testing.assert_allclose(out, 0.75, rtol=0, atol=1e-15)
    p = make_problem(20, [50, 3], Hq=4, Hkv=2, D=16, cache_dtype=O.F32, q_dtype=O.F32)
    o1, _ = O.decode_attention(**p)
    p2 = dict(p, v_cache=(p["v_cache"] * 2).astype(np.float32))  # exact in fp32
    o2, _ = O.decode_attention(**p2)
    assert np.array_equal(o2, 2 * o1)


def test_empty_sequence():
    p = make_problem(21, [0, 9], Hq=4, Hkv=2, D=16)
    out, lse = O.decode_attention(**p)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(out[1]))


def test_scales_are_applied():
    """k_scale multiplies the scores, v_scale the output (fp8 cache)."""
    p = make_problem(22, [40, 70], cache_dtype=O.E4M3, k_scale=0.01, v_scale=0.02)
    out, _ = O.decode_attention(**p)
    ref, _ = dense_ref.dense_attention(*dense_args(p))
    np.testing.assert_allclose(out, ref, atol=1e-13)
    out_v, _ = O.decode_attention(**dict(p, v_scale=0.04))
    np.testing.assert_allclose(out_v, 2 * out, atol=1e-13)
    out_k, _ = O.decode_attention(**dict(p, k_scale=0.02))
    assert not np.allclose(out_k, out)


@pytest.mark.parametrize("part", [16, 32, 48, 512])
def test_split_merge_equals_unsplit(part):
    p = make_problem(23, [1, 15, 16, 17, 100, 511, 513, 1100], Hq=8, Hkv=2, D=32)
    out, lse = O.decode_attention(**p)
    out2, lse2 = O.decode_attention_split(**p, partition_tokens=part)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


def test_poisoned_unused_slots_never_read():
    p = make_problem(24, [5, 17, 32], cache_dtype=O.BF16)
    out, _ = O.decode_attention(**p)
    k, v = p["k_cache"].copy(), p["v_cache"].copy()
    used = set()
    for s, L in enumerate(p["context_lens"]):
        n = -(-int(L) // BS)
        for j in range(n):
            b = p["block_tables"][s][j]
            used.add(int(b))
            if j == n - 1 and L % BS:
                k[b, :, :, L % BS:, :] = 0x7FC0
                v[b, :, :, L % BS:] = 0x7FC0
    for b in range(k.shape[0]):
        if b not in used:
            k[b] = 0x7FC0
            v[b] = 0x7FC0
    out2, _ = O.decode_attention(**dict(p, k_cache=k, v_cache=v))
    assert np.array_equal(out, out2)


# ----------------------------------------------------------------- cache write
@pytest.mark.parametrize("src,dst", [(O.F32, O.F32), (O.BF16, O.BF16), (O.F32, O.BF16),
                                     (O.BF16, O.E4M3), (O.F32, O.E4M3)])
def test_cache_write_layout_and_rounding(src, dst):
    rng = np.random.default_rng(30)
    T, H, D, nb = 6, 2, 32, 5
    X = 16 // {O.F32: 4, O.BF16: 2, O.E4M3: 1}[dst]
    kn = rand_storage(rng, (T, H, D), src)
    vn = rand_storage(rng, (T, H, D), src)
    k = np.zeros((nb, H, D // X, BS, X), {0: np.float32, 1: np.uint16, 2: np.uint8}[dst])
    v = np.zeros((nb, H, D, BS), k.dtype)
    slots = np.array([3, 17, -1, 79, 40, 0], dtype=np.int64)
    ks, vs = (0.013, 0.029) if dst == O.E4M3 else (1.0, 1.0)
    O.reshape_and_cache(kn, vn, src, k, v, dst, slots, BS, ks, vs)
    K, V = dense_ref.token_major(k, v)

    def expect(x, scale):
        xf = torch.from_numpy(dense_ref.decode_np(x, src).astype(np.float32))
        if dst == O.F32:
            return xf.numpy()
        if dst == O.BF16:
            return xf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return (xf / np.float32(scale)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    written = set()
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        b, o = divmod(int(sl), BS)
        written.add((b, o))
        assert np.array_equal(K[b, :, o, :], expect(kn[t], ks))
        assert np.array_equal(V[b, :, o, :], expect(vn[t], vs))
    for b in range(nb):
        for o in range(BS):
            if (b, o) not in written:
                assert not K[b, :, o, :].any() and not V[b, :, o, :].any()


# ----------------------------------------------------------------- block allocation
def test_allocation_closed_form_fifo_and_uniqueness():
    nb, mb = 40, 8
    order = np.random.default_rng(40).permutation(nb).astype(np.int32)
    A = O.BlockAllocator(nb, BS, mb, order)
    for s in range(3):
        assert A.add_seq(s) == O.OK
    taken = []
    plan = [0] * 20 + [1] * 16 + [2] * 1 + [0, 1, 2] * 10
    lens = [0, 0, 0]
    for sid in plan:
        rc, slot = A.append_slots([sid])
        assert rc == O.OK
        p = lens[sid]
        if p % BS == 0:
            taken.append(int(slot[0]) // BS)
        lens[sid] += 1
    assert taken == list(order[:len(taken)])  # FIFO in the given order
    rc, tables, L = A.export([0, 1, 2])
    assert rc == O.OK and list(L) == lens
    # closed form for every live token, and uniqueness
    seen = set()
    for s in range(3):
        for p in range(lens[s]):
            slot = tables[s][p // BS] * BS + p % BS
            assert slot not in seen
            seen.add(slot)
        assert np.all(tables[s][-(-lens[s] // BS):] == -1)
    assert A.num_free() == nb - len(taken)


def test_allocation_batch_slots_match_closed_form():
    A = O.BlockAllocator(16, BS, 4, np.arange(16)[::-1].copy())
    A.add_seq(5)
    A.add_seq(9)
    rc, slots = A.append_slots([5, 9, 5, 5, 9])
    assert rc == O.OK
    rc, t, L = A.export([5, 9])
    assert list(slots) == [t[0][0] * BS + 0, t[1][0] * BS + 0, t[0][0] * BS + 1, t[0][0] * BS + 2,
                           t[1][0] * BS + 1]
    assert t[0][0] == 15 and t[1][0] == 14


def test_allocation_out_of_blocks_is_all_or_nothing():
    A = O.BlockAllocator(3, BS, 4)
    A.add_seq(0)
    A.add_seq(1)
    rc, _ = A.append_slots([0] * 33)  # needs 3 blocks
    assert rc == O.OK and A.num_free() == 0
    before = A.export([0, 1])
    rc, _ = A.append_slots([0] * 15 + [1])  # seq 1 needs a block: none left
    assert rc == O.OUT_OF_BLOCKS
    after = A.export([0, 1])
    assert np.array_equal(before[1], after[1]) and np.array_equal(before[2], after[2])


def test_allocation_fork_refcounts_free_and_reuse():
    nb = 10
    A = O.BlockAllocator(nb, BS, 6)
    A.add_seq(0)
    A.append_slots([0] * 32)  # two full blocks: 0, 1
    for c in (1, 2, 3):
        assert A.fork_seq(0, c) == O.OK
    assert A.refcount(0) == 4 and A.refcount(1) == 4
    for c in (0, 1, 2, 3):
        rc, _ = A.append_slots([c])
        assert rc == O.OK  # block aligned: each gets a private block
    _, t, L = A.export([0, 1, 2, 3])
    total_refs = sum(A.refcount(b) for b in range(nb))
    assert total_refs == int((t >= 0).sum())
    assert len({int(t[c][2]) for c in range(4)}) == 4
    assert A.free_seq(1) == O.OK
    assert A.refcount(0) == 3
    free_before = A.num_free()
    for c in (0, 2, 3):
        A.free_seq(c)
    assert A.num_free() == nb and free_before == nb - 6 + 1
    assert A.free_seq(0) == O.UNKNOWN_SEQ


def test_allocation_shared_tail_refused():
    A = O.BlockAllocator(8, BS, 4)
    A.add_seq(0)
    A.append_slots([0] * 20)  # second block partially filled
    A.fork_seq(0, 1)
    rc, _ = A.append_slots([1])
    assert rc == O.SHARED_TAIL
    assert A.add_seq(0) == O.SEQ_EXISTS
    rc, _ = A.append_slots([7])
    assert rc == O.UNKNOWN_SEQ


def test_cow_fork_inside_a_block_then_diverge():
    """Fork in the middle of a block, then both sequences append different
    tokens through copy-on-write: each sequence's attention equals dense
    attention over its own logical token list (computed from the token
    arrays, no pool or table involved), and only the first writer copies."""
    rng = np.random.default_rng(51)
    Hq, Hkv, D, nb = 4, 2, 16, 12
    A = O.BlockAllocator(nb, BS, 8, rng.permutation(nb).astype(np.int32))
    pk = np.zeros((nb, Hkv, D // 4, BS, 4), np.float32)
    pv = np.zeros((nb, Hkv, D, BS), np.float32)

    def toks(n):
        return (rng.standard_normal((n, Hkv, D)).astype(np.float32),
                rng.standard_normal((n, Hkv, D)).astype(np.float32))

    base = toks(37)  # blocks 0, 1 full, block 2 holds 5 tokens
    A.add_seq(0)
    rc, slots = A.append_slots([0] * 37)
    assert rc == O.OK
    O.reshape_and_cache(base[0], base[1], O.F32, pk, pv, O.F32, slots, BS)
    assert A.fork_seq(0, 1) == O.OK
    new1, new0 = toks(10), toks(7)
    rc, slots, src, dst = A.append_slots_cow([1] * 10 + [0] * 7)
    assert rc == O.OK
    _, t, lens = A.export([0, 1])
    assert len(src) == 1 and src[0] == t[0][2] and dst[0] == t[1][2] and src[0] != dst[0]
    assert A.refcount(int(src[0])) == 1 and A.refcount(int(dst[0])) == 1
    assert all(A.refcount(int(b)) == 2 for b in t[0][:2])
    O.copy_blocks(pk, pv, src, dst)
    O.reshape_and_cache(np.concatenate([new1[0], new0[0]]), np.concatenate([new1[1], new0[1]]),
                        O.F32, pk, pv, O.F32, slots, BS)
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    scale = float(np.float32(0.25))
    out, lse = O.decode_attention(q, O.F32, pk, pv, O.F32, t, lens, Hkv, BS, scale)
    assert list(lens) == [44, 47]
    for s, extra in ((0, new0), (1, new1)):
        K = np.concatenate([base[0], extra[0]]).astype(np.float64)  # [L][Hkv][D]
        V = np.concatenate([base[1], extra[1]]).astype(np.float64)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            sc = K[:, g, :] @ q[s, h].astype(np.float64) * scale
            w = np.exp(sc - sc.max())
            ref = (w / w.sum()) @ V[:, g, :]
            assert np.max(np.abs(out[s, h] - ref)) <= 1e-12
            assert abs(lse[s, h] - (sc.max() + np.log(w.sum()))) <= 1e-12


def test_allocation_freed_blocks_go_to_fifo_tail():
    """After a free, allocation drains the never-used blocks in the given
    order first, then the freed blocks in the order the table held them."""
    nb = 12
    order = np.random.default_rng(41).permutation(nb).astype(np.int32)
    A = O.BlockAllocator(nb, BS, nb, order)
    A.add_seq(0)
    A.add_seq(1)
    A.append_slots([0] * (3 * BS))  # seq 0 takes order[0:3]
    A.append_slots([1] * (2 * BS))  # seq 1 takes order[3:5]
    _, t, _ = A.export([0])
    freed = list(t[0][:3])
    assert A.free_seq(0) == O.OK
    A.add_seq(2)
    rc, slots = A.append_slots([2] * ((nb - 2) * BS))
    assert rc == O.OK and A.num_free() == 0
    got = [int(slots[j * BS]) // BS for j in range(nb - 2)]
    assert got == list(order[5:]) + freed


# ----------------------------------------------------------------- chunked prefill
def prefill_problem(seed, lens, chunks, **kw):
    p = make_problem(seed, lens, **kw)
    rng = np.random.default_rng(seed + 1000)
    qstart = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    Hq, D = p["q"].shape[1], p["q"].shape[2]
    p["q"] = rand_storage(rng, (int(qstart[-1]), Hq, D), p["q_dtype"])
    p["query_start"] = qstart
    return p


def prefill_args(p):
    return dict(q=p["q"], q_dtype=p["q_dtype"], k_cache=p["k_cache"], v_cache=p["v_cache"],
                cache_dtype=p["cache_dtype"], block_tables=p["block_tables"],
                context_lens=p["context_lens"], query_start=p["query_start"],
                num_kv_heads=p["num_kv_heads"], block_size=p["block_size"], scale=p["scale"],
                k_scale=p["k_scale"], v_scale=p["v_scale"])


@pytest.mark.parametrize("cache_dtype,q_dtype", [(O.F32, O.F32), (O.BF16, O.BF16), (O.E4M3, O.BF16)])
def test_prefill_equals_dense_causal(cache_dtype, q_dtype):
    ks = 0.02 if cache_dtype == O.E4M3 else 1.0
    p = prefill_problem(61, [40, 17, 100, 5], [40, 3, 37, 1], cache_dtype=cache_dtype,
                        q_dtype=q_dtype, k_scale=ks, v_scale=ks)
    out, lse = O.prefill_attention(**prefill_args(p))
    ref, rlse = dense_ref.dense_prefill(p["q"], q_dtype, p["k_cache"], p["v_cache"], cache_dtype,
                                        p["block_tables"], p["context_lens"], p["query_start"],
                                        p["scale"], ks, ks)
    assert np.max(np.abs(out - ref)) <= 1e-12
    assert np.max(np.abs(lse - rlse)) <= 1e-12


def test_prefill_full_sequence_is_causal_self_attention():
    """C = L: every token of the sequence is a query; torch's causal SDPA
    (fp64, KV heads repeated over their group) gives the same rows."""
    p = prefill_problem(62, [33, 70], [33, 70], cache_dtype=O.F32, q_dtype=O.F32, Hq=8, Hkv=2,
                        D=32)
    out, _ = O.prefill_attention(**prefill_args(p))
    qs = p["query_start"]
    for s in range(2):
        L = int(p["context_lens"][s])
        Ks, Vs = dense_ref.gather(p["k_cache"], p["v_cache"], p["block_tables"][s], L)
        Kt = torch.from_numpy(Ks.astype(np.float64)).repeat_interleave(4, dim=1).permute(1, 0, 2)
        Vt = torch.from_numpy(Vs.astype(np.float64)).repeat_interleave(4, dim=1).permute(1, 0, 2)
        Qt = torch.from_numpy(p["q"][qs[s]:qs[s + 1]].astype(np.float64)).permute(1, 0, 2)
        r = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, is_causal=True,
                                                             scale=dense_ref.f32(p["scale"]))
        assert np.max(np.abs(out[qs[s]:qs[s + 1]] - r.permute(1, 0, 2).numpy())) <= 1e-12


def test_prefill_single_token_chunk_is_decode():
    p = prefill_problem(63, [1, 16, 17, 300], [1, 1, 1, 1])
    out, lse = O.prefill_attention(**prefill_args(p))
    d_out, d_lse = O.decode_attention(p["q"], p["q_dtype"], p["k_cache"], p["v_cache"],
                                      p["cache_dtype"], p["block_tables"], p["context_lens"],
                                      p["num_kv_heads"], BS, p["scale"])
    assert np.array_equal(out, d_out) and np.array_equal(lse, d_lse)


def test_prefill_two_chunks_equal_one():
    """Queries [a, b) in one call equal [a, m) with the context cut at m,
    then [m, b): the position bookkeeping L - C + j agrees."""
    p = prefill_problem(64, [90], [50])
    whole, wl = O.prefill_attention(**prefill_args(p))
    first = dict(prefill_args(p), q=np.ascontiguousarray(p["q"][:20]),
                 context_lens=np.array([60], np.int32), query_start=np.array([0, 20], np.int32))
    second = dict(prefill_args(p), q=np.ascontiguousarray(p["q"][20:]),
                  query_start=np.array([0, 30], np.int32))
    o1, l1 = O.prefill_attention(**first)
    o2, l2 = O.prefill_attention(**second)
    assert np.array_equal(np.concatenate([o1, o2]), whole)
    assert np.array_equal(np.concatenate([l1, l2]), wl)


def test_prefill_chunk_longer_than_context_rows_are_empty():
    p = prefill_problem(65, [3], [5])
    out, lse = O.prefill_attention(**prefill_args(p))
    assert np.all(out[:2] == 0) and np.all(np.isneginf(lse[:2]))
    assert np.all(np.isfinite(lse[2:]))
