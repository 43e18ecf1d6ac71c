"""Seeded synthetic inputs for paged decode attention (tests, smoke and bench).

This module holds none of the method's arithmetic: it draws random numbers,
lets torch round them to storage dtypes, lays them into pool tensors of the
library's layout, poisons never-read slots, and drives an allocator (either
the library's block manager or the oracle's) through a fixed recipe of
add / fork / append calls.  Both the HIP path and the oracle consume what it
makes.

The five workloads stand in for the pages' serving scenarios (Llama-3-8B,
Llama-3.1-70B with a shared system prompt, 70B with an fp8 E4M3 KV cache, and
405B at long context); they take the pages' knobs (16-token pages,
max_num_seqs 256, max_model_len 8192 / 32768 / 128000).  The pages measure on
no public dataset; every value here is N(0, 1).

Seeds: workload k uses numpy ``SeedSequence(k)``; its children feed, in
order, the lengths, the free-block shuffle, Q, the K pool, the V pool, new K
and new V.  Large tensors come from ``torch.Generator`` seeded from those
children, chunk by chunk, so the same bytes appear on any device of one kind.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Optional

import numpy as np
import torch

F32, BF16, E4M3 = 0, 1, 2
TORCH_STORAGE = {F32: torch.float32, BF16: torch.bfloat16, E4M3: torch.uint8}
ELEM_BYTES = {F32: 4, BF16: 2, E4M3: 1}
BLOCK = 16
CHUNK = 1 << 26  # elements per generation chunk


@dataclasses.dataclass
class Spec:
    """Shape and distribution of one workload."""
    index: int
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: int
    cache_dtype: int
    out_dtype: int
    lengths: Callable[[np.random.Generator, int], np.ndarray]
    prefix_tokens: int = 0          # shared system-prompt tokens (block aligned)
    pool_blocks: Optional[int] = None  # fixed pool size; None = needed + 10% slack
    partition_size: int = 0         # 0 = library default
    max_model_len: int = 0          # table width in tokens; 0 = max length rounded up
    block_size: int = BLOCK         # tokens per physical block (16 or 32)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _uniform(lo, hi):
    return lambda rng, n: rng.integers(lo, hi, size=n, endpoint=True).astype(np.int64)


def _prefix_lognormal(prefix, median, sigma, cap):
    def draw(rng, n):
        suf = np.rint(rng.lognormal(mean=math.log(median), sigma=sigma, size=n))
        suf = np.clip(suf, 1, cap - prefix).astype(np.int64)
        return prefix + suf
    return draw


SPECS = {
    1: Spec(1, "tiny fp32 paged decode (4 seqs, 8/2 heads, D 64, L in [1,200], 64-block pool)",
            4, 8, 2, 64, F32, F32, F32, _uniform(1, 200), pool_blocks=64),
    2: Spec(2, "Llama-3-8B-shaped bf16 decode layer (64 seqs, 32/8 heads, D 128, L in [512,8192])",
            64, 32, 8, 128, BF16, BF16, BF16, _uniform(512, 8192), max_model_len=8192),
    3: Spec(3, "Llama-3.1-70B-shaped bf16 decode with a shared 1024-token prefix "
               "(256 seqs, 64/8 heads, D 128, lognormal suffix median 1500 sigma 1.0, L <= 32768)",
            256, 64, 8, 128, BF16, BF16, BF16, _prefix_lognormal(1024, 1500.0, 1.0, 32768),
            prefix_tokens=1024, max_model_len=32768),
    4: Spec(4, "Llama-3.1-70B-shaped decode, fp8 E4M3 KV cache (256 seqs, 64/8 heads, D 128, "
               "L in [1024,32768])",
            256, 64, 8, 128, BF16, E4M3, BF16, _uniform(1024, 32768), max_model_len=32768),
    5: Spec(5, "Llama-3.1-405B-shaped bf16 long-context layer (8 seqs, 128/8 heads, D 128, "
               "L in [65536,131072], split-KV 512)",
            8, 128, 8, 128, BF16, BF16, BF16, _uniform(65536, 131072), partition_size=512,
            max_model_len=131072),
}


def _children(index: int):
    ss = np.random.SeedSequence(index)
    return ss.spawn(7)  # lengths, shuffle, q, k pool, v pool, new k, new v


def _seed_of(child) -> int:
    return int(child.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFF)


# --------------------------------------------------------------------- lengths / pool
def lengths(spec: Spec, num_seqs: Optional[int] = None) -> np.ndarray:
    """Final context lengths L_s (the decode step attends over L_s tokens)."""
    ch = _children(spec.index)
    n = spec.num_seqs if num_seqs is None else num_seqs
    return spec.lengths(np.random.Generator(np.random.PCG64(ch[0])), n)


def blocks_needed(spec: Spec, lens: np.ndarray) -> int:
    B = spec.block_size
    if spec.prefix_tokens:
        pre = spec.prefix_tokens // B
        return pre + int(sum(-(-(int(L) - spec.prefix_tokens) // B) for L in lens))
    return int(sum(-(-int(L) // B) for L in lens))


def pool_blocks(spec: Spec, lens: np.ndarray) -> int:
    if spec.pool_blocks is not None:
        return spec.pool_blocks
    return int(math.ceil(blocks_needed(spec, lens) * 1.1))


def max_blocks_per_seq(spec: Spec, lens: np.ndarray) -> int:
    width = spec.max_model_len or int(lens.max())
    return -(-width // spec.block_size)


def free_order(spec: Spec, num_blocks: int) -> np.ndarray:
    ch = _children(spec.index)
    return np.random.Generator(np.random.PCG64(ch[1])).permutation(num_blocks).astype(np.int32)


# --------------------------------------------------------------------- allocation recipe
def allocate_context(alloc, spec: Spec, lens: np.ndarray):
    """Drive an allocator (add_seq / fork_seq / append_slots) to hold L_s - 1
    tokens per sequence, then append the decode token of every sequence.

    Order: sequences are created in index order; with a shared prefix,
    sequence 0 receives the prefix tokens and sequences 1.. fork from it;
    then each sequence in index order receives its remaining context tokens;
    finally one append call adds the new token of every sequence.
    Returns the slot of each sequence's new token (int64 [S]).
    """
    S = len(lens)

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"allocation recipe: {what} returned {rc}")

    if spec.prefix_tokens:
        check(alloc.add_seq(0), "add_seq(0)")
        rc, _ = alloc.append_slots(np.zeros(spec.prefix_tokens, dtype=np.int64))
        check(rc, "prefix append")
        for s in range(1, S):
            check(alloc.fork_seq(0, s), f"fork_seq(0,{s})")
        start = spec.prefix_tokens
    else:
        for s in range(S):
            check(alloc.add_seq(s), f"add_seq({s})")
        start = 0
    for s in range(S):
        n = int(lens[s]) - 1 - start
        if n > 0:
            rc, _ = alloc.append_slots(np.full(n, s, dtype=np.int64))
            check(rc, f"context append seq {s}")
    rc, slots = alloc.append_slots(np.arange(S, dtype=np.int64))
    check(rc, "decode append")
    return slots


# --------------------------------------------------------------------- values
def _randn_chunks(seed: int, n: int, device) -> torch.Tensor:
    """n N(0,1) fp32 values, generated chunk by chunk with derived seeds."""
    out = torch.empty(n, dtype=torch.float32, device=device)
    for i, lo in enumerate(range(0, n, CHUNK)):
        hi = min(n, lo + CHUNK)
        g = torch.Generator(device=device)
        g.manual_seed(seed + i)
        out[lo:hi] = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32)
    return out


def _draw_into(dst_flat: torch.Tensor, seed: int, dtype_code: int, scale: Optional[float],
               device):
    """Fill a flat storage tensor with N(0,1) values rounded to dtype_code.
    bf16 by torch's round-to-nearest-even cast; fp8 codes are torch's E4M3FN
    cast of fp32(bf16(x)) / scale (the pool as an earlier cache write left it)."""
    n = dst_flat.numel()
    for i, lo in enumerate(range(0, n, CHUNK)):
        hi = min(n, lo + CHUNK)
        g = torch.Generator(device=device)
        g.manual_seed(seed + i)
        x = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32)
        if dtype_code == F32:
            dst_flat[lo:hi] = x
        elif dtype_code == BF16:
            dst_flat[lo:hi] = x.to(torch.bfloat16)
        else:
            xb = x.to(torch.bfloat16).to(torch.float32)
            dst_flat[lo:hi] = (xb / scale).to(torch.float8_e4m3fn).view(torch.uint8)


def _amax_bf16(seed: int, n: int, device) -> float:
    m = torch.zeros((), dtype=torch.float32, device=device)
    for i, lo in enumerate(range(0, n, CHUNK)):
        hi = min(n, lo + CHUNK)
        g = torch.Generator(device=device)
        g.manual_seed(seed + i)
        x = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32)
        m = torch.maximum(m, x.to(torch.bfloat16).to(torch.float32).abs().max())
    return float(m.item())


def pool_shapes(num_blocks, H, D, cache_dtype, block_size=BLOCK):
    X = 16 // ELEM_BYTES[cache_dtype]
    return (num_blocks, H, D // X, block_size, X), (num_blocks, H, D, block_size)


@dataclasses.dataclass
class Workload:
    spec: Spec
    lens: np.ndarray            # final L_s (host)
    num_blocks: int
    max_blocks: int
    free_order: np.ndarray
    q: torch.Tensor             # [S][Hq][D] storage dtype
    k_cache: torch.Tensor       # [nb][Hkv][D/X][block_size][X]
    v_cache: torch.Tensor       # [nb][Hkv][D][block_size]
    k_new: torch.Tensor         # [S][Hkv][D] (f32 or bf16)
    v_new: torch.Tensor
    k_scale: float
    v_scale: float
    scale: float


def make(spec: Spec, device="cpu", num_seqs: Optional[int] = None,
         lens: Optional[np.ndarray] = None) -> Workload:
    """Seeded values for a workload (pools not yet poisoned, tables not built)."""
    ch = _children(spec.index)
    if lens is None:
        lens = lengths(spec, num_seqs)
    S = len(lens)
    nb = pool_blocks(spec, lens)
    mb = max_blocks_per_seq(spec, lens)
    Hq, Hkv, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    kshape, vshape = pool_shapes(nb, Hkv, D, spec.cache_dtype, spec.block_size)
    new_dtype = torch.float32 if spec.q_dtype == F32 else torch.bfloat16
    pool_n = int(np.prod(kshape))
    new_n = S * Hkv * D
    k_scale = v_scale = 1.0
    if spec.cache_dtype == E4M3:
        # per-tensor scale: fp32 amax over every generated value (pool and new
        # tokens) divided by the largest finite E4M3 value, 448
        amk = max(_amax_bf16(_seed_of(ch[3]), pool_n, device),
                  _amax_bf16(_seed_of(ch[5]), new_n, device))
        amv = max(_amax_bf16(_seed_of(ch[4]), pool_n, device),
                  _amax_bf16(_seed_of(ch[6]), new_n, device))
        k_scale = float(np.float32(amk) / np.float32(448.0))
        v_scale = float(np.float32(amv) / np.float32(448.0))
    k_cache = torch.empty(kshape, dtype=TORCH_STORAGE[spec.cache_dtype], device=device)
    v_cache = torch.empty(vshape, dtype=TORCH_STORAGE[spec.cache_dtype], device=device)
    _draw_into(k_cache.view(-1), _seed_of(ch[3]), spec.cache_dtype, k_scale, device)
    _draw_into(v_cache.view(-1), _seed_of(ch[4]), spec.cache_dtype, v_scale, device)
    q = torch.empty((S, Hq, D), dtype=TORCH_STORAGE[spec.q_dtype], device=device)
    _draw_into(q.view(-1), _seed_of(ch[2]), spec.q_dtype, None, device)
    k_new = _randn_chunks(_seed_of(ch[5]), new_n, device).to(new_dtype).view(S, Hkv, D)
    v_new = _randn_chunks(_seed_of(ch[6]), new_n, device).to(new_dtype).view(S, Hkv, D)
    return Workload(spec, np.asarray(lens, dtype=np.int64), nb, mb, free_order(spec, nb), q,
                    k_cache, v_cache, k_new, v_new, k_scale, v_scale,
                    float(np.float32(1.0 / math.sqrt(D))))


# --------------------------------------------------------------------- poison
def poison_value(cache_dtype):
    return {F32: float("nan"), BF16: float("nan"), E4M3: 0x7F}[cache_dtype]


def poison_unused(w: Workload, tables: np.ndarray, filled: np.ndarray):
    """Write NaN (fp32/bf16) or the E4M3 NaN code into every slot that holds
    no token: blocks referenced by no table, and the slots at or beyond each
    sequence's filled length in its blocks.  `filled` is tokens held per
    sequence before the decode token is written."""
    nb = w.num_blocks
    B = w.spec.block_size
    used = np.zeros(nb, dtype=bool)
    for s in range(len(filled)):
        n = -(-int(filled[s]) // B)
        used[tables[s, :n]] = True
    val = poison_value(w.spec.cache_dtype)
    dev = w.k_cache.device
    free_ids = torch.from_numpy(np.nonzero(~used)[0]).to(dev)
    if free_ids.numel():
        w.k_cache[free_ids] = val
        w.v_cache[free_ids] = val
    # tail slots of each sequence's last (partial) block; shared prefix blocks are full
    for s in range(len(filled)):
        L = int(filled[s])
        if L % B:
            b = int(tables[s, L // B])
            w.k_cache[b, :, :, L % B:, :] = val
            w.v_cache[b, :, :, L % B:] = val
