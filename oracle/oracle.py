"""TEST INFRASTRUCTURE ONLY: numpy/ctypes front end of the fp64 CPU oracle.

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It loads ``oracle/liboracle.so`` (built
from ``oracle/oracle.c`` by :func:`build`) and shares nothing with the HIP
library in ``paged_kv_cache_189_amd``.

Dtype codes: 0 = fp32, 1 = bf16 (stored as uint16 bit patterns),
2 = fp8 OCP E4M3FN (stored as uint8 codes).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# A test may point the oracle at another build of oracle.c (a copy with a
# planted mistake, to show that the pins catch it); that build is used as is.
LIB_OVERRIDE = os.environ.get("PKV_ORACLE_LIB")

F32, BF16, E4M3 = 0, 1, 2
NP_STORAGE = {F32: np.float32, BF16: np.uint16, E4M3: np.uint8}

OK, INVALID, OUT_OF_BLOCKS, UNKNOWN_SEQ, SEQ_EXISTS, SHARED_TAIL = 0, -1, -2, -3, -4, -5


def compile_to(src: str, out: str) -> str:
    """Compile an oracle source with gcc (OpenMP, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build() -> str:
    return compile_to(SRC, LIB)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if LIB_OVERRIDE:
            L = C.CDLL(LIB_OVERRIDE)
        else:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
            L = C.CDLL(LIB)
        P, I, I64, F, D = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_double
        L.oracle_e4m3_decode.restype = D
        L.oracle_e4m3_decode.argtypes = [C.c_uint8]
        L.oracle_e4m3_encode.restype = C.c_uint8
        L.oracle_e4m3_encode.argtypes = [F]
        L.oracle_bf16_decode.restype = D
        L.oracle_bf16_decode.argtypes = [C.c_uint16]
        L.oracle_bf16_encode.restype = C.c_uint16
        L.oracle_bf16_encode.argtypes = [F]
        L.oracle_bf16_encode_array.argtypes = [P, P, I64]
        L.oracle_e4m3_encode_array.argtypes = [P, P, I64]
        L.oracle_kv_bytes_per_token.restype = I64
        L.oracle_kv_bytes_per_token.argtypes = [I64, I64, I64, I64]
        L.oracle_reshape_and_cache.restype = I
        L.oracle_reshape_and_cache.argtypes = [I, I, I, I, I64, I, P, P, I, P, P, P, F, F]
        L.oracle_decode_attention.restype = I
        L.oracle_decode_attention.argtypes = [I, I, I, I, I, I, I, P, I, P, P, P, P, F, F, F,
                                              P, P, P, I64, I]
        L.oracle_decode_attention_split.restype = I
        L.oracle_decode_attention_split.argtypes = [I, I, I, I, I, I, I, P, I, P, P, P, P, F, F,
                                                    F, I, P, P, I]
        L.oracle_prefill_attention.restype = I
        L.oracle_prefill_attention.argtypes = [I, I, I, I, I, I, I, P, I, P, P, P, P, P, F, F, F,
                                               P, P, I]
        L.oracle_bm_create.restype = P
        L.oracle_bm_create.argtypes = [I, I, I, P]
        L.oracle_bm_destroy.argtypes = [P]
        L.oracle_bm_add_seq.restype = I
        L.oracle_bm_add_seq.argtypes = [P, I64]
        L.oracle_bm_fork_seq.restype = I
        L.oracle_bm_fork_seq.argtypes = [P, I64, I64]
        L.oracle_bm_append_slots.restype = I
        L.oracle_bm_append_slots.argtypes = [P, P, I, P]
        L.oracle_bm_append_slots_cow.restype = I
        L.oracle_bm_append_slots_cow.argtypes = [P, P, I, P, P, P, P]
        L.oracle_bm_free_seq.restype = I
        L.oracle_bm_free_seq.argtypes = [P, I64]
        L.oracle_bm_export.restype = I
        L.oracle_bm_export.argtypes = [P, P, I, P, P]
        L.oracle_bm_num_free.restype = I
        L.oracle_bm_num_free.argtypes = [P]
        L.oracle_bm_refcount.restype = I
        L.oracle_bm_refcount.argtypes = [P, I]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


# ---------------------------------------------------------------- codecs
def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code))


def e4m3_encode(x: float) -> int:
    return int(lib().oracle_e4m3_encode(float(x)))


def bf16_decode(bits: int) -> float:
    return lib().oracle_bf16_decode(int(bits))


def bf16_encode_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_encode_array(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(x), _ptr(out), x.size)
    return out


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    return int(lib().oracle_kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_elem))


# ---------------------------------------------------------------- cache write
def reshape_and_cache(k_new, v_new, src_dtype, k_cache, v_cache, cache_dtype, slot_mapping,
                      block_size, k_scale=1.0, v_scale=1.0):
    """In place on the numpy pools; shapes: k_new/v_new [T][Hkv][D] storage arrays."""
    T, Hkv, D = k_new.shape
    nb = k_cache.shape[0]
    slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    rc = lib().oracle_reshape_and_cache(T, Hkv, D, block_size, nb, src_dtype, _ptr(k_new),
                                        _ptr(v_new), cache_dtype, _ptr(k_cache), _ptr(v_cache),
                                        _ptr(slot_mapping), float(k_scale), float(v_scale))
    if rc != OK:
        raise ValueError(f"oracle_reshape_and_cache failed: {rc}")


def copy_blocks(k_cache, v_cache, src, dst):
    """Block dst[i] of both pools becomes a copy of block src[i], pair by pair
    in order (the copy-on-write pairs)."""
    for a, b in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        k_cache[b] = k_cache[a]
        v_cache[b] = v_cache[a]


# ---------------------------------------------------------------- attention
def decode_attention(q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, context_lens,
                     num_kv_heads, block_size, scale, k_scale=1.0, v_scale=1.0,
                     want_weights=False, threads=0):
    """fp64 attention.  q: [S][Hq][D] storage array.  Returns (out, lse[, weights])."""
    S, Hq, D = q.shape
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    max_blocks = block_tables.shape[1] if block_tables.ndim == 2 else 0
    out = np.zeros((S, Hq, D), dtype=np.float64)
    lse = np.zeros((S, Hq), dtype=np.float64)
    wstride = int(context_lens.max()) if S and context_lens.size else 0
    w = np.zeros((S, Hq, max(wstride, 1)), dtype=np.float64) if want_weights else None
    rc = lib().oracle_decode_attention(
        S, Hq, num_kv_heads, D, block_size, max_blocks, q_dtype, _ptr(q), cache_dtype,
        _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), float(scale),
        float(k_scale), float(v_scale), _ptr(out), _ptr(lse), _ptr(w) if w is not None else None,
        max(wstride, 1), threads)
    if rc != OK:
        raise ValueError(f"oracle_decode_attention failed: {rc}")
    return (out, lse, w) if want_weights else (out, lse)


def decode_attention_split(q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, context_lens,
                           num_kv_heads, block_size, scale, partition_tokens, k_scale=1.0,
                           v_scale=1.0, threads=0):
    S, Hq, D = q.shape
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    lse = np.zeros((S, Hq), dtype=np.float64)
    rc = lib().oracle_decode_attention_split(
        S, Hq, num_kv_heads, D, block_size, block_tables.shape[1], q_dtype, _ptr(q), cache_dtype,
        _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), float(scale),
        float(k_scale), float(v_scale), int(partition_tokens), _ptr(out), _ptr(lse), threads)
    if rc != OK:
        raise ValueError(f"oracle_decode_attention_split failed: {rc}")
    return out, lse


def prefill_attention(q, q_dtype, k_cache, v_cache, cache_dtype, block_tables, context_lens,
                      query_start, num_kv_heads, block_size, scale, k_scale=1.0, v_scale=1.0,
                      threads=0):
    """fp64 chunked-prefill attention.  q: [rows][Hq][D] storage array (rows =
    query_start[-1]).  Returns (out [rows][Hq][D], lse [rows][Hq])."""
    R, Hq, D = q.shape
    S = len(context_lens)
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    query_start = np.ascontiguousarray(query_start, dtype=np.int32)
    assert query_start.shape == (S + 1,) and query_start[-1] == R
    out = np.zeros((R, Hq, D), dtype=np.float64)
    lse = np.zeros((R, Hq), dtype=np.float64)
    rc = lib().oracle_prefill_attention(
        S, Hq, num_kv_heads, D, block_size, block_tables.shape[1], q_dtype, _ptr(q), cache_dtype,
        _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), _ptr(query_start),
        float(scale), float(k_scale), float(v_scale), _ptr(out), _ptr(lse), threads)
    if rc != OK:
        raise ValueError(f"oracle_prefill_attention failed: {rc}")
    return out, lse


# ---------------------------------------------------------------- block allocation
class BlockAllocator:
    """The oracle's FIFO block allocation (free order, refcounts, fork, free)."""

    def __init__(self, num_blocks, block_size, max_blocks_per_seq, free_order=None):
        fo = None
        if free_order is not None:
            self._fo = np.ascontiguousarray(free_order, dtype=np.int32)
            fo = _ptr(self._fo)
        self.max_blocks = max_blocks_per_seq
        self.h = lib().oracle_bm_create(num_blocks, block_size, max_blocks_per_seq, fo)
        if not self.h:
            raise ValueError("oracle_bm_create failed")

    def __del__(self):
        try:
            if getattr(self, "h", None):
                lib().oracle_bm_destroy(self.h)
                self.h = None
        except Exception:  # interpreter shutdown
            pass

    def add_seq(self, sid):
        return lib().oracle_bm_add_seq(self.h, sid)

    def fork_seq(self, parent, child):
        return lib().oracle_bm_fork_seq(self.h, parent, child)

    def append_slots(self, seq_ids):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        slots = np.full(ids.shape, -7, dtype=np.int64)
        rc = lib().oracle_bm_append_slots(self.h, _ptr(ids), ids.size, _ptr(slots))
        return rc, slots

    def append_slots_cow(self, seq_ids):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        slots = np.full(ids.shape, -7, dtype=np.int64)
        src = np.full(max(ids.size, 1), -7, dtype=np.int32)
        dst = np.full(max(ids.size, 1), -7, dtype=np.int32)
        n = np.zeros(1, dtype=np.int32)
        rc = lib().oracle_bm_append_slots_cow(self.h, _ptr(ids), ids.size, _ptr(slots), _ptr(src),
                                              _ptr(dst), _ptr(n))
        k = int(n[0]) if rc == OK else 0
        return rc, slots, src[:k].copy(), dst[:k].copy()

    def free_seq(self, sid):
        return lib().oracle_bm_free_seq(self.h, sid)

    def export(self, seq_ids):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((ids.size, self.max_blocks), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        rc = lib().oracle_bm_export(self.h, _ptr(ids), ids.size, _ptr(tables), _ptr(lens))
        return rc, tables, lens

    def num_free(self):
        return lib().oracle_bm_num_free(self.h)

    def refcount(self, block):
        return lib().oracle_bm_refcount(self.h, block)
