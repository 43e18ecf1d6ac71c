"""Python binding of libpkv (include/pkv.h): paged KV-cache decode attention
for AMD MI355X (gfx950).

Argument marshalling only.  Every function keeps its C name; tensors are
passed as ``data_ptr()`` plus their dtype code, and device calls are
enqueued on torch's current HIP stream unless a stream is given.  Nothing
here computes: all device work runs in the HIP kernels of libpkv.so, and a
missing library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIB names another build of the library (a variant built with
# `python -m paged_kv_cache_189_amd.build --define ... --out ...`).
LIB_PATH = os.environ.get("PKV_LIB") or os.path.join(HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_OUT_OF_BLOCKS = -2
PKV_ERR_UNKNOWN_SEQ = -3
PKV_ERR_SEQ_EXISTS = -4
PKV_ERR_SHARED_TAIL = -5
PKV_ERR_UNSUPPORTED = -6
PKV_ERR_HIP = -7

PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2

# every symbol include/pkv.h declares
EXPORTED = (
    "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_add_seq", "pkv_bm_fork_seq",
    "pkv_bm_append_slots", "pkv_bm_append_slots_cow", "pkv_bm_add_seq_prompt",
    "pkv_bm_append_tokens", "pkv_bm_num_cached_blocks", "pkv_bm_free_seq", "pkv_bm_export",
    "pkv_bm_num_free_blocks", "pkv_bm_refcount", "pkv_reshape_and_cache",
    "pkv_append_decode_tokens", "pkv_copy_blocks",
    "pkv_decode_workspace_bytes",
    "pkv_decode_partition_size", "pkv_decode_num_ranges", "pkv_decode_attention",
    "pkv_decode_attention_noalloc", "pkv_decode_attention_partitions",
    "pkv_decode_attention_merge", "pkv_prefill_attention", "pkv_sim_run", "pkv_status_string",
    "pkv_last_error", "pkv_version", "pkv_read_probe",
)


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = ""
        try:
            msg = _lib.pkv_last_error().decode()
        except Exception:
            pass
        super().__init__(f"{where}: {_status_name(status)} ({status}): {msg}")


class pkv_decode_params(C.Structure):
    _fields_ = [
        ("num_seqs", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("block_size", C.c_int32), ("max_blocks_per_seq", C.c_int32),
        ("max_context_len", C.c_int32), ("partition_size", C.c_int32), ("num_blocks", C.c_int64),
        ("scale", C.c_float), ("k_scale", C.c_float), ("v_scale", C.c_float),
        ("q_dtype", C.c_int32), ("cache_dtype", C.c_int32), ("out_dtype", C.c_int32),
    ]


class pkv_prefill_params(C.Structure):
    _fields_ = [
        ("num_seqs", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("block_size", C.c_int32), ("max_blocks_per_seq", C.c_int32),
        ("max_context_len", C.c_int32), ("num_query_tokens", C.c_int32), ("num_blocks", C.c_int64),
        ("scale", C.c_float), ("k_scale", C.c_float), ("v_scale", C.c_float),
        ("q_dtype", C.c_int32), ("cache_dtype", C.c_int32), ("out_dtype", C.c_int32),
    ]


class pkv_sim_config(C.Structure):
    _fields_ = [("num_blocks", C.c_int32), ("block_size", C.c_int32),
                ("max_model_len", C.c_int32), ("max_num_seqs", C.c_int32),
                ("policy", C.c_int32), ("prefix_cache", C.c_int32)]


class pkv_sim_result(C.Structure):
    _fields_ = [("iterations", C.c_int64), ("generated_tokens", C.c_int64),
                ("preemptions", C.c_int64), ("peak_running", C.c_int64),
                ("mean_running", C.c_double), ("mean_kv_utilization", C.c_double),
                ("admitted_tokens", C.c_int64), ("cached_tokens", C.c_int64)]


PKV_SIM_PAGED, PKV_SIM_STATIC = 0, 1

_lib = None


def lib():
    """The loaded libpkv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_189_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I32, I64, F = C.c_void_p, C.c_int32, C.c_int64, C.c_float
        st = C.c_int
        sig = {
            "pkv_bm_create": (st, [I32, I32, I32, P, C.POINTER(P)]),
            "pkv_bm_destroy": (None, [P]),
            "pkv_bm_add_seq": (st, [P, I64]),
            "pkv_bm_fork_seq": (st, [P, I64, I64]),
            "pkv_bm_append_slots": (st, [P, P, I32, P]),
            "pkv_bm_append_slots_cow": (st, [P, P, I32, P, P, P, P]),
            "pkv_bm_add_seq_prompt": (st, [P, I64, P, I32, P, P]),
            "pkv_bm_append_tokens": (st, [P, P, P, I32, P]),
            "pkv_bm_num_cached_blocks": (I32, [P]),
            "pkv_bm_free_seq": (st, [P, I64]),
            "pkv_bm_export": (st, [P, P, I32, P, P]),
            "pkv_bm_num_free_blocks": (I32, [P]),
            "pkv_bm_refcount": (I32, [P, I32]),
            "pkv_reshape_and_cache": (st, [P, P, st, P, P, st, P, I32, I32, I32, I32, I64, F, F, P]),
            "pkv_append_decode_tokens": (st, [P, P, st, P, P, st, P, P, P, I32, I32, I32, I32, I32,
                                              I64, F, F, P]),
            "pkv_copy_blocks": (st, [P, P, st, P, P, I32, I32, I32, I32, I64, P]),
            "pkv_decode_workspace_bytes": (C.c_size_t, [C.POINTER(pkv_decode_params)]),
            "pkv_decode_partition_size": (I32, [C.POINTER(pkv_decode_params)]),
            "pkv_decode_num_ranges": (I32, [C.POINTER(pkv_decode_params)]),
            "pkv_decode_attention": (st, [C.POINTER(pkv_decode_params), P, P, P, P, P, P, P,
                                          C.c_size_t, P, P]),
            "pkv_decode_attention_noalloc": (st, [C.POINTER(pkv_decode_params), P, P, P, P, P,
                                                  P, P, P]),
            "pkv_decode_attention_partitions": (st, [C.POINTER(pkv_decode_params), P, P, P, P, P,
                                                     P, P, C.c_size_t, P, P]),
            "pkv_decode_attention_merge": (st, [C.POINTER(pkv_decode_params), P, P, P, C.c_size_t,
                                                P, P]),
            "pkv_prefill_attention": (st, [C.POINTER(pkv_prefill_params), P, P, P, P, P, P, P,
                                           P, P]),
            "pkv_sim_run": (st, [C.POINTER(pkv_sim_config), P, P, P, I32,
                                 C.POINTER(pkv_sim_result), P, I64]),
            "pkv_status_string": (C.c_char_p, [st]),
            "pkv_last_error": (C.c_char_p, []),
            "pkv_version": (C.c_char_p, []),
            "pkv_read_probe": (st, [P, I64, I32, P, I64, I64, P, I32, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().pkv_status_string(s).decode()
    except Exception:
        return str(s)


def _check(status: int, where: str):
    if status != PKV_OK:
        raise PkvError(status, where)


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return PKV_F32
    if t == torch.bfloat16:
        return PKV_BF16
    if t in (torch.uint8, torch.float8_e4m3fn):
        return PKV_FP8_E4M3
    raise TypeError(f"no pkv dtype for {t}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("pkv arguments must be contiguous")
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if t is not None and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


# ------------------------------------------------------------------ block manager
class BlockManager:
    """The host block manager (pkv_bm_*): tables, refcounts, FIFO free list."""

    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int,
                 free_order: Optional[np.ndarray] = None):
        h = C.c_void_p()
        fo = None
        if free_order is not None:
            fo_arr = np.ascontiguousarray(free_order, dtype=np.int32)
            fo = fo_arr.ctypes.data
        _check(lib().pkv_bm_create(num_blocks, block_size, max_blocks_per_seq, fo, C.byref(h)),
               "pkv_bm_create")
        self.h = h
        self.block_size = block_size
        self.max_blocks = max_blocks_per_seq
        self.num_blocks = num_blocks

    def close(self):
        if getattr(self, "h", None):
            lib().pkv_bm_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass

    # raw status codes (the allocation recipe and the tests read them)
    def add_seq(self, seq_id: int) -> int:
        return lib().pkv_bm_add_seq(self.h, seq_id)

    def fork_seq(self, parent: int, child: int) -> int:
        return lib().pkv_bm_fork_seq(self.h, parent, child)

    def append_slots(self, seq_ids, out: Optional[np.ndarray] = None):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        slots = out if out is not None else np.empty(ids.shape, dtype=np.int64)
        rc = lib().pkv_bm_append_slots(self.h, ids.ctypes.data, ids.size, slots.ctypes.data)
        return rc, slots

    def append_slots_cow(self, seq_ids, out: Optional[np.ndarray] = None):
        """Returns (status, slots, copy_src, copy_dst): the copy-on-write pairs
        the caller must copy on the device before writing the tokens."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        slots = out if out is not None else np.empty(ids.shape, dtype=np.int64)
        src = np.empty(max(ids.size, 1), dtype=np.int32)
        dst = np.empty(max(ids.size, 1), dtype=np.int32)
        n = C.c_int32(0)
        rc = lib().pkv_bm_append_slots_cow(self.h, ids.ctypes.data, ids.size, slots.ctypes.data,
                                           src.ctypes.data, dst.ctypes.data, C.byref(n))
        k = n.value if rc == PKV_OK else 0
        return rc, slots, src[:k].copy(), dst[:k].copy()

    def add_seq_prompt(self, seq_id: int, token_ids):
        """Returns (status, slots of every prompt token, number of cached tokens)."""
        ids = np.ascontiguousarray(token_ids, dtype=np.int32)
        slots = np.empty(max(ids.size, 1), dtype=np.int64)
        n = C.c_int32(0)
        rc = lib().pkv_bm_add_seq_prompt(self.h, seq_id, ids.ctypes.data, ids.size,
                                         slots.ctypes.data, C.byref(n))
        return rc, slots[:ids.size].copy(), n.value

    def append_tokens(self, seq_ids, token_ids, out: Optional[np.ndarray] = None):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tok = np.ascontiguousarray(token_ids, dtype=np.int32)
        if tok.shape != ids.shape:
            raise ValueError("one token id per appended token")
        slots = out if out is not None else np.empty(ids.shape, dtype=np.int64)
        rc = lib().pkv_bm_append_tokens(self.h, ids.ctypes.data, tok.ctypes.data, ids.size,
                                        slots.ctypes.data)
        return rc, slots

    def num_cached(self) -> int:
        return lib().pkv_bm_num_cached_blocks(self.h)

    def free_seq(self, seq_id: int) -> int:
        return lib().pkv_bm_free_seq(self.h, seq_id)

    def export(self, seq_ids, tables: Optional[np.ndarray] = None,
               lens: Optional[np.ndarray] = None):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        if tables is None:
            tables = np.empty((ids.size, self.max_blocks), dtype=np.int32)
        if lens is None:
            lens = np.empty(ids.size, dtype=np.int32)
        rc = lib().pkv_bm_export(self.h, ids.ctypes.data, ids.size, tables.ctypes.data,
                                 lens.ctypes.data)
        return rc, tables, lens

    def num_free(self) -> int:
        return lib().pkv_bm_num_free_blocks(self.h)

    def refcount(self, block: int) -> int:
        return lib().pkv_bm_refcount(self.h, block)


# ------------------------------------------------------------------ device ops
def pkv_reshape_and_cache(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float = 1.0,
                          v_scale: float = 1.0, stream=None):
    """k_new, v_new: [T][Hkv][D]; caches in the pool layout; slot_mapping int64 [T]."""
    T, Hkv, D = k_new.shape
    _check(lib().pkv_reshape_and_cache(
        _ptr(k_new), _ptr(v_new), dtype_code(k_new.dtype), _ptr(k_cache), _ptr(v_cache),
        dtype_code(k_cache.dtype), _ptr(slot_mapping), T, Hkv, D, k_cache.shape[3], k_cache.shape[0],
        float(k_scale), float(v_scale), _stream(stream, k_cache)), "pkv_reshape_and_cache")


def pkv_append_decode_tokens(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                             v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                             context_lens: torch.Tensor, block_tables: torch.Tensor,
                             k_scale: float = 1.0, v_scale: float = 1.0, stream=None):
    """Decode append: k_new, v_new [S][Hkv][D] (token i = sequence i's newest,
    at position context_lens[i] - 1); writes them into their slots and sets
    block_tables[i][(context_lens[i] - 1) // block_size] = slot_mapping[i] // block_size."""
    S, Hkv, D = k_new.shape
    if block_tables.dim() != 2 or block_tables.shape[0] < S:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    _check(lib().pkv_append_decode_tokens(
        _ptr(k_new), _ptr(v_new), dtype_code(k_new.dtype), _ptr(k_cache), _ptr(v_cache),
        dtype_code(k_cache.dtype), _ptr(slot_mapping), _ptr(context_lens), _ptr(block_tables),
        block_tables.shape[1], S, Hkv, D, k_cache.shape[3], k_cache.shape[0], float(k_scale),
        float(v_scale), _stream(stream, k_cache)), "pkv_append_decode_tokens")


def pkv_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, src: torch.Tensor,
                    dst: torch.Tensor, stream=None):
    """Copies physical blocks src[i] -> dst[i] (device int32 arrays) of both caches."""
    n = src.numel()
    if dst.numel() != n:
        raise ValueError("src and dst differ in length")
    _check(lib().pkv_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache.dtype), _ptr(src), _ptr(dst), n,
        k_cache.shape[1], v_cache.shape[2], k_cache.shape[3], k_cache.shape[0],
        _stream(stream, k_cache)),
        "pkv_copy_blocks")


def make_decode_params(q: torch.Tensor, k_cache: torch.Tensor, block_tables: torch.Tensor,
                       max_context_len: int, scale: float, k_scale: float = 1.0,
                       v_scale: float = 1.0, out_dtype: Optional[torch.dtype] = None,
                       partition_size: int = 0) -> pkv_decode_params:
    S, Hq, D = q.shape
    p = pkv_decode_params()
    p.num_seqs, p.num_q_heads, p.num_kv_heads, p.head_dim = S, Hq, k_cache.shape[1], D
    p.block_size = k_cache.shape[3]  # [num_blocks][Hkv][D / X][block_size][X]
    p.max_blocks_per_seq = block_tables.shape[1]
    p.max_context_len = int(max_context_len)
    p.partition_size = int(partition_size)
    p.num_blocks = k_cache.shape[0]
    p.scale, p.k_scale, p.v_scale = float(scale), float(k_scale), float(v_scale)
    p.q_dtype = dtype_code(q.dtype)
    p.cache_dtype = dtype_code(k_cache.dtype)
    p.out_dtype = dtype_code(out_dtype if out_dtype is not None else q.dtype)
    return p


def pkv_decode_workspace_bytes(params: pkv_decode_params) -> int:
    return int(lib().pkv_decode_workspace_bytes(C.byref(params)))


def pkv_decode_partition_size(params: pkv_decode_params) -> int:
    return int(lib().pkv_decode_partition_size(C.byref(params)))


def pkv_decode_num_ranges(params: pkv_decode_params) -> int:
    """Pass-1 ranges on the current device (raises on invalid params)."""
    r = int(lib().pkv_decode_num_ranges(C.byref(params)))
    if r < 0:
        raise PkvError(PKV_ERR_INVALID_ARG, "pkv_decode_num_ranges")
    return r


def _ws(workspace):
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def pkv_decode_attention(params: pkv_decode_params, out: torch.Tensor, q: torch.Tensor,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, stream=None):
    wp, wb = _ws(workspace)
    _check(lib().pkv_decode_attention(
        C.byref(params), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), wp, wb, _ptr(lse), _stream(stream, out)), "pkv_decode_attention")


PKV_NOALLOC_SCRATCH_BYTES = 64 << 20


def pkv_decode_attention_noalloc(params: pkv_decode_params, out: torch.Tensor, q: torch.Tensor,
                                 k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 block_tables: torch.Tensor, context_lens: torch.Tensor,
                                 lse: Optional[torch.Tensor] = None, stream=None):
    """pkv_decode_attention without a workspace: the library's own scratch of
    the current device holds the partial states (calls on one device must be
    ordered on one stream)."""
    _check(lib().pkv_decode_attention_noalloc(
        C.byref(params), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(lse), _stream(stream, out)), "pkv_decode_attention_noalloc")


def pkv_decode_attention_partitions(params, out, q, k_cache, v_cache, block_tables,
                                    context_lens, workspace=None, lse=None, stream=None):
    wp, wb = _ws(workspace)
    _check(lib().pkv_decode_attention_partitions(
        C.byref(params), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), wp, wb, _ptr(lse), _stream(stream, out)),
        "pkv_decode_attention_partitions")


def pkv_decode_attention_merge(params, out, context_lens, workspace=None, lse=None, stream=None):
    wp, wb = _ws(workspace)
    _check(lib().pkv_decode_attention_merge(
        C.byref(params), _ptr(out), _ptr(context_lens), wp, wb, _ptr(lse),
        _stream(stream, out)), "pkv_decode_attention_merge")


def pkv_read_probe(buf: torch.Tensor, mode: int, sink: torch.Tensor,
                   order: Optional[torch.Tensor] = None, tile_bytes: int = 0, grid: int = 0,
                   stream=None):
    """Read-bandwidth probe over buf (mode 0 sweep, 1 non-temporal sweep, 2
    tiles in `order`); sink: int32 tensor of grid * 256 words."""
    nbytes = buf.numel() * buf.element_size()
    grid = grid or sink.numel() // 256
    tiles = order.numel() if order is not None else 0
    _check(lib().pkv_read_probe(_ptr(buf), nbytes, int(mode), _ptr(order), int(tile_bytes), tiles,
                                _ptr(sink), int(grid), _stream(stream, buf)), "pkv_read_probe")


def pkv_version() -> str:
    return lib().pkv_version().decode()


# ------------------------------------------------------------------ chunked prefill
def make_prefill_params(q: torch.Tensor, k_cache: torch.Tensor, block_tables: torch.Tensor,
                        num_seqs: int, max_context_len: int, scale: float, k_scale: float = 1.0,
                        v_scale: float = 1.0,
                        out_dtype: Optional[torch.dtype] = None) -> pkv_prefill_params:
    R, Hq, D = q.shape
    p = pkv_prefill_params()
    p.num_seqs, p.num_q_heads, p.num_kv_heads, p.head_dim = num_seqs, Hq, k_cache.shape[1], D
    p.block_size = k_cache.shape[3]
    p.max_blocks_per_seq = block_tables.shape[1]
    p.max_context_len = int(max_context_len)
    p.num_query_tokens = R
    p.num_blocks = k_cache.shape[0]
    p.scale, p.k_scale, p.v_scale = float(scale), float(k_scale), float(v_scale)
    p.q_dtype = dtype_code(q.dtype)
    p.cache_dtype = dtype_code(k_cache.dtype)
    p.out_dtype = dtype_code(out_dtype if out_dtype is not None else q.dtype)
    return p


def pkv_prefill_attention(params: pkv_prefill_params, out: torch.Tensor, q: torch.Tensor,
                          k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_tables: torch.Tensor, context_lens: torch.Tensor,
                          query_start: torch.Tensor, lse: Optional[torch.Tensor] = None,
                          stream=None):
    _check(lib().pkv_prefill_attention(
        C.byref(params), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start), _ptr(lse), _stream(stream, out)),
        "pkv_prefill_attention")


# ------------------------------------------------------------------ batching simulation
def pkv_sim_run(num_blocks, block_size, max_model_len, max_num_seqs, policy, prompt_lens,
                output_lens, prompt_ids=None, prefix_cache=False, max_iters=1 << 22,
                want_trace=False):
    """Returns (status, result dict, running count per iteration or None)."""
    cfg = pkv_sim_config(num_blocks, block_size, max_model_len, max_num_seqs, policy,
                         1 if prefix_cache else 0)
    pl = np.ascontiguousarray(prompt_lens, dtype=np.int32)
    ol = np.ascontiguousarray(output_lens, dtype=np.int32)
    ids = None if prompt_ids is None else np.ascontiguousarray(prompt_ids, dtype=np.int32)
    res = pkv_sim_result()
    trace = np.zeros(max_iters, dtype=np.int32) if want_trace else None
    rc = lib().pkv_sim_run(C.byref(cfg), pl.ctypes.data, ol.ctypes.data,
                           None if ids is None else ids.ctypes.data, pl.size, C.byref(res),
                           None if trace is None else trace.ctypes.data, max_iters)
    out = {name: getattr(res, name) for name, _ in pkv_sim_result._fields_}
    if trace is not None and rc == PKV_OK:
        trace = trace[: res.iterations].copy()
    return rc, out, trace
