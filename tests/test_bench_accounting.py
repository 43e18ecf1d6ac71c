"""CPU tests of the benchmark's algorithmic byte count (no GPU).

The decode metric counts the KV bytes the method must move: the tokens used in
every physical block the step touches, each block once, times 2 (K and V) x
kv heads x head dim x element size.  Blocks shared by a common prefix count
once; the logical figure counts them per sequence.  Checked here against
totals written out by hand for small tables, including a shared prefix, a
partially filled last block and an fp8 cache.
"""
import dataclasses
import os

import numpy as np

import bench
import workloads


def spec_of(cache_dtype, Hkv=8, D=128, Hq=64):
    return dataclasses.replace(workloads.SPECS[3], num_kv_heads=Hkv, head_dim=D, num_q_heads=Hq,
                               cache_dtype=cache_dtype, block_size=16)


def test_private_blocks_count_every_token():
    spec = spec_of(workloads.BF16)
    lens = np.array([16, 17, 1])
    tables = np.array([[5, -1], [7, 2], [9, -1]], dtype=np.int32)
    per_tok = 2 * 8 * 128 * 2
    unique, logical = bench.kv_bytes(spec, tables, lens)
    assert unique == logical == (16 + 17 + 1) * per_tok


def test_shared_prefix_counts_once():
    # three sequences share blocks 3 and 4 (a 32-token prefix); suffixes are private
    spec = spec_of(workloads.BF16)
    lens = np.array([40, 33, 64])
    tables = np.array([[3, 4, 10, -1], [3, 4, 11, -1], [3, 4, 12, 13]], dtype=np.int32)
    per_tok = 2 * 8 * 128 * 2
    unique, logical = bench.kv_bytes(spec, tables, lens)
    assert logical == (40 + 33 + 64) * per_tok
    assert unique == (32 + 8 + 1 + 32) * per_tok


def test_shared_partial_block_counts_its_fullest_use():
    # a block shared while partially filled (before a copy-on-write) is read
    # up to the longest sequence's use of it
    spec = spec_of(workloads.BF16)
    lens = np.array([20, 25])
    tables = np.array([[6, 8], [6, 8]], dtype=np.int32)
    per_tok = 2 * 8 * 128 * 2
    unique, logical = bench.kv_bytes(spec, tables, lens)
    assert unique == 25 * per_tok
    assert logical == 45 * per_tok


def test_fp8_cache_is_one_byte_per_element():
    spec = spec_of(workloads.E4M3)
    lens = np.array([100])
    tables = np.arange(7, dtype=np.int32)[None, :]
    unique, _ = bench.kv_bytes(spec, tables, lens)
    assert unique == 100 * 2 * 8 * 128 * 1


def test_other_bytes_are_q_out_tables_and_lengths():
    spec = dataclasses.replace(workloads.SPECS[2], block_size=16)   # bf16 q and out
    lens = [1, 16, 17]
    S, Hq, D = 3, spec.num_q_heads, spec.head_dim
    want = S * Hq * D * (2 + 2) + 4 * (1 + 1 + 2) + 4 * S
    assert bench.other_bytes(spec, lens) == want


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=root, capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
