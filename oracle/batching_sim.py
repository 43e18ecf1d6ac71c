"""TEST INFRASTRUCTURE ONLY: the oracle of the continuous-batching
simulation (plain Python over the oracle allocators, small traces).

Only tests/ may import this module.  The scheduler, restated from its
reading ("Optimizing vLLM Throughput with PagedAttention and Continuous
Batching for Llama 3": a request joins the batch as soon as there is room,
max-num-seqs caps the batch; "vLLM PagedAttention: Memory Optimization &
High-Throughput LLM Inference Tuning" §2: static reservation of the maximum
length versus blocks on demand), one iteration at a time:
1. admit requests in queue order while fewer than max_num_seqs run -- paged:
   the request's tokens so far (prompt, plus generated tokens after a
   preemption) are allocated as one prompt; static: the request reserves
   ceil(max_model_len / block_size) blocks -- stopping at the first that
   does not fit;
2. every running request in admission order appends one token; when no
   block is left, the most recently admitted running request is preempted
   (freed, put back at the front of the queue) and the append is retried;
   a request that has generated its output length is freed at once;
3. record the running count, the tokens held and the blocks in use.
Generated token t of request r has id (r * 7919 + t) % 32000.
"""
from __future__ import annotations

from collections import deque

import numpy as np

from oracle import oracle as O
from oracle.prefix_cache import PrefixCacheAllocator

PAGED, STATIC = 0, 1


def gen_id(r, t):
    return (r * 7919 + t) % 32000


def simulate(num_blocks, block_size, max_model_len, max_num_seqs, policy, prompt_lens,
             output_lens, prompt_ids=None, prefix_cache=False, max_iters=1 << 20):
    BS, NB = block_size, num_blocks
    R = len(prompt_lens)
    mb = -(-max_model_len // BS)
    paged = policy == PAGED
    cache = paged and prefix_cache
    if not paged and mb > NB:
        raise ValueError("one static reservation does not fit the pool")
    offs = np.concatenate([[0], np.cumsum(prompt_lens)]).astype(int)
    prompts = [list(prompt_ids[offs[r]:offs[r + 1]]) if prompt_ids is not None
               else [0] * int(prompt_lens[r]) for r in range(R)]
    gen = [0] * R
    if cache:
        A = PrefixCacheAllocator(NB, BS, mb)
    elif paged:
        A = O.BlockAllocator(NB, BS, mb)
    waiting = deque(range(R))
    running = []
    alive = [False] * R
    reserved = 0
    it = done = generated = preempt = peak = 0
    admitted = cached = 0
    sum_run = sum_util = 0.0
    trace = []

    def tokens(r):
        return int(prompt_lens[r]) + gen[r]

    def free(r):
        nonlocal reserved
        if paged:
            A.free_seq(r)
        else:
            reserved -= mb

    while done < R:
        if it >= max_iters:
            raise RuntimeError("max_iters reached")
        while waiting and len(running) < max_num_seqs:
            r = waiting[0]
            n = tokens(r)
            if paged:
                ids = prompts[r] + [gen_id(r, t) for t in range(gen[r])]
                if cache:
                    rc, _, c = A.add_seq_prompt(r, ids)
                else:
                    A.add_seq(r)
                    rc, _ = A.append_slots([r] * n)
                    if rc != 0:
                        A.free_seq(r)
                    c = 0
                if rc == O.OUT_OF_BLOCKS:
                    break
                assert rc == 0, rc
                cached += c
            else:
                if reserved + mb > NB:
                    break
                reserved += mb
            admitted += n
            waiting.popleft()
            alive[r] = True
            running.append(r)
        nxt = []
        for r in running:
            if not alive[r]:
                continue
            ok = not paged
            while paged:
                if cache:
                    rc, _ = A.append([r], [gen_id(r, gen[r])])
                else:
                    rc, _ = A.append_slots([r])
                if rc == 0:
                    ok = True
                    break
                assert rc == O.OUT_OF_BLOCKS, rc
                victim = [x for x in running if alive[x]][-1]
                free(victim)
                alive[victim] = False
                waiting.appendleft(victim)
                preempt += 1
                if victim == r:
                    break
            if not ok:
                continue
            gen[r] += 1
            generated += 1
            if gen[r] == int(output_lens[r]):
                free(r)
                alive[r] = False
                done += 1
            else:
                nxt.append(r)
        running = nxt
        held = sum(tokens(r) for r in running)
        if paged:
            used = NB - (A.available() if cache else A.num_free())
        else:
            used = reserved
        trace.append(len(running))
        sum_run += len(running)
        sum_util += held / (used * BS) if used > 0 else 0.0
        peak = max(peak, len(running))
        it += 1
    res = dict(iterations=it, generated_tokens=generated, preemptions=preempt, peak_running=peak,
               mean_running=sum_run / it if it else 0.0,
               mean_kv_utilization=sum_util / it if it else 0.0, admitted_tokens=admitted,
               cached_tokens=cached)
    return res, np.array(trace, dtype=np.int32)
