"""TEST INFRASTRUCTURE ONLY: the oracle of block allocation with automatic
prefix caching (plain Python, small cases).

Only tests/ may import this module.  It restates the reading the library's
block manager implements, without its hashing: a full block of a sequence
with known token ids is cached under the tuple of ALL token ids from the
sequence start to the block's end (the key fixes the block's K and V), and
a new prompt reuses the cached block of each of its full-block prefixes in
turn, stopping at the first prefix that is not cached and never reusing the
block holding the prompt's last token.

Reading of what the pages leave open ("Optimizing Llama 3.1 405B Inference
with vLLM PagedAttention", production settings, and "vLLM PagedAttention
Optimization: Complete Step-by-Step Tuning Guide", Step 2, only turn prefix
caching on):
- free blocks form a FIFO queue seeded with a given order;
- a block is cached when it becomes full, if the block before it in the
  same table is the cached block of that shorter prefix (or it is block 0)
  and no block is cached for its prefix yet;
- a cached block whose reference count drops to 0 waits in an LRU list
  (release order); other blocks rejoin the free queue's tail;
- a new block comes from the free queue's head; if the queue is empty the
  least recently released cached block is evicted first: it and every cached
  block whose prefix extends its prefix (its descendants, children in the
  order they were cached, depth first) leave the cache and the unreferenced
  ones join the free queue, the evicted block first;
- a sequence that receives a token without its id stops being cached from
  then on; appending into a partially filled shared block is refused
  (SHARED_TAIL), as in the allocator without caching.
"""
from __future__ import annotations

from collections import OrderedDict, deque

OK, INVALID, OUT_OF_BLOCKS, UNKNOWN_SEQ, SEQ_EXISTS, SHARED_TAIL = 0, -1, -2, -3, -4, -5


class PrefixCacheAllocator:
    def __init__(self, num_blocks, block_size, max_blocks_per_seq, free_order=None):
        self.BS = block_size
        self.max_blocks = max_blocks_per_seq
        self.free = deque(int(b) for b in (free_order if free_order is not None
                                           else range(num_blocks)))
        self.ref = [0] * num_blocks
        self.key_of = {}        # cached block -> prefix tuple
        self.block_of = {}      # prefix tuple -> cached block
        self.children = {}      # cached block -> cached blocks one block longer, in caching order
        self.lru = OrderedDict()  # unreferenced cached blocks, oldest first
        self.seqs = {}          # id -> dict(len, table, tokens or None)

    # ---------------------------------------------------------------- helpers
    def available(self):
        return len(self.free) + len(self.lru)

    def _uncache(self, b):
        key = self.key_of.pop(b)
        del self.block_of[key]
        if b in self.lru:
            del self.lru[b]
            self.free.append(b)
        for c in self.children.pop(b, []):
            self._uncache(c)

    def _pop(self):
        if not self.free:
            victim = next(iter(self.lru))
            key = self.key_of[victim]
            parent = self.block_of.get(key[:-self.BS]) if len(key) > self.BS else None
            if parent is not None:
                self.children[parent].remove(victim)
            self._uncache(victim)
        return self.free.popleft()

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.lru[b] = None
            else:
                self.free.append(b)

    def _acquire(self, b):
        if self.ref[b] == 0:
            self.lru.pop(b, None)
        self.ref[b] += 1

    def _register(self, q, i):
        b = q["table"][i]
        if b in self.key_of:
            return
        if i > 0 and q["table"][i - 1] not in self.key_of:
            return
        key = tuple(q["tokens"][: (i + 1) * self.BS])
        if key in self.block_of:
            return
        self.key_of[b] = key
        self.block_of[key] = b
        self.children[b] = []
        if i > 0:
            self.children[q["table"][i - 1]].append(b)

    # ---------------------------------------------------------------- calls
    def add_seq_prompt(self, sid, tokens):
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        if sid in self.seqs:
            return SEQ_EXISTS, [], 0
        nblk = -(-n // self.BS)
        if nblk > self.max_blocks:
            return INVALID, [], 0
        hit = []
        for i in range((n - 1) // self.BS if n > 0 else 0):
            b = self.block_of.get(tuple(tokens[: (i + 1) * self.BS]))
            if b is None:
                break
            hit.append(b)
        from_lru = sum(1 for b in hit if self.ref[b] == 0)
        if nblk - len(hit) > self.available() - from_lru:
            return OUT_OF_BLOCKS, [], 0
        q = dict(len=0, table=[], tokens=[])
        for b in hit:
            self._acquire(b)
            q["table"].append(b)
        cached = len(hit) * self.BS
        q["tokens"] = tokens[:cached]
        q["len"] = cached
        self.seqs[sid] = q
        slots = [q["table"][t // self.BS] * self.BS + t % self.BS for t in range(cached)]
        for t in range(cached, n):
            if t % self.BS == 0:
                b = self._pop()
                self.ref[b] = 1
                q["table"].append(b)
            slots.append(q["table"][t // self.BS] * self.BS + t % self.BS)
            q["tokens"].append(tokens[t])
            q["len"] = t + 1
            if (t + 1) % self.BS == 0:
                self._register(q, t // self.BS)
        return OK, slots, cached

    def add_seq(self, sid):
        if sid in self.seqs:
            return SEQ_EXISTS
        self.seqs[sid] = dict(len=0, table=[], tokens=None)
        return OK

    def fork_seq(self, parent, child):
        if parent not in self.seqs:
            return UNKNOWN_SEQ
        if child in self.seqs:
            return SEQ_EXISTS
        p = self.seqs[parent]
        for b in p["table"]:
            self.ref[b] += 1
        self.seqs[child] = dict(len=p["len"], table=list(p["table"]),
                                tokens=None if p["tokens"] is None else list(p["tokens"]))
        return OK

    def append(self, sids, tokens=None):
        """tokens None: ids unknown (the sequences stop being cached)."""
        pending, need = {}, 0
        for sid in sids:
            if sid not in self.seqs:
                return UNKNOWN_SEQ, []
            q = self.seqs[sid]
            extra = pending.get(sid, 0)
            p = q["len"] + extra
            if p // self.BS >= self.max_blocks:
                return INVALID, []
            if p % self.BS == 0:
                need += 1
            elif extra == 0 and self.ref[q["table"][p // self.BS]] > 1:
                return SHARED_TAIL, []
            pending[sid] = extra + 1
        if need > self.available():
            return OUT_OF_BLOCKS, []
        slots = []
        for k, sid in enumerate(sids):
            q = self.seqs[sid]
            p = q["len"]
            if p % self.BS == 0:
                b = self._pop()
                self.ref[b] = 1
                q["table"].append(b)
            slots.append(q["table"][p // self.BS] * self.BS + p % self.BS)
            q["len"] = p + 1
            if tokens is not None and q["tokens"] is not None:
                q["tokens"].append(int(tokens[k]))
                if (p + 1) % self.BS == 0:
                    self._register(q, p // self.BS)
            else:
                q["tokens"] = None
        return OK, slots

    def free_seq(self, sid):
        if sid not in self.seqs:
            return UNKNOWN_SEQ
        for b in self.seqs.pop(sid)["table"]:
            self._release(b)
        return OK

    def table(self, sid):
        return list(self.seqs[sid]["table"]), self.seqs[sid]["len"]

    def num_cached(self):
        return len(self.key_of)
