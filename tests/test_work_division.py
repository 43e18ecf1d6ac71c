"""CPU model of the decode kernels' work division (no GPU).

The pass-1 kernel cuts the line of all (kv head, sequence) pairs, head major,
into R equal ranges of 16-token tiles, one per wave; segments are the pieces
between pair starts, range starts and (with split-KV partitions) partition
cuts.  A segment either finishes its pair (final row) or leaves a partial
state in slot K(x) + range(x); with folding, the first piece of a pair in a
range that is not first in its workgroup of four is handed to the previous
wave in LDS and leaves nothing.  Pass 2 must read exactly the partial states
of each pair: the one-wave-per-row merge (no partition cuts) from range
indices alone, the four-wave merge (partition cuts) per partition item.

This model restates those integer rules in Python and checks, over random
batches and the benchmark workloads' own length draws, that every tile is
covered once, slots are unique and below the workspace bound, unfinished
pairs are read back from exactly the slots written for them, and finished
pairs are written once.  The kernels' own index arithmetic is exercised on
the GPU by the parity tests; this pins the rules they implement.
"""
import random

import numpy as np
import pytest

import workloads

NW = 4  # waves per pass-1 workgroup


def range_start(r, total, R):
    return r * total // R


def range_of(x, total, R):
    return ((x + 1) * R + total - 1) // total - 1


def plan(nblocks, pb):
    cb = [0]
    cp = [0]
    for n in nblocks:
        cb.append(cb[-1] + n)
        parts = (n + pb - 1) // pb if pb > 0 else (1 if n > 0 else 0)
        cp.append(cp[-1] + parts)
    return cb, cp


def pass1(nblocks, H, R, pb):
    """Partial slots written (slot -> pair), final rows (pair -> count) and
    tiles covered (pair -> count per tile), as pass 1 does them."""
    S = len(nblocks)
    cb, cp = plan(nblocks, pb)
    T, PT = cb[S], cp[S]
    total = T * H
    partial, final = {}, {}
    covered = {}
    events = []  # (range, pair, 'publish' | 'absorb')
    segs = []  # (range, pair, lo, hi): the tiles [lo, hi) of the pair this range takes
    fold_on = pb == 0 and total >= R
    for rg in range(R):
        w = rg % NW
        x, x1 = range_start(rg, total, R), range_start(rg + 1, total, R)
        if x >= x1:
            continue
        x_first = x
        g = x // T
        s = max(i for i in range(S) if cb[i] <= x - g * T)
        while x < x1 and g < H:
            ps = g * T + cb[s]
            nblk = cb[s + 1] - cb[s]
            if ps + nblk <= x:
                s += 1
                if s == S:
                    s, g = 0, g + 1
                continue
            lo = x - ps
            hi = min(nblk, x1 - ps)
            pe = ps + nblk
            segs.append((rg, (g, s), lo, hi))
            cov = covered.setdefault((g, s), np.zeros(nblk, dtype=np.int64))
            cov[lo:hi] += 1
            publish = fold_on and x == x_first and lo > 0 and w != 0
            absorb = fold_on and ps + hi == x1 and hi < nblk and w != NW - 1
            if publish:
                events.append((rg, (g, s), "publish"))
            if absorb:
                events.append((rg, (g, s), "absorb"))
            if fold_on:
                whole = lo == 0 and range_of(pe - 1, total, R) // NW == rg // NW
            else:
                whole = lo == 0 and hi == nblk and (pb == 0 or nblk <= pb)
            slot = g * PT + cp[s] + (lo // pb if pb > 0 else 0) + rg
            if whole:
                final[(g, s)] = final.get((g, s), 0) + 1
            elif not publish:
                # one partial per partition the segment touches
                n_pieces = ((hi - 1) // pb - lo // pb + 1) if pb > 0 else 1
                for k in range(n_pieces):
                    assert slot + k not in partial, "slot written twice"
                    partial[slot + k] = (g, s)
            x = ps + hi
    return partial, final, covered, PT, events, segs


def merge_reads(nblocks, H, R, pb):
    """Slots pass 2 reads per pair (pair -> list) and pairs it leaves alone."""
    S = len(nblocks)
    cb, cp = plan(nblocks, pb)
    T, PT = cb[S], cp[S]
    total = T * H
    reads, skipped = {}, set()
    all_nonempty = total >= R
    fold = pb == 0 and all_nonempty

    def nonempty(r):
        return all_nonempty or range_start(r + 1, total, R) > range_start(r, total, R)

    for g in range(H):
        for s in range(S):
            nblk = cb[s + 1] - cb[s]
            if nblk == 0:
                skipped.add((g, s))
                continue
            ps = g * T + cb[s]
            pe = ps + nblk
            r_lo, r_hi = range_of(ps, total, R), range_of(pe - 1, total, R)
            k0 = g * PT + cp[s]
            got = []
            if pb == 0:
                # one-wave-per-row merge: slots from the range indices alone
                if (r_lo // NW == r_hi // NW) if fold else (r_lo == r_hi):
                    skipped.add((g, s))
                    continue
                for r in range(r_lo, r_hi + 1):
                    if r == r_lo or ((r % NW == 0) if fold else nonempty(r)):
                        got.append(k0 + r)
            else:
                # four-wave merge: one item per partition, split at range starts
                if r_lo == r_hi and nblk <= pb:
                    skipped.add((g, s))
                    continue
                for i in range((nblk + pb - 1) // pb):
                    a = ps + i * pb
                    b = min(a + pb, pe)
                    ra, rb = range_of(a, total, R), range_of(b - 1, total, R)
                    got.append(k0 + i + ra)
                    got += [k0 + i + r for r in range(ra + 1, rb + 1) if nonempty(r)]
            reads[(g, s)] = got
    return reads, skipped


def check(nblocks, H, R, pb):
    nblocks = [int(n) for n in nblocks]
    partial, final, covered, PT, events, _ = pass1(nblocks, H, R, pb)
    check_fold_waits(events, R)
    reads, skipped = merge_reads(nblocks, H, R, pb)
    S = len(nblocks)
    # every tile of every pair covered exactly once
    for g in range(H):
        for s in range(S):
            if nblocks[s]:
                assert np.all(covered[(g, s)] == 1), (g, s)
    # slots below the workspace bound (partitions of all pairs + ranges)
    assert all(0 <= k < H * PT + R for k in partial)
    # pass 2 reads exactly the partials written for each pair, each once
    read_flat = {}
    for pair, slots in reads.items():
        assert len(slots) == len(set(slots)), pair
        for k in slots:
            assert k not in read_flat
            read_flat[k] = pair
    assert read_flat == partial
    # finished pairs: one final row and no partials; the rest: no final row
    nonempty_pairs = {(g, s) for g in range(H) for s in range(S) if nblocks[s]}
    assert set(final) == skipped & nonempty_pairs
    assert all(v == 1 for v in final.values())
    assert not set(final) & set(partial.values())


def case_flags(nblocks, H, R, pb):
    """Which work-division cases each sequence meets (under some kv head):
      publish / absorb   its piece in a range is handed to, or takes in, the
                         piece of the neighbouring wave of a workgroup (fold);
      whole              a pair finished inside pass 1 (final row there);
      merged             a pair left to pass 2;
      merge_gt64         pass 2 merges more than 64 pieces of a pair;
      odd_cut            a range boundary falls inside the pair at an odd
                         16-token tile (the fp8 block-pair stages then mask
                         one half of a pair);
      cut_at_range_start a partition cut coincides with a range start;
      range_in_partition a range start falls strictly inside a partition.
    Returns {sequence: set of case names}."""
    nblocks = [int(n) for n in nblocks]
    S = len(nblocks)
    partial, final, _, PT, events, segs = pass1(nblocks, H, R, pb)
    reads, _ = merge_reads(nblocks, H, R, pb)
    cb, _ = plan(nblocks, pb)
    total = cb[S] * H
    starts = {range_start(r, total, R) for r in range(R)}
    flags = {s: set() for s in range(S)}
    for rg, (g, s), kind in events:
        flags[s].add(kind)
    for (g, s) in final:
        flags[s].add("whole")
    for (g, s), slots in reads.items():
        flags[s].add("merged")
        if len(slots) > 64:
            flags[s].add("merge_gt64")
    for rg, (g, s), lo, hi in segs:
        if lo > 0 and lo % 2 == 1:
            flags[s].add("odd_cut")
    if pb > 0:
        for g in range(H):
            for s in range(S):
                ps = g * cb[-1] + cb[s]
                for i in range((nblocks[s] + pb - 1) // pb):
                    a, b = ps + i * pb, min(ps + (i + 1) * pb, ps + nblocks[s])
                    if i > 0 and a in starts:
                        flags[s].add("cut_at_range_start")
                    if any(a < x < b for x in (range_start(range_of(b - 1, total, R), total, R),)):
                        flags[s].add("range_in_partition")
    return flags


def targeted_sample(flags, lens, k, cases, seed):
    """Up to two sequences per case, the shortest and the longest, then
    random ones up to k (all when k >= the batch)."""
    S = len(lens)
    if k >= S:
        return np.arange(S)
    pick = {int(np.argmin(lens)), int(np.argmax(lens))}
    for c in cases:
        hit = [s for s in range(S) if c in flags[s]]
        pick.update(hit[:2])
    rng = np.random.default_rng(seed)
    while len(pick) < k:
        pick.add(int(rng.integers(0, S)))
    return np.array(sorted(pick))


def check_fold_waits(events, R):
    """The LDS fold's waits, as pass 1 takes them: wave w of a workgroup that
    absorbs waits for a publish by wave w + 1 of the same workgroup, for the
    same pair.  Checked: every absorb has exactly that publish and every
    publish is absorbed (no piece is dropped); the last wave never waits, so
    a wave waits only on higher waves of its workgroup, each wave waits at
    most once and publishes at most once, and the longest chain of waits
    (w -> w + 1 -> ...) is at most NW - 1 long: no cycle, every wait ends."""
    pub = {}
    absorbs = {}
    for rg, pair, kind in events:
        table = pub if kind == "publish" else absorbs
        assert rg not in table, f"range {rg} {kind}es twice"
        table[rg] = pair
    for rg, pair in absorbs.items():
        assert rg % NW != NW - 1, "the last wave of a workgroup waits"
        assert pub.get(rg + 1) == pair, f"range {rg} waits for a publish that never comes"
    for rg, pair in pub.items():
        assert rg % NW != 0, "the first wave of a workgroup publishes"
        assert absorbs.get(rg - 1) == pair, f"range {rg} publishes a piece nobody absorbs"
    # chains of waits: w waits on w + 1 (which may itself wait on w + 2)
    for rg in absorbs:
        n, r = 0, rg
        while r in absorbs:
            n += 1
            r += 1
            assert r // NW == rg // NW, "a wait leaves its workgroup"
        assert n <= NW - 1


@pytest.mark.parametrize("seed", range(6))
def test_random_batches(seed):
    rng = random.Random(seed)
    for _ in range(120):
        S = rng.randint(1, 12)
        H = rng.choice([1, 2, 8])
        R = rng.choice([32, 64, 256])
        pb = rng.choice([0, 0, 1, 2, 8, 32])
        mode = rng.random()
        if mode < 0.3:
            lens = [rng.randint(0, 40) for _ in range(S)]
        elif mode < 0.6:
            lens = [rng.randint(0, 2000) for _ in range(S)]
        else:
            lens = [rng.choice([0, 1, 16, 17, rng.randint(1, 9000)]) for _ in range(S)]
        if sum(lens) == 0:
            continue
        check([(L + 15) // 16 for L in lens], H, R, pb)


@pytest.mark.parametrize("index,pb", [(2, 0), (3, 0), (5, 32), (5, 0)])
def test_benchmark_workloads(index, pb):
    """The lengths the benchmark draws, at the range count of bf16 D=128
    (two waves per SIMD on 256 CUs: 2048); partition 512 tokens = 32 tiles."""
    spec = workloads.SPECS[index]
    lens = workloads.lengths(spec)
    nblocks = [(int(L) + 15) // 16 for L in lens]
    check(nblocks, spec.num_kv_heads, 2048, pb)
    if pb == 0:  # the fold is on, and its waits reach the longest chain (3)
        events = pass1(nblocks, spec.num_kv_heads, 2048, pb)[4]
        absorbs = {rg for rg, _, kind in events if kind == "absorb"}
        assert any(rg in absorbs and rg + 1 in absorbs and rg + 2 in absorbs for rg in absorbs)


# the cases the full-size GPU parity samples must contain, per workload and
# partition (in 16-token tiles)
FULL_SIZE_CASES = {
    (3, 0): ("publish", "absorb", "whole", "merged"),
    (4, 0): ("publish", "absorb", "whole", "merged", "odd_cut"),
    (4, 3): ("merged", "cut_at_range_start", "range_in_partition", "odd_cut"),
    (5, 32): ("merged", "merge_gt64", "cut_at_range_start", "range_in_partition"),
}


@pytest.mark.parametrize("index,pb", list(FULL_SIZE_CASES))
def test_full_size_workloads_meet_every_case(index, pb):
    """At the range count of bf16 and fp8 D=128 on MI355X (2048), the
    workloads' own length draws meet every case their GPU parity sample must
    contain."""
    spec = workloads.SPECS[index]
    lens = workloads.lengths(spec)
    flags = case_flags([(int(L) + 15) // 16 for L in lens], spec.num_kv_heads, 2048, pb)
    for c in FULL_SIZE_CASES[(index, pb)]:
        assert any(c in f for f in flags.values()), c
