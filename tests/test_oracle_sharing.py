"""Pins of the oracle's shared blocks (reference counts, fork, copy-on-write).

What the pages fix (serving tutorial): section 4.2 - a physical block can
be shared by a common prefix or by beam / parallel-sampling branches
through reference counts, and a shared writable tail block that one holder
changes is copied and remapped for that holder only; section 1.7 - a shared
block goes back to the allocator only when its last holder releases it,
with no double free and no leak; demo D08 - sequences of 6 and 7 tokens
(block size 4) sharing one full block need 3 physical blocks instead of 4;
its best-of-n question - the prompt's KV is held once, only the branches'
own tokens grow with the number of branches.
"""
import collections
import json
import os
import random

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _physical(rows):
    return len({b for r in rows for b in r.blocks})


def test_demo_d08_sharing_one_full_block():
    g = _golden("serving_tutorial_demos.json")
    plain = g["physical_blocks_no_sharing"]
    shared = g["physical_blocks_sharing_one_full_block"]
    B = shared["block_size"]
    L6, L7 = shared["lengths"]
    # without sharing
    a = oracle.BlockAllocator(16)
    r = [oracle.SequenceBlocks(B) for _ in range(2)]
    r[0].ensure(a, L6)
    r[1].ensure(a, L7)
    assert _physical(r) == plain["expected_blocks"]
    # the 7-token sequence starts from the 6-token one's first full block
    a = oracle.BlockAllocator(16)
    r = [oracle.SequenceBlocks(B) for _ in range(2)]
    r[0].ensure(a, L6)
    r[1].fork(a, r[0], shared["shared_full_blocks"] * B)
    r[1].ensure(a, L7)
    assert _physical(r) == shared["expected_blocks"]
    assert a.refcount(r[0].blocks[0]) == 2 and r[1].blocks[0] == r[0].blocks[0]
    assert a.num_free == 16 - shared["expected_blocks"]


def test_shared_block_returns_only_with_its_last_holder():
    a = oracle.BlockAllocator(8)
    p = oracle.SequenceBlocks(4)
    p.ensure(a, 10)                       # blocks 0, 1, 2
    kids = [oracle.SequenceBlocks(4) for _ in range(3)]
    for k in kids:
        k.fork(a, p, 10)
    assert [a.refcount(b) for b in p.blocks] == [4, 4, 4]
    p.release(a)
    p.release(a)                          # idempotent
    assert a.num_free == 5 and [a.refcount(b) for b in kids[0].blocks] == [3, 3, 3]
    kids[0].release(a)
    kids[1].release(a)
    assert a.num_free == 5
    kids[2].release(a)
    assert a.num_free == 8 and a.free_ids() == list(range(8)) and a.refs == {}


def test_best_of_n_block_count_closed_form():
    """n branches forked from a P-token prompt, the prompt row released,
    each branch then appending g >= 1 tokens: the full prompt blocks are
    held once, every branch owns its (copied) tail block and its growth.
    Distinct blocks = floor(P/B) + n (ceil((P+g)/B) - floor(P/B)); without
    sharing n ceil((P+g)/B)."""
    rng = random.Random(3)
    for _ in range(300):
        B = rng.choice([1, 2, 4, 16])
        P = rng.randint(1, 80)
        g = rng.randint(1, 40)
        n = rng.randint(1, 6)
        a = oracle.BlockAllocator(2000)
        prompt = oracle.SequenceBlocks(B)
        prompt.ensure(a, P)
        kids = [oracle.SequenceBlocks(B) for _ in range(n)]
        for k in kids:
            k.fork(a, prompt, P)
        prompt.release(a)
        copies = 0
        for k in kids:
            copies += len(k.cow(a, P, g))
            k.ensure(a, P + g)
        per_branch = -(-(P + g) // B) - P // B
        assert _physical(kids) == P // B + n * per_branch
        assert 2000 - a.num_free == P // B + n * per_branch
        # the tail block is copied by every branch but the last writer
        assert copies == (n - 1 if P % B else 0)
        for k in kids:
            k.release(a)
        assert a.num_free == 2000


def test_refcount_model_against_a_brute_force_counter():
    """Random alloc / share / free / fork / cow / release scripts: the
    allocator's counts equal a plain multiset of the rows' entries plus the
    loose holds, free ids are exactly the uncounted ones (in rank order),
    and errors change nothing."""
    for seed in range(40):
        rng = random.Random(seed)
        n, B = rng.choice([(12, 4), (40, 2), (64, 16)])
        order = list(range(n))
        rng.shuffle(order)
        a = oracle.BlockAllocator(n, order)
        rows = [oracle.SequenceBlocks(B) for _ in range(6)]
        lens = [0] * 6
        loose = collections.Counter()       # holds taken by bare alloc / share
        for _ in range(200):
            op = rng.random()
            s = rng.randrange(6)
            snapshot = (dict(a.refs), list(a.free_ranks), [list(r.blocks) for r in rows])
            try:
                if op < 0.3:
                    L = lens[s] + rng.randint(0, 3 * B)
                    rows[s].ensure(a, L)
                    lens[s] = max(lens[s], L)
                elif op < 0.45:
                    t = rng.randrange(6)
                    if t != s and not rows[s].blocks and rows[t].blocks:
                        L = rng.randint(0, lens[t])
                        rows[s].fork(a, rows[t], L)
                        lens[s] = L
                elif op < 0.6:
                    if lens[s]:
                        start = rng.randint(0, lens[s])
                        pairs = rows[s].cow(a, start, rng.randint(1, 2 * B))
                        assert all(a.refcount(new) == 1 for _, new in pairs)
                elif op < 0.7:
                    rows[s].release(a)
                    lens[s] = 0
                elif op < 0.8:
                    ids = a.alloc(rng.randint(0, 2))
                    loose.update(ids)
                elif op < 0.9:
                    held = list(loose.elements())
                    if held:
                        b = rng.choice(held)
                        if rng.random() < 0.5:
                            a.share([b])
                            loose[b] += 1
                        else:
                            a.free([b])
                            loose[b] -= 1
                            if loose[b] == 0:
                                del loose[b]
                else:
                    bad = rng.choice([[n], [-1], a.free_ids()[:1] or [n]])
                    with pytest.raises((oracle.InvalidFree, oracle.InvalidBlock)):
                        (a.free if rng.random() < 0.5 else a.share)(bad)
            except oracle.OutOfBlocks:
                assert (dict(a.refs), list(a.free_ranks), [list(r.blocks) for r in rows]) == snapshot
            count = collections.Counter(b for r in rows for b in r.blocks) + loose
            assert dict(count) == a.refs
            assert a.free_ids() == [order[k] for k in range(n) if order[k] not in count]


def test_copy_on_write_keeps_every_branch_exact():
    """Gathering a branch after fork + copy-on-write + append returns the
    prompt's rows followed by the branch's own rows, bit for bit, and the
    other branches still see theirs."""
    rng = np.random.default_rng(5)
    B, n_kv, d = 4, 2, 3
    a = oracle.BlockAllocator(40)
    pool_k = np.full((40, n_kv, B, d), np.nan, dtype=np.float32)
    pool_v = pool_k.copy()
    P = 6
    pk, pv = rng.standard_normal((2, P, n_kv, d)).astype(np.float32)
    prompt = oracle.SequenceBlocks(B)
    prompt.ensure(a, P)
    oracle.append(pool_k, pool_v, prompt.blocks, 0, pk, pv, B)
    kids, own = [], []
    for i in range(3):
        k = oracle.SequenceBlocks(B)
        k.fork(a, prompt, P)
        kids.append(k)
    for i, k in enumerate(kids):
        g = 1 + 3 * i
        kk, vv = rng.standard_normal((2, g, n_kv, d)).astype(np.float32)
        oracle.copy_blocks(pool_k, pool_v, k.cow(a, P, g))
        k.ensure(a, P + g)
        oracle.append(pool_k, pool_v, k.blocks, P, kk, vv, B)
        own.append((kk, vv))
    for k, (kk, vv) in zip(kids, own):
        L = P + len(kk)
        got_k = oracle.gather(pool_k, k.blocks, L, B)
        got_v = oracle.gather(pool_v, k.blocks, L, B)
        assert np.array_equal(got_k.transpose(1, 0, 2), np.concatenate([pk, kk]))
        assert np.array_equal(got_v.transpose(1, 0, 2), np.concatenate([pv, vv]))
    # the prompt row itself still reads the prompt only
    got = oracle.gather(pool_k, prompt.blocks, P, B)
    assert np.array_equal(got.transpose(1, 0, 2), pk)
