"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

None of these retypes the oracle's formulas; each compares it with something
independent (printed page values, closed forms, a pure-Python brute force, a
library routine, or an invariant the pages state).
"""
import json
import math
import os
import random

import numpy as np
import pytest

import oracle
from oracle import scalar
from workloads import BF16, F32, build_workload, config_workload, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- storage ---


def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x3FC0, 0x8000, 0x4049], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    want = [1.0, -2.0, math.inf, -math.inf, 2.0 ** -133, 1.5, -0.0, 3.140625]
    for g, w in zip(got, want):
        assert g == w
    assert math.copysign(1.0, got[6]) == -1.0


def test_generator_rounds_to_nearest_even():
    # 1 + 2^-8 sits halfway between bf16 1.0 (even) and 1 + 2^-7 (odd) -> 1.0;
    # 1 + 3*2^-8 sits halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> the latter.
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.0], dtype=np.float32)
    assert f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F82, 0x3F81, 0xC000]


# ------------------------------------------------------- byte/slot counts ---


def test_serving_tutorial_byte_and_slot_demos():
    g = _golden("serving_tutorial_demos.json")
    k = g["kv_bytes_per_token"]
    m = oracle.kv_bytes_per_token(k["n_layer"], k["n_kv_head"], k["d_head"], k["bytes_per_elem"])
    assert m == k["expected"]
    b = g["block_alloc_slots"]
    logical, allocated = oracle.block_alloc_slots(b["lengths"], b["block_size"])
    assert (logical, allocated) == (b["expected_logical_slots"], b["expected_allocated_slots"])
    assert (logical * m, allocated * m) == (b["expected_logical_bytes"], b["expected_allocated_bytes"])
    p = g["physical_blocks_no_sharing"]
    _, alloc_slots = oracle.block_alloc_slots(p["lengths"], p["block_size"])
    assert alloc_slots // p["block_size"] == p["expected_blocks"]


def test_lab_and_chapter5_byte_counts():
    g = _golden("lab_values.json")
    k = g["kv_bytes_per_token_float64"]
    assert oracle.kv_bytes_per_token(k["n_layer"], k["n_kv_head"], k["d_head"], k["bytes_per_elem"]) == k["expected"]
    e = g["example_sequence_bytes"]
    per_tok = oracle.kv_bytes_per_token(e["n_layer"], e["n_kv_head"], e["d_head"], e["bytes_per_elem"])
    assert round(per_tok * e["tokens"] / 2 ** 30, 2) == e["expected_gib"]
    f = _golden("foundations_ch5_values.json")
    k = f["mha_70b_kv_bytes_per_token"]
    per_tok = oracle.kv_bytes_per_token(k["n_layer"], k["n_kv_head"], k["d_head"], k["bytes_per_elem"])
    assert per_tok == k["expected"]
    b = f["mha_70b_batch_kv"]
    assert per_tok * b["batch"] * b["context"] / 2 ** 30 == b["expected_gib"]


# --------------------------------------------------------------- allocator ---


def test_allocator_identity_order_is_the_lab_free_list():
    rng = random.Random(3)
    for trial in range(200):
        n = rng.randint(1, 20)
        alloc = oracle.BlockAllocator(n)
        script, held = [], []
        for _ in range(30):
            if held and rng.random() < 0.4:
                k = rng.randint(1, len(held))
                give = rng.sample(held, k)
                held = [b for b in held if b not in give]
                alloc.free(give)
                script.append(("give", give))
            else:
                k = rng.randint(0, alloc.num_free)
                got = alloc.alloc(k)
                held += got
                script.append(("take", k))
                script[-1] = ("take", k, got)
        model_script = [(op[0], op[1]) for op in script]
        taken, free = scalar.lab_free_list_model(n, model_script)
        ours = [op[2] for op in script if op[0] == "take"]
        assert ours == taken
        assert alloc.free_ids() == free


def test_allocator_permuted_order_hands_out_lowest_rank():
    order = [5, 2, 7, 0, 1, 6, 3, 4]
    a = oracle.BlockAllocator(8, order)
    assert a.alloc(3) == [5, 2, 7]
    a.free([2])
    assert a.alloc(2) == [2, 0]
    a.free([5, 0])
    assert a.free_ids() == [5, 0, 1, 6, 3, 4]


def test_allocator_errors_change_nothing():
    a = oracle.BlockAllocator(4)
    got = a.alloc(3)
    before = a.free_ids()
    with pytest.raises(oracle.OutOfBlocks):
        a.alloc(2)
    assert a.free_ids() == before
    for bad in ([3], [0, 0], [0, 9], [-1], [1, 3]):
        with pytest.raises(oracle.InvalidFree):
            a.free(bad)
        assert a.free_ids() == before
    a.free(got)
    assert a.num_free == 4 and a.free_ids() == [0, 1, 2, 3]


def test_sequence_release_is_idempotent():
    a = oracle.BlockAllocator(6)
    s = oracle.SequenceBlocks(4)
    s.ensure(a, 9)
    assert s.blocks == [0, 1, 2]
    s.ensure(a, 12)          # still 3 blocks
    assert s.blocks == [0, 1, 2]
    s.ensure(a, 13)          # position 12 opens block 3
    assert s.blocks == [0, 1, 2, 3]
    s.release(a)
    s.release(a)             # second reclaim is a no-op, not a double free
    assert a.num_free == 6


def test_config1_uses_seven_of_twelve_blocks_and_returns_all():
    g = _golden("lab_values.json")
    wl = config_workload(1)
    assert wl.seq_lens.tolist() == [10, 8, 6]
    cache = oracle.build_cache(wl)
    used = wl.num_blocks - cache.allocator.num_free
    assert used == g["peak_blocks"]["expected_used"] and wl.num_blocks == g["peak_blocks"]["pool_blocks"]
    for sb in cache.seqs:
        sb.release(cache.allocator)
    assert cache.allocator.num_free == wl.num_blocks
    assert sorted(cache.allocator.free_ids()) == list(range(wl.num_blocks))


# ---------------------------------------------------------- append/gather ---


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_gather_returns_exactly_what_was_appended(dtype):
    wl = build_workload(n_q=4, n_kv=2, head_dim=8, block_size=4, dtype=dtype,
                        hist_lens=[0, 3, 4, 7, 8, 13], new_lens=[1, 1, 5, 1, 4, 3], seed=11)
    cache = oracle.build_cache(wl)
    written = 0
    for s in range(wl.num_seqs):
        L = int(wl.seq_lens[s])
        k, v = wl.rows(s, 0, L)
        K = oracle.gather(cache.pool_k, cache.seqs[s].blocks, L, wl.block_size)
        V = oracle.gather(cache.pool_v, cache.seqs[s].blocks, L, wl.block_size)
        assert np.array_equal(K.view(np.uint8), k.transpose(1, 0, 2).view(np.uint8))
        assert np.array_equal(V.view(np.uint8), v.transpose(1, 0, 2).view(np.uint8))
        written += L
    # every slot nobody wrote still holds the NaN poison
    finite = np.isfinite(oracle.widen(cache.pool_k, dtype)).all(axis=(1, 3)).sum()
    assert finite == written
    # the table rows are distinct blocks
    t = cache.tables()
    used = t[t >= 0]
    assert len(np.unique(used)) == len(used)


def test_lab_prefill_cache_shape():
    g = _golden("lab_values.json")["prefill_cache_shape"]
    wl = build_workload(n_q=2, n_kv=2, head_dim=4, block_size=4, dtype=F32,
                        hist_lens=[0], new_lens=[g["tokens"]], num_blocks=12, seed=7)
    cache = oracle.build_cache(wl)
    K, _ = cache.sequence_kv(0)
    assert list(K.shape) == g["expected_k_shape"]


# --------------------------------------------------------------- attention ---


def _random_case(rng, B, d, L, n_q, n_kv, C):
    q = rng.standard_normal((C, n_q, d))
    K = rng.standard_normal((n_kv, L, d))
    V = rng.standard_normal((n_kv, L, d))
    return q, K, V


def test_attention_matches_brute_force_on_tiny_cases():
    rng = np.random.default_rng(5)
    cases = 0
    for B in (1, 2, 4):
        for d in (1, 4):
            for L in range(1, 25):
                for (n_q, n_kv) in ((2, 2), (2, 1), (4, 2)):
                    C = int(rng.integers(1, L + 1))
                    q, K, V = _random_case(rng, B, d, L, n_q, n_kv, C)
                    scale = 1 / math.sqrt(d)
                    pos = np.arange(L - C, L)
                    out, lse, _ = oracle.attention(q, K, V, scale, pos)
                    G = n_q // n_kv
                    for t in range(C):
                        for h in range(n_q):
                            g = h // G
                            o, l, _ = scalar.attention_row(q[t, h].tolist(), K[g].tolist(), V[g].tolist(),
                                                           scale, int(pos[t]))
                            assert np.max(np.abs(out[t, h] - np.array(o))) <= 1e-12
                            assert abs(lse[t, h] - l) <= 1e-12
                    cases += 1
    assert cases == 3 * 2 * 24 * 3


def test_config1_matches_brute_force():
    wl = config_workload(1)
    cache = oracle.build_cache(wl)
    out, lse = oracle.paged_attention_all(cache)
    for s in range(wl.num_seqs):
        L = int(wl.seq_lens[s])
        k, v = wl.rows(s, 0, L)
        q = wl.q[s]
        for h in range(wl.n_q):
            o, l, w = scalar.attention_row(q[h].astype(float).tolist(), k[:, h].astype(float).tolist(),
                                           v[:, h].astype(float).tolist(), wl.scale, L - 1)
            assert np.max(np.abs(out[s, h] - np.array(o))) <= 1e-12
            assert abs(lse[s, h] - l) <= 1e-12
            assert len(w) == L and abs(math.fsum(w) - 1.0) < 1e-12


def test_weights_sum_to_one_and_lse_matches_library_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(9)
    q, K, V = _random_case(rng, 4, 16, 37, 8, 2, 6)
    pos = np.arange(31, 37)
    out, lse, p = oracle.attention(q, K, V, 0.25, pos)
    assert np.all(np.abs(p.sum(axis=-1) - 1.0) < 1e-9)
    G = 4
    for t in range(6):
        for h in range(8):
            s = 0.25 * (K[h // G, :pos[t] + 1] @ q[t, h])
            assert abs(lse[t, h] - logsumexp(s)) < 1e-12
            # masked keys get exactly zero weight
            assert np.all(p[h, t, pos[t] + 1:] == 0.0)


def test_closed_forms():
    rng = np.random.default_rng(1)
    # one key: the output is that key's value, exactly
    q, K, V = _random_case(rng, 4, 8, 1, 4, 2, 1)
    out, lse, _ = oracle.attention(q, K, V, 0.3, [0])
    for h in range(4):
        assert np.array_equal(out[0, h], V[h // 2, 0])
        assert abs(lse[0, h] - 0.3 * float(q[0, h] @ K[h // 2, 0])) < 1e-15
    # identical keys: uniform weights, output is the mean of V, lse = s + ln L
    L = 13
    K = np.repeat(rng.standard_normal((2, 1, 8)), L, axis=1)
    V = rng.standard_normal((2, L, 8))
    q = rng.standard_normal((1, 4, 8))
    out, lse, p = oracle.attention(q, K, V, 0.5, [L - 1])
    for h in range(4):
        assert np.allclose(out[0, h], V[h // 2].mean(axis=0), atol=1e-14, rtol=0)
        assert abs(lse[0, h] - (0.5 * float(q[0, h] @ K[h // 2, 0]) + math.log(L))) < 1e-12
    # two keys, hand-computed: s = (1, 0) -> weights e/(e+1), 1/(e+1)
    q = np.array([[[1.0, 0.0]]])
    K = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    V = np.array([[[2.0, 0.0], [0.0, 4.0]]])
    out, lse, _ = oracle.attention(q, K, V, 1.0, [1])
    e = math.e
    assert np.allclose(out[0, 0], [2 * e / (e + 1), 4 / (e + 1)], atol=1e-15, rtol=0)
    assert abs(lse[0, 0] - math.log(e + 1)) < 1e-15
    # causal: the first query of a chunk at position 0 sees only key 0
    out, _, _ = oracle.attention(np.ones((2, 1, 2)), K, V, 1.0, [0, 1])
    assert np.array_equal(out[0, 0], V[0, 0])


def test_query_heads_map_to_kv_heads_in_contiguous_groups():
    # kv head g holds values equal to g everywhere; head h must read kv head h // 4
    n_q, n_kv, d, L = 8, 2, 4, 5
    K = np.random.default_rng(2).standard_normal((n_kv, L, d))
    V = np.stack([np.full((L, d), float(g)) for g in range(n_kv)])
    q = np.random.default_rng(3).standard_normal((1, n_q, d))
    out, _, _ = oracle.attention(q, K, V, 1.0, [L - 1])
    for h in range(n_q):
        assert np.allclose(out[0, h], h // 4, atol=1e-14)
    # heads of one group given the same query give identical outputs
    q[0, 1] = q[0, 0]
    out, _, _ = oracle.attention(q, K, np.random.default_rng(4).standard_normal((n_kv, L, d)), 1.0, [L - 1])
    assert np.array_equal(out[0, 0], out[0, 1])
    with pytest.raises(ValueError):
        oracle.attention(np.ones((1, 3, d)), K, V, 1.0, [0])


def test_matches_library_sdpa_for_a_causal_prefill():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    L, n_h, d = 23, 3, 16
    q, K, V = _random_case(rng, 4, d, L, n_h, n_h, L)
    out, _, _ = oracle.attention(q, K, V, 1 / math.sqrt(d), np.arange(L))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2).copy()), torch.from_numpy(K.copy()), torch.from_numpy(V.copy()),
        is_causal=True)
    assert np.max(np.abs(out - ref.numpy().transpose(1, 0, 2))) < 1e-12


def test_split_merge_is_exact():
    rng = np.random.default_rng(12)
    for trial in range(40):
        L = int(rng.integers(1, 60))
        C = int(rng.integers(1, min(L, 8) + 1))
        q, K, V = _random_case(rng, 4, 8, L, 4, 2, C)
        pos = np.arange(L - C, L)
        cuts = sorted(set(rng.integers(0, L + 1, size=int(rng.integers(0, 6))).tolist()) | {0, L})
        bounds = list(zip(cuts[:-1], cuts[1:])) + [(L, L)]
        out, lse, _ = oracle.attention(q, K, V, 0.35, pos)
        out2, lse2 = oracle.attention_split_merge(q, K, V, 0.35, pos, bounds)
        assert np.max(np.abs(out - out2)) <= 1e-12
        assert np.max(np.abs(lse - lse2)) <= 1e-12
    # a split whose keys are all masked (beyond every query's position) has weight 0
    q, K, V = _random_case(rng, 4, 8, 20, 2, 2, 3)
    pos = np.array([5, 6, 7])
    out, lse, _ = oracle.attention(q, K, V, 0.35, pos)
    out2, lse2 = oracle.attention_split_merge(q, K, V, 0.35, pos, [(0, 4), (4, 10), (10, 20)])
    assert np.max(np.abs(out - out2)) <= 1e-12 and np.isfinite(out2).all()


# ------------------------------------------------- paged versus contiguous ---


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_paged_equals_contiguous(dtype):
    bound = _golden("lab_values.json")["parity_bound"]
    wl = build_workload(n_q=8, n_kv=2, head_dim=16, block_size=4, dtype=dtype,
                        hist_lens=[0, 1, 3, 4, 5, 15, 16, 33], new_lens=[1, 4, 1, 1, 3, 1, 9, 2], seed=21)
    cache = oracle.build_cache(wl)
    for s in range(wl.num_seqs):
        o1, l1 = cache.attend(s)
        o2, l2 = oracle.contiguous_attend(wl, s)
        assert np.max(np.abs(o1 - o2)) <= bound and np.max(np.abs(l1 - l2)) <= bound


def test_relabelling_physical_blocks_changes_nothing():
    kw = dict(n_q=4, n_kv=2, head_dim=8, block_size=2, dtype=BF16,
              hist_lens=[6, 1, 9], new_lens=[1, 1, 3], num_blocks=20, seed=4)
    a = oracle.build_cache(build_workload(order="identity", **kw))
    b = oracle.build_cache(build_workload(order=np.random.default_rng(0).permutation(20), **kw))
    assert not np.array_equal(a.tables(), b.tables())
    oa, la = oracle.paged_attention_all(a)
    ob, lb = oracle.paged_attention_all(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_lab_prompt_chunks_equal_one_chunk_and_recompute():
    lab = _golden("lab_values.json")
    chunks = lab["prompt_chunks"]["chunks"]
    n = lab["prompt_chunks"]["prompt_tokens"]
    one = build_workload(n_q=2, n_kv=2, head_dim=4, block_size=4, dtype=F32, hist_lens=[0], new_lens=[n],
                         num_blocks=12, seed=7)
    K = oracle.widen(one.k_seq, F32).transpose(1, 0, 2)
    V = oracle.widen(one.v_seq, F32).transpose(1, 0, 2)
    q = oracle.widen(one.q, F32)
    full, _, p = oracle.attention(q, K, V, one.scale, np.arange(n))
    # the last prompt position's weights: n entries that sum to one
    w = lab["last_prefill_weights"]
    assert p[0, -1].shape[0] == w["expected_count"] and abs(p[0, -1].sum() - w["expected_sum"]) < 1e-12
    # chunked through the pool: first chunk over an empty cache, then the rest
    lo = 0
    alloc = oracle.BlockAllocator(12, one.alloc_order)
    seq = oracle.SequenceBlocks(4)
    pk = np.full((12, 2, 4, 4), np.nan, dtype=np.float32)
    pv = pk.copy()
    outs = []
    for c in chunks:
        seq.ensure(alloc, lo + c)
        oracle.append(pk, pv, seq.blocks, lo, one.k_seq[lo:lo + c], one.v_seq[lo:lo + c], 4)
        Kc = oracle.widen(oracle.gather(pk, seq.blocks, lo + c, 4), F32)
        Vc = oracle.widen(oracle.gather(pv, seq.blocks, lo + c, 4), F32)
        o, _, _ = oracle.attention(q[lo:lo + c], Kc, Vc, one.scale, np.arange(lo, lo + c))
        outs.append(o)
        lo += c
    assert np.max(np.abs(np.concatenate(outs) - full)) <= lab["parity_bound"]
    seq.release(alloc)
    assert alloc.num_free == 12


def test_fp32_rounding_is_far_inside_the_fp32_tolerance():
    # chapter 5's cache-vs-recompute demo shows fp32 rounding near 3e-8; the
    # fp32 tolerance 1e-5 leaves a wide margin. Same here for attention
    # computed entirely in float32 against the float64 oracle.
    printed = _golden("foundations_ch5_values.json")["fp32_cache_vs_recompute_max_abs"]
    rng = np.random.default_rng(7)
    q, K, V = _random_case(rng, 4, 64, 24, 1, 1, 1)
    out, _, _ = oracle.attention(q, K, V, 1 / 8, [23])
    q32, K32, V32 = q.astype(np.float32), K.astype(np.float32), V.astype(np.float32)
    s = (K32[0] @ q32[0, 0]) * np.float32(1 / 8)
    e = np.exp(s - s.max())
    o32 = (e / e.sum()) @ V32[0]
    err = np.max(np.abs(o32 - out[0, 0]))
    assert err < 100 * printed < 1e-5


def _lab_pool_replay(wl):
    """The lab page's KVPool, token by token: a sequence takes the next free
    block (lowest rank, here the pool's order) each time a position reaches
    the end of the blocks it holds; history of every sequence first, then
    the step's new tokens, sequences in index order. Nothing is released
    during a step, so "take the next free" is a walk along the order."""
    from collections import deque
    free = deque(int(b) for b in wl.alloc_order)
    rows = [[] for _ in range(wl.num_seqs)]
    B = wl.block_size
    for lo, hi in ((np.zeros_like(wl.hist_lens), wl.hist_lens), (wl.hist_lens, wl.seq_lens)):
        for s in range(wl.num_seqs):
            for p in range(int(lo[s]), int(hi[s])):
                if p // B == len(rows[s]):
                    rows[s].append(free.popleft())
    return rows


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_build_tables_is_the_lab_pool_replayed_token_by_token(cfg):
    """oracle.build_tables (ceil-division bulk allocation) against a literal
    per-token replay of the lab's pool on every configuration, plus the
    invariants a table must satisfy: ceil(L / B) blocks per sequence, no
    block in two rows, padding -1, and the blocks in use are exactly the
    first ones of the allocation order."""
    wl = config_workload(cfg)
    t = oracle.build_tables(wl)
    rows = _lab_pool_replay(wl)
    B = wl.block_size
    used = []
    for s in range(wl.num_seqs):
        nb = -(-int(wl.seq_lens[s]) // B)
        assert len(rows[s]) == nb
        assert t[s, :nb].tolist() == rows[s]
        assert (t[s, nb:] == -1).all()
        used += rows[s]
    assert len(set(used)) == len(used)
    assert sorted(used) == sorted(wl.alloc_order[:len(used)].tolist())
    if cfg in (1, 4):   # the cache replay (history, then the step) makes the same rows
        assert np.array_equal(t, oracle.build_cache(wl).tables())
