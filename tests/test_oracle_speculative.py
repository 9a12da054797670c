"""Pins of verify / rollback bookkeeping (chapter 5 section 5; serving
tutorial, question on speculative decoding).

The pages fix: the target verifies gamma drafts in one pass, producing
gamma + 1 distributions; drafts after the first rejection are discarded; a
cycle yields at least 1 and at most gamma + 1 tokens, E[tokens] =
(1 - alpha^(gamma+1)) / (1 - alpha) for acceptance rate alpha; the KV of
rejected candidates is rolled back and not committed.
"""
import random

import numpy as np

import oracle
from workloads import BF16, F32, build_spec_workload

from spec_replay import OracleSpec


def test_rollback_releases_exactly_the_blocks_past_the_committed_length():
    rng = random.Random(4)
    for _ in range(400):
        B = rng.choice([1, 2, 4, 16])
        L = rng.randint(1, 90)
        gamma = rng.randint(1, 8)
        acc = rng.randint(0, gamma)
        a = oracle.BlockAllocator(200)
        row = oracle.SequenceBlocks(B)
        row.ensure(a, L)
        row.ensure(a, L + gamma + 1)                    # verify appends gamma + 1 tokens
        held = len(row.blocks)
        row.truncate(a, L + 1 + acc)
        row.truncate(a, L + 1 + acc)                    # idempotent
        assert len(row.blocks) == -(-(L + 1 + acc) // B)
        assert a.num_free == 200 - len(row.blocks)
        assert held - len(row.blocks) == -(-(L + gamma + 1) // B) - -(-(L + 1 + acc) // B)
        # a block shared with another row only loses this row's hold
        other = oracle.SequenceBlocks(B)
        other.fork(a, row, L + 1 + acc)
        row.truncate(a, 0)
        assert a.num_free == 200 - len(other.blocks)


def test_rollback_cycles_follow_the_acceptance_formula():
    """Speculative cycles on one oracle row: each cycle grows the row for
    gamma + 1 tokens (SequenceBlocks.ensure), then rolls it back to the
    committed length (SequenceBlocks.truncate), the accepted drafts plus one
    sampled token, with drafts accepted independently with probability alpha
    until the first rejection (chapter 5 section 5). After every cycle the
    row holds exactly ceil(L / B) blocks and the pool the rest; over the
    cycles the committed tokens per cycle lie in [1, gamma + 1] with mean
    (1 - alpha^(gamma+1)) / (1 - alpha)."""
    rng = np.random.default_rng(9)
    B, N = 16, 8192
    for alpha in (0.3, 0.6, 0.85):
        for gamma in (1, 4, 5):
            n = 3000
            accept = rng.random((n, gamma)) < alpha
            n_acc = np.where(accept.all(axis=1), gamma, np.argmin(accept, axis=1))
            a = oracle.BlockAllocator(N)
            row = oracle.SequenceBlocks(B)
            L = 7
            row.ensure(a, L)
            committed = []
            for c in range(n):
                row.ensure(a, L + gamma + 1)
                row.truncate(a, L + int(n_acc[c]) + 1)
                committed.append(int(n_acc[c]) + 1)
                L += int(n_acc[c]) + 1
                assert len(row.blocks) == -(-L // B)
                assert a.num_free == N - len(row.blocks)
            tokens = np.array(committed)
            assert tokens.min() >= 1 and tokens.max() <= gamma + 1
            expect = (1 - alpha ** (gamma + 1)) / (1 - alpha)
            sd = tokens.std() / np.sqrt(n)
            assert abs(tokens.mean() - expect) < 5 * sd
            row.release(a)
            assert a.num_free == N and a.free_ids() == list(range(N))


def test_verify_chunk_equals_one_query_at_a_time():
    """The gamma + 1 verification queries in one causal chunk give what each
    query gives alone over the keys up to its own position."""
    sw = build_spec_workload(n_q=4, n_kv=2, head_dim=8, block_size=4, dtype=F32, hist_lens=[3, 9, 16],
                             gamma=4, cycles=1, seed=3)
    o = OracleSpec(sw)
    o.append_cycle(0)
    chunk = o.verify(0)
    g1 = sw.gamma + 1
    for s in range(sw.num_seqs):
        L = int(o.lens[s])
        K = oracle.widen(np.concatenate([sw.hist_k[s], sw.cyc_k[0][s]]), sw.dtype).transpose(1, 0, 2)
        V = oracle.widen(np.concatenate([sw.hist_v[s], sw.cyc_v[0][s]]), sw.dtype).transpose(1, 0, 2)
        for i in range(g1):
            q = oracle.widen(sw.cyc_q[0][s * g1 + i:s * g1 + i + 1], sw.dtype)
            one, _, _ = oracle.attention(q, K[:, :L + i + 1], V[:, :L + i + 1], sw.scale, [L + i])
            assert np.abs(one[0] - chunk[s * g1 + i]).max() < 1e-12


def test_after_rollback_the_pool_reads_the_committed_history():
    sw = build_spec_workload(n_q=4, n_kv=2, head_dim=8, block_size=4, dtype=BF16, hist_lens=[1, 6, 13, 20],
                             gamma=5, cycles=3, seed=5)
    o = OracleSpec(sw)
    for c in range(sw.cycles):
        o.append_cycle(c)
        o.rollback(c)
        assert (o.lens == sw.lens_before(c + 1)).all()
        for s in range(sw.num_seqs):
            L = int(o.lens[s])
            got = oracle.gather(o.pool_k, o.rows[s].blocks, L, sw.block_size).transpose(1, 0, 2)
            assert np.array_equal(got.view(np.uint16), o.hist[s][0].view(np.uint16))
            assert len(o.rows[s].blocks) == -(-L // sw.block_size)
