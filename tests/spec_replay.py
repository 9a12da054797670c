"""Replays of speculative-decoding cycles for the tests (oracle side and
library side), kept apart so both GPU tests and CPU pins can use them."""
from __future__ import annotations

import numpy as np

import oracle
from workloads.synth import BF16, poison_bits, storage_dtype


class OracleSpec:
    """The oracle's pool and rows driven through verify / rollback cycles."""

    def __init__(self, sw):
        self.sw = sw
        B = sw.block_size
        shape = (sw.num_blocks, sw.n_kv, B, sw.head_dim)
        fill = poison_bits(sw.dtype) if sw.dtype == BF16 else np.float32(np.nan)
        self.pool_k = np.full(shape, fill, dtype=storage_dtype(sw.dtype))
        self.pool_v = self.pool_k.copy()
        self.alloc = oracle.BlockAllocator(sw.num_blocks, sw.alloc_order)
        self.rows = [oracle.SequenceBlocks(B) for _ in range(sw.num_seqs)]
        self.lens = np.array(sw.hist_lens, dtype=np.int64)
        self.hist = [(sw.hist_k[s], sw.hist_v[s]) for s in range(sw.num_seqs)]   # committed rows
        for s in range(sw.num_seqs):
            self.rows[s].ensure(self.alloc, int(self.lens[s]))
            oracle.append(self.pool_k, self.pool_v, self.rows[s].blocks, 0, sw.hist_k[s], sw.hist_v[s], B)

    def append_cycle(self, c):
        sw = self.sw
        for s in range(sw.num_seqs):
            self.rows[s].ensure(self.alloc, int(self.lens[s]) + sw.gamma + 1)
            oracle.append(self.pool_k, self.pool_v, self.rows[s].blocks, int(self.lens[s]), sw.cyc_k[c][s],
                          sw.cyc_v[c][s], sw.block_size)

    def verify(self, c):
        """Outputs of the cycle's gamma + 1 queries per sequence, each query
        attending causally over the committed history plus the cycle's tokens
        up to itself: [S * (gamma + 1), n_q, d]."""
        sw = self.sw
        g1 = sw.gamma + 1
        outs = []
        for s in range(sw.num_seqs):
            k = np.concatenate([self.hist[s][0], sw.cyc_k[c][s]])
            v = np.concatenate([self.hist[s][1], sw.cyc_v[c][s]])
            K = oracle.widen(k, sw.dtype).transpose(1, 0, 2)
            V = oracle.widen(v, sw.dtype).transpose(1, 0, 2)
            L = int(self.lens[s])
            q = oracle.widen(sw.cyc_q[c][s * g1:(s + 1) * g1], sw.dtype)
            o, _, _ = oracle.attention(q, K, V, sw.scale, np.arange(L, L + g1))
            outs.append(o)
        return np.concatenate(outs)

    def rollback(self, c):
        sw = self.sw
        for s in range(sw.num_seqs):
            keep = int(sw.accepted[c, s]) + 1
            self.rows[s].truncate(self.alloc, int(self.lens[s]) + keep)
            self.hist[s] = (np.concatenate([self.hist[s][0], sw.cyc_k[c][s][:keep]]),
                            np.concatenate([self.hist[s][1], sw.cyc_v[c][s][:keep]]))
            self.lens[s] += keep

    def tables(self):
        t = np.full((self.sw.num_seqs, self.sw.table_stride), -1, dtype=np.int32)
        for s, r in enumerate(self.rows):
            t[s, :len(r.blocks)] = r.blocks
        return t


class OracleSpecQ8(OracleSpec):
    """The same cycles over an 8-bit pool: codes (unwritten: -128) and one
    fp32 scale per (block, kv head, slot) (unwritten: NaN); verification
    attends over s * code of the committed history plus the cycle's tokens."""

    def __init__(self, sw):
        self.sw = sw
        B = sw.block_size
        shape = (sw.num_blocks, sw.n_kv, B, sw.head_dim)
        self.pool_k = np.full(shape, oracle.QUANT_POISON_CODE, dtype=np.int8)
        self.pool_v = self.pool_k.copy()
        self.scale_k = np.full(shape[:3], np.nan, dtype=np.float32)
        self.scale_v = self.scale_k.copy()
        self.alloc = oracle.BlockAllocator(sw.num_blocks, sw.alloc_order)
        self.rows = [oracle.SequenceBlocks(B) for _ in range(sw.num_seqs)]
        self.lens = np.array(sw.hist_lens, dtype=np.int64)
        self.hist = [(sw.hist_k[s], sw.hist_v[s]) for s in range(sw.num_seqs)]
        for s in range(sw.num_seqs):
            self.rows[s].ensure(self.alloc, int(self.lens[s]))
            oracle.append_quantized(self.pool_k, self.pool_v, self.scale_k, self.scale_v, self.rows[s].blocks, 0,
                                    sw.hist_k[s], sw.hist_v[s], B, sw.dtype)

    def append_cycle(self, c):
        sw = self.sw
        for s in range(sw.num_seqs):
            self.rows[s].ensure(self.alloc, int(self.lens[s]) + sw.gamma + 1)
            oracle.append_quantized(self.pool_k, self.pool_v, self.scale_k, self.scale_v, self.rows[s].blocks,
                                    int(self.lens[s]), sw.cyc_k[c][s], sw.cyc_v[c][s], sw.block_size, sw.dtype)

    def verify(self, c):
        sw = self.sw
        g1 = sw.gamma + 1
        outs = []
        for s in range(sw.num_seqs):
            K = oracle.quantized_rows(np.concatenate([self.hist[s][0], sw.cyc_k[c][s]]), sw.dtype).transpose(1, 0, 2)
            V = oracle.quantized_rows(np.concatenate([self.hist[s][1], sw.cyc_v[c][s]]), sw.dtype).transpose(1, 0, 2)
            L = int(self.lens[s])
            q = oracle.widen(sw.cyc_q[c][s * g1:(s + 1) * g1], sw.dtype)
            o, _, _ = oracle.attention(q, K, V, sw.scale, np.arange(L, L + g1))
            outs.append(o)
        return np.concatenate(outs)
