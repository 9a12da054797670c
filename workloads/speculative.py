"""Seeded inputs for speculative-decoding cycles over a paged cache.

Each cycle of each sequence appends gamma + 1 tokens (the token sampled in
the previous cycle, then gamma drafted tokens) and verifies them with one
causal chunk of gamma + 1 queries; then the number of drafts the target
accepts (0..gamma) is drawn, and the cache is rolled back to the committed
length. This module only draws numbers: history lengths, the pool order,
history and per-cycle K/V, per-cycle queries and accepted counts (the
accept/reject outcome is an input here, not computed). Draw order: lengths,
permutation and accepted counts from ``default_rng(seed)``; sequence s's
history K then V from ``default_rng([seed, 7, s])``; cycle c's K then V
rows of sequence s from ``default_rng([seed, 8, c, s])``; cycle c's queries
from ``default_rng([seed, 9, c])``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from .synth import BF16, _draw


@dataclasses.dataclass
class SpecWorkload:
    name: str
    n_q: int
    n_kv: int
    head_dim: int
    block_size: int
    dtype: str
    scale: float
    gamma: int
    hist_lens: np.ndarray          # [S] committed tokens before the first cycle
    accepted: np.ndarray           # [cycles, S] drafts accepted in each cycle (0..gamma)
    hist_k: list                   # per sequence [hist, n_kv, d]
    hist_v: list
    cyc_k: list                    # [cycle][S] -> [gamma + 1, n_kv, d]
    cyc_v: list
    cyc_q: list                    # [cycle] -> [S * (gamma + 1), n_q, d]
    num_blocks: int
    table_stride: int
    alloc_order: np.ndarray

    @property
    def num_seqs(self) -> int:
        return len(self.hist_lens)

    @property
    def cycles(self) -> int:
        return self.accepted.shape[0]

    def lens_before(self, c: int) -> np.ndarray:
        """Committed length of every sequence when cycle c starts."""
        return self.hist_lens + (self.accepted[:c] + 1).sum(axis=0)


def build_spec_workload(*, n_q, n_kv, head_dim, block_size, dtype, hist_lens, gamma, cycles, seed=7,
                        name="speculative", scale=None) -> SpecWorkload:
    hist = np.asarray(hist_lens, dtype=np.int64)
    S = len(hist)
    rng = np.random.default_rng(seed)
    longest = int(hist.max()) + cycles * (gamma + 1)
    need = sum(-(-(int(L) + cycles * (gamma + 1)) // block_size) for L in hist)
    num_blocks = max(1, int(math.ceil(1.25 * need)))
    alloc_order = rng.permutation(num_blocks).astype(np.int32)
    accepted = rng.integers(0, gamma + 1, size=(cycles, S))
    hk, hv = [], []
    for s in range(S):
        r = np.random.default_rng([seed, 7, s])
        hk.append(_draw(r, (int(hist[s]), n_kv, head_dim), dtype))
        hv.append(_draw(r, (int(hist[s]), n_kv, head_dim), dtype))
    ck, cv, cq = [], [], []
    for c in range(cycles):
        ks, vs = [], []
        for s in range(S):
            r = np.random.default_rng([seed, 8, c, s])
            ks.append(_draw(r, (gamma + 1, n_kv, head_dim), dtype))
            vs.append(_draw(r, (gamma + 1, n_kv, head_dim), dtype))
        ck.append(ks)
        cv.append(vs)
        cq.append(_draw(np.random.default_rng([seed, 9, c]), (S * (gamma + 1), n_q, head_dim), dtype))
    return SpecWorkload(name=name, n_q=n_q, n_kv=n_kv, head_dim=head_dim, block_size=block_size, dtype=dtype,
                        scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)), gamma=int(gamma),
                        hist_lens=hist, accepted=accepted, hist_k=hk, hist_v=hv, cyc_k=ck, cyc_v=cv, cyc_q=cq,
                        num_blocks=num_blocks, table_stride=-(-longest // block_size), alloc_order=alloc_order)


def verify_workload(seed=7) -> SpecWorkload:
    """The 64-sequence decode batch (lengths uniform in 512..4096) verifying
    gamma = 4 drafts per cycle: chunks of 5 queries; 32 query / 8 kv heads,
    d 128, block 16, bf16."""
    lens = np.random.default_rng(seed).integers(512, 4097, size=64)
    return build_spec_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=lens - 5,
                               gamma=4, cycles=2, seed=seed,
                               name="verify-64seq-L512..4096-gamma4-32q8kv-d128-b16-bf16")
