"""Seeded inputs for shared-prefix (forked) sequences.

Parallel sampling / beam search shape: P prompts, each continued by n
branches that share the prompt's cache and then add tokens of their own.
This module only draws numbers: prompt K/V, each branch's own K/V, one
decode query per branch, one query per own token (for attending the branches'
own tokens as chunks) and the pool's allocation order. Draw order:
lengths and the permutation from ``default_rng(seed)``; prompt p's K then
V rows from ``default_rng([seed, 3, p])``; branch b's own K then V rows
from ``default_rng([seed, 4, b])``; decode queries from
``default_rng([seed, 5])``, chunk queries from ``default_rng([seed, 6])``.
Branch b = p * n + j belongs to prompt p.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from .synth import BF16, _draw


@dataclasses.dataclass
class ForkWorkload:
    name: str
    n_q: int
    n_kv: int
    head_dim: int
    block_size: int
    dtype: str
    scale: float
    branches: int                 # n branches per prompt
    prompt_lens: np.ndarray       # [P]
    own_lens: np.ndarray          # [P * n] tokens each branch adds (>= 1)
    prompt_k: list                # per prompt [len, n_kv, d] raw storage
    prompt_v: list
    own_k: list                   # per branch [own, n_kv, d]
    own_v: list
    q: np.ndarray                 # [P * n, n_q, d] one decode query per branch
    chunk_q: np.ndarray           # [sum own, n_q, d] a query per own token (chunk form)
    num_blocks: int
    table_stride: int
    alloc_order: np.ndarray

    @property
    def num_prompts(self) -> int:
        return len(self.prompt_lens)

    @property
    def num_branches(self) -> int:
        return len(self.own_lens)

    def prompt_of(self, b: int) -> int:
        return b // self.branches

    def branch_lens(self) -> np.ndarray:
        return np.array([int(self.prompt_lens[self.prompt_of(b)]) + int(self.own_lens[b])
                         for b in range(self.num_branches)], dtype=np.int64)

    def logical_kv_bytes(self) -> int:
        """K+V bytes the branches' decode reads through their tables."""
        eb = 2 if self.dtype == BF16 else 4
        return int(self.branch_lens().sum()) * self.n_kv * self.head_dim * eb * 2


def build_fork_workload(*, n_q, n_kv, head_dim, block_size, dtype, prompt_lens, branches, own_lens,
                        seed=7, name="forks", scale=None, slack=1.25) -> ForkWorkload:
    prompt_lens = np.asarray(prompt_lens, dtype=np.int64)
    own_lens = np.asarray(own_lens, dtype=np.int64)
    assert len(own_lens) == len(prompt_lens) * branches and (own_lens >= 1).all()
    rng = np.random.default_rng(seed)
    unshared = sum(-(-int(prompt_lens[b // branches] + own_lens[b]) // block_size)
                   for b in range(len(own_lens))) + sum(-(-int(P) // block_size) for P in prompt_lens)
    num_blocks = max(1, int(math.ceil(slack * unshared)))
    alloc_order = rng.permutation(num_blocks).astype(np.int32)
    longest = max(int(prompt_lens[b // branches] + own_lens[b]) for b in range(len(own_lens)))
    table_stride = -(-longest // block_size)
    pk, pv, ok, ov = [], [], [], []
    for p, P in enumerate(prompt_lens):
        r = np.random.default_rng([seed, 3, p])
        pk.append(_draw(r, (int(P), n_kv, head_dim), dtype))
        pv.append(_draw(r, (int(P), n_kv, head_dim), dtype))
    for b, g in enumerate(own_lens):
        r = np.random.default_rng([seed, 4, b])
        ok.append(_draw(r, (int(g), n_kv, head_dim), dtype))
        ov.append(_draw(r, (int(g), n_kv, head_dim), dtype))
    q = _draw(np.random.default_rng([seed, 5]), (len(own_lens), n_q, head_dim), dtype)
    chunk_q = _draw(np.random.default_rng([seed, 6]), (int(own_lens.sum()), n_q, head_dim), dtype)
    return ForkWorkload(name=name, n_q=n_q, n_kv=n_kv, head_dim=head_dim, block_size=block_size, dtype=dtype,
                        scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
                        branches=int(branches), prompt_lens=prompt_lens, own_lens=own_lens, prompt_k=pk,
                        prompt_v=pv, own_k=ok, own_v=ov, q=q, chunk_q=chunk_q, num_blocks=num_blocks,
                        table_stride=int(table_stride), alloc_order=alloc_order)


def best_of_n_workload(seed=7) -> ForkWorkload:
    """Parallel-sampling decode step: 8 prompts of 2048 tokens, 8 branches
    each with 64 tokens of their own; 32 query / 8 kv heads, d 128, block
    16, bf16."""
    return build_fork_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16,
                               prompt_lens=[2048] * 8, branches=8, own_lens=[64] * 64, seed=seed,
                               name="bestof8-8prompt-P2048+own64-32q8kv-d128-b16-bf16")
