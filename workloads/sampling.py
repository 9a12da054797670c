"""Seeded inputs for token sampling: rows of logits, per-row temperature,
top-k, top-p and the uniform number of the draw.

Only numbers are drawn here (``default_rng(seed)``): logits ~ N(0, sigma^2)
per row (sigma from ``sigmas``), optionally rounded to a grid so that rows
contain ties; parameters from the given choice lists; u ~ U[0, 1).
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class SampleWorkload:
    name: str
    logits: np.ndarray        # [rows, vocab] float32
    temperature: np.ndarray   # [rows] float32
    top_k: np.ndarray         # [rows] int32
    top_p: np.ndarray         # [rows] float32
    u: np.ndarray             # [rows] float32


def build_sample_workload(rows, vocab, seed=7, temps=(0.0, 0.3, 0.8, 1.5), ks=(0, 1, 5, 50),
                          ps=(1.0, 0.95, 0.9, 0.5, 0.05), sigmas=(1.0, 4.0), tie_grid=None,
                          name="sampling") -> SampleWorkload:
    rng = np.random.default_rng(seed)
    sig = rng.choice(sigmas, size=rows)
    logits = (rng.standard_normal((rows, vocab)) * sig[:, None]).astype(np.float32)
    if tie_grid:
        logits = (np.round(logits / tie_grid) * tie_grid).astype(np.float32)
    return SampleWorkload(name=name, logits=logits,
                          temperature=rng.choice(temps, size=rows).astype(np.float32),
                          top_k=rng.choice(ks, size=rows).astype(np.int32),
                          top_p=rng.choice(ps, size=rows).astype(np.float32),
                          u=rng.random(rows).astype(np.float32))


def lm_head_workload(seed=7, top_k=50) -> SampleWorkload:
    """64 rows over a 128256-entry vocabulary: temperature 0.8, top-k 50
    (0 = off), top-p 0.9 (a common serving setting), logits ~ N(0, 4)."""
    rng = np.random.default_rng(seed)
    rows, vocab = 64, 128256
    return SampleWorkload(name=f"sample-64rows-vocab128256-T0.8-k{top_k}-p0.9",
                          logits=(rng.standard_normal((rows, vocab)) * 2.0).astype(np.float32),
                          temperature=np.full(rows, 0.8, dtype=np.float32),
                          top_k=np.full(rows, top_k, dtype=np.int32), top_p=np.full(rows, 0.9, dtype=np.float32),
                          u=rng.random(rows).astype(np.float32))
