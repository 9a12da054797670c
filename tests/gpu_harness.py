"""Helpers for the GPU parity tests: run a workload through the C ABI and
compare with the oracle. Imported by tests only."""
from __future__ import annotations

import numpy as np

from workloads import BF16

from paged_kv_cache_17_amd.replay import (  # noqa: F401  (re-exported for the tests)
    GpuSpec, build_gpu_cache, build_gpu_fork_cache, i32, raw_to_torch, torch_dtype, torch_to_raw)

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None

# Tolerances (also stated in the tests that use them):
#  fp32 K/V: max |out - ref| <= 1e-5 per element;
#  bf16 K/V: per (query row, head), max_d |out - ref| <= 2e-2 * max_d |ref|;
#  lse: |lse - ref| <= 1e-4 (fp32) / 1e-2 (bf16), i.e. sum_j exp(s_j - lse)
#  is 1 to that accuracy.
TOL_F32 = 1e-5
TOL_BF16_REL = 2e-2
TOL_LSE = {"f32": 1e-4, "bf16": 1e-2}


def run_decode(c, wl, split_tokens=0, with_lse=True):
    q = raw_to_torch(wl.q, wl.dtype)
    lse = torch.empty((wl.num_seqs, wl.n_q), dtype=torch.float32, device="cuda") if with_lse else None
    out = c.decode(q, i32(wl.seq_lens), wl.max_seq_len, wl.scale, lse=lse, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out, lse


def run_chunk(c, wl, split_tokens=0, with_lse=True):
    q = raw_to_torch(wl.q, wl.dtype)
    lse = torch.empty((q.shape[0], wl.n_q), dtype=torch.float32, device="cuda") if with_lse else None
    out = c.chunk(q, i32(wl.q_offsets), i32(wl.seq_lens), wl.max_new, wl.max_seq_len, wl.scale,
                  lse=lse, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out, lse


def out_f64(out, dtype):
    import oracle
    return oracle.widen(torch_to_raw(out, dtype), dtype)


def check_rows(got, ref, dtype, where=""):
    """Compare ``[rows, n_q, d]`` outputs to the oracle at the stated tolerance.
    Returns the worst error (absolute for fp32, relative-to-row-max for bf16)."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"non-finite output {where}"
    err = np.abs(got - ref).max(axis=-1)
    if dtype == BF16:
        scale = np.abs(ref).max(axis=-1)
        rel = err / scale
        worst = float(rel.max())
        assert worst <= TOL_BF16_REL, f"bf16 row error {worst:.3e} > {TOL_BF16_REL} {where}"
        return worst
    worst = float(err.max())
    assert worst <= TOL_F32, f"fp32 error {worst:.3e} > {TOL_F32} {where}"
    return worst


def check_lse(got, ref, dtype, where=""):
    d = float(np.abs(got - ref).max())
    assert d <= TOL_LSE[dtype], f"lse error {d:.3e} {where}"
    return d


