"""GPU parity of speculative-decoding cycles: verify chunks and rollback.

Each cycle appends gamma + 1 tokens per sequence, verifies them with one
causal chunk of gamma + 1 queries (chapter 5 section 5: one target pass over
the drafts), then rolls every sequence back to its committed length (the
drafts after the first rejection are discarded; serving tutorial, question
on speculative decoding). Checked against the oracle doing the same steps:
tables after rollback and pool bytes bit-exact (stale slots included),
verification outputs within the stated tolerance of attention over the
committed history plus the cycle's tokens.
"""
import numpy as np
import pytest

import oracle
from workloads import BF16, F32, build_spec_workload

from gpu_harness import GpuSpec, check_rows, out_f64, torch_to_raw
from spec_replay import OracleSpec

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_17_amd as pkv
    pkv.load_library()


CASES = {
    "bf16-gqa": dict(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16,
                     hist_lens=[1, 11, 15, 16, 60, 63, 500, 1200], gamma=4, cycles=3, seed=51),
    "bf16-gamma7": dict(n_q=16, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=[3, 29, 250],
                        gamma=7, cycles=2, seed=52),
    "f32-small": dict(n_q=4, n_kv=2, head_dim=8, block_size=4, dtype=F32, hist_lens=[1, 2, 7, 12], gamma=3,
                      cycles=3, seed=53),
}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("split", [0, 64])
def test_verify_and_rollback_cycles(case, split):
    sw = build_spec_workload(**CASES[case])
    print(f"speculative {case} split {split}: lens {sw.hist_lens.tolist()}, accepted {sw.accepted.tolist()}",
          flush=True)
    ora = OracleSpec(sw)
    gpu = GpuSpec(sw)
    for c in range(sw.cycles):
        ora.append_cycle(c)
        gpu.append_cycle(c)
        out = gpu.verify(c, split_tokens=split)
        torch.cuda.synchronize()
        assert np.array_equal(gpu.c.table, ora.tables())
        assert np.array_equal(torch_to_raw(gpu.c.k_cache, sw.dtype).view(np.uint8), ora.pool_k.view(np.uint8))
        assert np.array_equal(torch_to_raw(gpu.c.v_cache, sw.dtype).view(np.uint8), ora.pool_v.view(np.uint8))
        check_rows(out_f64(out, sw.dtype), ora.verify(c), sw.dtype, f"{case} cycle {c}")
        ora.rollback(c)
        gpu.rollback(c)
        assert np.array_equal(gpu.c.table, ora.tables())
        assert (gpu.lens == ora.lens).all()
        assert gpu.c.pool.kvpool_free_ids().tolist() == ora.alloc.free_ids()
    for s in range(sw.num_seqs):
        gpu.c.release(s)
    assert gpu.c.pool.kvpool_num_free() == sw.num_blocks


@pytest.mark.parametrize("case", ["bf16-gqa", "bf16-gamma7"])
def test_verify_and_rollback_cycles_over_an_8bit_pool(case):
    """The same cycles over an 8-bit pool: kv_append_q8 writes each cycle's
    tokens, paged_attn_chunk_q8 verifies them as one causal chunk, and
    kvpool_truncate rolls back. Codes, scales and tables bit-exact against
    the oracle's quantised replay; outputs within the bar against attention
    over s * code of the committed history plus the cycle's tokens."""
    from spec_replay import OracleSpecQ8
    sw = build_spec_workload(**CASES[case])
    print(f"8-bit speculative {case}: lens {sw.hist_lens.tolist()}, accepted {sw.accepted.tolist()}", flush=True)
    ora = OracleSpecQ8(sw)
    gpu = GpuSpec(sw, quantized=True)
    for c in range(sw.cycles):
        ora.append_cycle(c)
        gpu.append_cycle(c)
        out = gpu.verify(c)
        torch.cuda.synchronize()
        assert np.array_equal(gpu.c.table, ora.tables())
        assert np.array_equal(gpu.c.k_cache.cpu().numpy(), ora.pool_k)
        assert np.array_equal(gpu.c.v_cache.cpu().numpy(), ora.pool_v)
        assert np.array_equal(gpu.c.k_scale.cpu().numpy().view(np.uint32), ora.scale_k.view(np.uint32))
        assert np.array_equal(gpu.c.v_scale.cpu().numpy().view(np.uint32), ora.scale_v.view(np.uint32))
        check_rows(out_f64(out, sw.dtype), ora.verify(c), sw.dtype, f"8-bit {case} cycle {c}")
        ora.rollback(c)
        gpu.rollback(c)
        assert np.array_equal(gpu.c.table, ora.tables())
    for s in range(sw.num_seqs):
        gpu.c.release(s)
    assert gpu.c.pool.kvpool_num_free() == sw.num_blocks
