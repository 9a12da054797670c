"""The allocation-free decode step (paged_attn_decode_append_noalloc)
against paged_attn_decode_append with a caller workspace.

Both run the same kernels on the same partition, so outputs, lse and both
pools must be bit-identical (the parity bar for a variant of an entry point
that only moves its workspace). Two calls in a row on one cache family,
the second with a smaller batch, exercise reuse of the static scratch with
stale contents from the first. A batch whose partition needs more than the
scratch holds is rejected with PKV_ERR_SCRATCH_LIMIT and writes nothing.
"""
import numpy as np
import pytest

from workloads import BF16, build_workload

from gpu_harness import build_gpu_cache, check_rows, i32, out_f64, raw_to_torch

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_17_amd as pkv
    pkv.load_library()


def say(*a):
    print(*a, flush=True)


def _step_both(wl):
    """Run the step once with a caller workspace and once allocation-free,
    each on its own copy of the pre-step cache."""
    import oracle
    import paged_kv_cache_17_amd as pkv
    q = raw_to_torch(wl.q, BF16)
    kn, vn = wl.packed_new_kv()
    kn, vn = raw_to_torch(kn, BF16), raw_to_torch(vn, BF16)
    lens = i32(wl.seq_lens)
    res = []
    for noalloc in (False, True):
        c = build_gpu_cache(wl, fill_nan=True, with_new=False)
        out = torch.empty_like(q)
        lse = torch.empty((wl.num_seqs, wl.n_q), dtype=torch.float32, device="cuda")
        if noalloc:
            pkv.paged_attn_decode_append_noalloc(out, lse, q, c.k_cache, c.v_cache, kn, vn, c.table_dev, lens,
                                                 wl.max_seq_len, wl.scale)
        else:
            ws = c.workspace(wl.num_seqs, wl.n_q, wl.max_seq_len)
            pkv.paged_attn_decode_append(out, lse, q, c.k_cache, c.v_cache, kn, vn, c.table_dev, lens,
                                         wl.max_seq_len, wl.scale, ws)
        torch.cuda.synchronize()
        res.append((c, out, lse))
    (c0, o0, l0), (c1, o1, l1) = res
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "outputs differ from the workspace entry point"
    assert torch.equal(c0.k_cache.view(torch.int16), c1.k_cache.view(torch.int16))
    assert torch.equal(c0.v_cache.view(torch.int16), c1.v_cache.view(torch.int16))
    ref, _ = oracle.paged_attention_all(oracle.build_cache(wl))
    return check_rows(out_f64(o1, BF16), ref, BF16, "allocation-free step")


def test_noalloc_step_equals_workspace_step_twice_smaller_second():
    big = np.random.default_rng(71).integers(1, 4097, size=64)
    small = np.array([1, 17, 300, 1000, 2049])
    for L in (big, small):
        wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                            new_lens=np.ones_like(L), seed=int(L.sum()) % 1000)
        say(f"allocation-free step: {wl.num_seqs} sequences")
        err = _step_both(wl)
        say(f"  bit-identical to the workspace call; worst row rel err vs oracle {err:.2e}")


def test_noalloc_step_rejects_a_batch_beyond_the_scratch():
    import paged_kv_cache_17_amd as pkv
    L = np.full(2000, 3)
    wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=73)
    say("allocation-free step: 2000 sequences (beyond the scratch)")
    c = build_gpu_cache(wl, fill_nan=True, with_new=False)
    q = raw_to_torch(wl.q, BF16)
    kn, vn = wl.packed_new_kv()
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attn_decode_append_noalloc(torch.empty_like(q), None, q, c.k_cache, c.v_cache,
                                             raw_to_torch(kn, BF16), raw_to_torch(vn, BF16), c.table_dev,
                                             i32(wl.seq_lens), wl.max_seq_len, wl.scale)
    assert e.value.status == -11     # PKV_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    for s in range(wl.num_seqs):
        pos = int(wl.seq_lens[s]) - 1
        blk = int(c.table[s, pos // 16])
        assert torch.isnan(c.k_cache[blk, :, pos % 16].float()).all()
