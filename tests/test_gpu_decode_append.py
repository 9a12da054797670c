"""GPU parity of the one-call decode step (paged_attn_decode_append).

The new token of each sequence must land in the pool exactly where and as
kv_append writes it (pool bytes bit-exact against the oracle, NaN-poisoned
slots nobody wrote included), the rows must meet the bf16 bar against the
oracle (per (row, head) max_d |out - ref| <= 2e-2 * max_d |ref|; lse within
1e-2), and they must be bit-identical to kv_append followed by
paged_attn_decode on the same inputs, which run the same tile math.
"""
import numpy as np
import pytest

import oracle
from workloads import BF16, F32, build_workload

from gpu_harness import (build_gpu_cache, check_lse, check_rows, i32, out_f64, raw_to_torch, run_decode,
                         torch_to_raw)

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


def _history_only_cache(wl, quantized=False):
    """The cache as it stands before the step: history appended, tables
    already covering the new token (kvpool_ensure), new slots still NaN
    (8-bit: poison codes and scales)."""
    import paged_kv_cache_17_amd as pkv
    from gpu_harness import torch_dtype
    c = pkv.PagedKVCache(wl.num_blocks, wl.n_kv, wl.head_dim, wl.block_size,
                         torch.int8 if quantized else torch_dtype(wl.dtype),
                         wl.num_seqs, wl.table_stride, alloc_order=wl.alloc_order, fill_nan=True,
                         poison_workspace=True)
    for s in range(wl.num_seqs):
        c.ensure(s, int(wl.hist_lens[s]))
    c.upload_table()
    kh, vh = wl.packed_hist_kv()
    if len(kh):
        hs = np.zeros(wl.num_seqs + 1, dtype=np.int64)
        np.cumsum(wl.hist_lens, out=hs[1:])
        c.append(raw_to_torch(kh, wl.dtype), raw_to_torch(vh, wl.dtype), i32(np.zeros(wl.num_seqs)), i32(hs))
    for s in range(wl.num_seqs):
        c.ensure(s, int(wl.seq_lens[s]))
    c.upload_table()
    torch.cuda.synchronize()
    return c


def _step(c, wl):
    q = raw_to_torch(wl.q, wl.dtype)
    kn, vn = wl.packed_new_kv()
    lse = torch.empty((wl.num_seqs, wl.n_q), dtype=torch.float32, device="cuda")
    out = c.decode_step(q, raw_to_torch(kn, wl.dtype), raw_to_torch(vn, wl.dtype), i32(wl.seq_lens),
                        wl.max_seq_len, wl.scale, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _check_step(wl, where):
    c = _history_only_cache(wl)
    out, lse = _step(c, wl)
    ora = oracle.build_cache(wl)
    assert np.array_equal(c.table, ora.tables())
    assert np.array_equal(torch_to_raw(c.k_cache, wl.dtype).view(np.uint8), ora.pool_k.view(np.uint8))
    assert np.array_equal(torch_to_raw(c.v_cache, wl.dtype).view(np.uint8), ora.pool_v.view(np.uint8))
    ref, ref_lse = oracle.paged_attention_all(ora)
    err = check_rows(out_f64(out, wl.dtype), ref, wl.dtype, where)
    lerr = check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, wl.dtype, where)
    c2 = build_gpu_cache(wl)
    out2, lse2 = run_decode(c2, wl)
    assert torch.equal(out, out2), "not bit-identical to kv_append + paged_attn_decode"
    assert torch.equal(lse, lse2)
    return err, lerr


RAGGED = [1, 2, 15, 16, 17, 31, 33, 255, 256, 257, 1000, 2047, 2049, 3000]


@pytest.mark.parametrize("n_q,n_kv", [(32, 8), (8, 8), (16, 8), (64, 8)])
def test_step_ragged_lengths(n_q, n_kv):
    # lengths 1 (only the new token), 16 / 17 (the token fills or opens a block)
    L = np.array(RAGGED)
    wl = build_workload(n_q=n_q, n_kv=n_kv, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=31)
    say("decode step", n_q, n_kv)
    err, lerr = _check_step(wl, f"decode step {n_q}/{n_kv}")
    say(f"  worst row rel err {err:.2e} lse {lerr:.2e}")


def test_step_many_short_sequences():
    """700 sequences of 1..300 keys: most segments end inside one wave's
    range, many waves append several sequences' tokens."""
    L = np.random.default_rng(41).integers(1, 301, size=700)
    wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=41)
    say("decode step, 700 short sequences")
    err, lerr = _check_step(wl, "decode step 700")
    say(f"  worst row rel err {err:.2e} lse {lerr:.2e}")


def test_step_rejects_other_shapes():
    import paged_kv_cache_17_amd as pkv
    L = np.array([5, 9])
    wl = build_workload(n_q=4, n_kv=2, head_dim=64, block_size=16, dtype=F32, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=2)
    c = _history_only_cache(wl)
    with pytest.raises(pkv.PagedKVError) as e:
        _step(c, wl)
    assert e.value.status == -3   # PKV_ERR_UNSUPPORTED


@pytest.mark.parametrize("many", [False, True])
def test_step_invalid_length_row_is_nan_others_unchanged(many):
    """A length beyond max_seq_len: that sequence's rows are NaN (and it gets
    no append); every other row still meets the bar against the oracle (the
    rejected sequence's tiles leave the partition, so the others' rounding
    may change). With 14 sequences the append is folded into the split
    pass, with 700 it runs as its own launch."""
    rng = np.random.default_rng(43)
    L = rng.integers(1, 301, size=700) if many else np.array(RAGGED)
    wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=43)
    say("decode step, one invalid length, many =", many)
    ora = oracle.build_cache(wl)
    ref, ref_lse = oracle.paged_attention_all(ora)
    c = _history_only_cache(wl)
    bad = 3
    lens = wl.seq_lens.copy()
    lens[bad] = wl.max_seq_len + 5
    q = raw_to_torch(wl.q, wl.dtype)
    kn, vn = wl.packed_new_kv()
    lse = torch.empty((wl.num_seqs, wl.n_q), dtype=torch.float32, device="cuda")
    out = c.decode_step(q, raw_to_torch(kn, wl.dtype), raw_to_torch(vn, wl.dtype), i32(lens), wl.max_seq_len,
                        wl.scale, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(out[bad].float()).all() and torch.isnan(lse[bad]).all()
    keep = [s for s in range(wl.num_seqs) if s != bad]
    check_rows(out_f64(out, wl.dtype)[keep], ref[keep], wl.dtype, "invalid-length step")
    check_lse(lse.cpu().numpy().astype(np.float64)[keep], ref_lse[keep], wl.dtype, "invalid-length step")
    # the rejected sequence's new slot was not written (still the NaN poison)
    pos = int(wl.seq_lens[bad]) - 1
    blk = int(c.table[bad, pos // 16])
    assert torch.isnan(c.k_cache[blk, :, pos % 16].float()).all()


# --------------------------------------------------------------- 8-bit pool ---


def _check_step_q8(wl, where):
    """8-bit pool: codes and scales bit-identical to kv_append_q8 of the new
    tokens (the oracle pins kv_append_q8's codes in test_gpu_quant), and the
    rows bit-identical to paged_attn_decode_q8 after it."""
    c = _history_only_cache(wl, quantized=True)
    out, lse = _step(c, wl)
    c2 = build_gpu_cache(wl, quantized=True)
    out2, lse2 = run_decode(c2, wl)
    assert np.array_equal(c.table, c2.table)
    assert torch.equal(c.k_cache, c2.k_cache) and torch.equal(c.v_cache, c2.v_cache), "codes differ"
    assert np.array_equal(c.k_scale.cpu().numpy().view(np.uint32), c2.k_scale.cpu().numpy().view(np.uint32))
    assert np.array_equal(c.v_scale.cpu().numpy().view(np.uint32), c2.v_scale.cpu().numpy().view(np.uint32))
    assert torch.equal(out, out2), "not bit-identical to kv_append_q8 + paged_attn_decode_q8"
    assert torch.equal(lse, lse2)


@pytest.mark.parametrize("n_q,n_kv", [(32, 8), (8, 8), (16, 8), (64, 8)])
def test_step_q8_ragged_lengths(n_q, n_kv):
    L = np.array(RAGGED)
    wl = build_workload(n_q=n_q, n_kv=n_kv, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=33)
    say("8-bit decode step", n_q, n_kv)
    _check_step_q8(wl, f"8-bit decode step {n_q}/{n_kv}")


def test_step_q8_many_short_sequences():
    """5600 segments, more than the pass's waves: the append runs as its own
    launch inside the call."""
    L = np.random.default_rng(45).integers(1, 301, size=700)
    wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=45)
    say("8-bit decode step, 700 short sequences")
    _check_step_q8(wl, "8-bit decode step 700")


# ------------------------------------------------------------ chunk steps ---


def _check_chunk_step(wl, where):
    """paged_attn_chunk_append against kv_append + paged_attn_chunk: pool
    bytes bit-exact against the oracle, rows within the bar and
    bit-identical to the two-call path."""
    from gpu_harness import run_chunk
    c = _history_only_cache(wl)
    q = raw_to_torch(wl.q, wl.dtype)
    kn, vn = wl.packed_new_kv()
    lse = torch.empty((q.shape[0], wl.n_q), dtype=torch.float32, device="cuda")
    out = c.chunk_step(q, i32(wl.q_offsets), raw_to_torch(kn, wl.dtype), raw_to_torch(vn, wl.dtype),
                       i32(wl.seq_lens), wl.max_new, wl.max_seq_len, wl.scale, lse=lse)
    torch.cuda.synchronize()
    ora = oracle.build_cache(wl)
    assert np.array_equal(c.table, ora.tables())
    assert np.array_equal(torch_to_raw(c.k_cache, wl.dtype).view(np.uint8), ora.pool_k.view(np.uint8))
    assert np.array_equal(torch_to_raw(c.v_cache, wl.dtype).view(np.uint8), ora.pool_v.view(np.uint8))
    ref, ref_lse = oracle.paged_attention_all(ora)
    check_rows(out_f64(out, wl.dtype), ref, wl.dtype, where)
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, wl.dtype, where)
    c2 = build_gpu_cache(wl)
    out2, lse2 = run_chunk(c2, wl)
    assert torch.equal(out, out2), "not bit-identical to kv_append + paged_attn_chunk"
    assert torch.equal(lse, lse2)


@pytest.mark.parametrize("n_q,n_kv", [(32, 8), (8, 8), (16, 8)])
def test_chunk_step_verify_sized(n_q, n_kv):
    """5 new tokens per sequence (a verification pass), lengths that put the
    chunk across a block boundary or fill a block: the balanced small-chunk
    pass after the call's own append."""
    L = np.array([5, 6, 16, 17, 20, 21, 33, 300, 1000, 2051])
    wl = build_workload(n_q=n_q, n_kv=n_kv, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 5,
                        new_lens=np.full_like(L, 5), seed=51)
    say("chunk step, 5 tokens", n_q, n_kv)
    _check_chunk_step(wl, f"chunk step {n_q}/{n_kv}")


def test_chunk_step_many_sequences():
    """200 sequences x 8 kv heads on the balanced small-chunk pass."""
    L = np.random.default_rng(53).integers(5, 400, size=200)
    wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 5,
                        new_lens=np.full_like(L, 5), seed=53)
    say("chunk step, 200 sequences")
    _check_chunk_step(wl, "chunk step 200")


def test_chunk_step_large_chunks_and_decode_rows():
    """Chunks of 40 (the matrix-core chunk kernel, the append fused into it)
    beside 1-token rows."""
    L = np.array([40, 57, 300, 1, 90])
    C = np.array([40, 40, 40, 1, 1])
    wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - C,
                        new_lens=C, seed=55)
    say("chunk step, chunks of 40")
    _check_chunk_step(wl, "chunk step 40")


def test_chunk_step_fused_append_with_bad_rows():
    """The matrix-core chunk step with its append fused in, where one
    sequence's table names a block outside the pool (for a cached key) and
    another's length is out of range: those sequences' rows are NaN; the
    first still has its new tokens written (their blocks are valid), the
    second gets no append; every other row and pool byte as the oracle."""
    L = np.array([300, 200, 97, 150])
    C = np.array([64, 40, 33, 50])
    wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - C,
                        new_lens=C, seed=57)
    say("fused chunk step, bad rows")
    c = build_gpu_cache(wl, with_new=False)
    c.table_dev[1, 0] = 10 ** 6                   # a cached key's block outside the pool
    lens = wl.seq_lens.copy()
    lens[2] = wl.table_stride * wl.block_size + 1  # longer than the table holds
    q = raw_to_torch(wl.q, wl.dtype)
    kn, vn = wl.packed_new_kv()
    lse = torch.empty((q.shape[0], wl.n_q), dtype=torch.float32, device="cuda")
    out = c.chunk_step(q, i32(wl.q_offsets), raw_to_torch(kn, wl.dtype), raw_to_torch(vn, wl.dtype), i32(lens),
                       wl.max_new, int(lens.max()), wl.scale, lse=lse)
    torch.cuda.synchronize()
    got = out_f64(out, wl.dtype)
    qo = wl.q_offsets
    for s in (1, 2):
        assert np.isnan(got[qo[s]:qo[s + 1]]).all() and np.isnan(lse[qo[s]:qo[s + 1]].cpu().numpy()).all()
    ora = oracle.build_cache(wl)
    ref, _ = oracle.paged_attention_all(ora)
    for s in (0, 3):
        check_rows(got[qo[s]:qo[s + 1]], ref[qo[s]:qo[s + 1]], wl.dtype, f"valid sequence {s}")
    # pools: as the oracle's except sequence 2's new tokens, which stay as before the call
    kp = torch_to_raw(c.k_cache, wl.dtype).view(np.uint16).copy()
    vp = torch_to_raw(c.v_cache, wl.dtype).view(np.uint16).copy()
    ok, ov = ora.pool_k.view(np.uint16).copy(), ora.pool_v.view(np.uint16).copy()
    hist = build_gpu_cache(wl, with_new=False)
    hk = torch_to_raw(hist.k_cache, wl.dtype).view(np.uint16)
    hv = torch_to_raw(hist.v_cache, wl.dtype).view(np.uint16)
    for p in range(int(wl.hist_lens[2]), int(wl.seq_lens[2])):
        blk, slot = int(c.table[2, p // wl.block_size]), p % wl.block_size
        ok[blk, :, slot] = hk[blk, :, slot]
        ov[blk, :, slot] = hv[blk, :, slot]
    assert np.array_equal(kp, ok) and np.array_equal(vp, ov)


# ------------------------------------------------ errors before any write ---


def _slot_is_poison(c, wl, s, quantized=False):
    pos = int(wl.seq_lens[s]) - 1
    blk = int(c.table[s, pos // wl.block_size])
    if quantized:
        return bool((c.k_cache[blk, :, pos % wl.block_size] == -128).all()) and \
            bool(torch.isnan(c.k_scale[blk, :, pos % wl.block_size]).all())
    return bool(torch.isnan(c.k_cache[blk, :, pos % wl.block_size].float()).all())


def _smallest_accepted(call, hi):
    """Smallest workspace byte count a call accepts, by bisection. ``call(n)``
    runs an entry point with n bytes of workspace and returns its status."""
    lo = 0                      # rejected (a call with no room fails)
    assert call(hi) == 0
    while hi - lo > 1:
        mid = (lo + hi) // 2
        st = call(mid)
        assert st in (0, -6), st
        lo, hi = (lo, mid) if st == 0 else (mid, hi)
    return hi


@pytest.mark.parametrize("quantized", [False, True])
def test_step_too_small_workspace_writes_nothing(quantized):
    """700 sequences (the append is a launch of its own inside the call): a
    workspace one byte short of what the step's partition needs, or
    misaligned, is rejected before the append, so every new slot still holds
    the poison. The exact need is found with the decode call of the same
    partition, which writes nothing into the pool."""
    import paged_kv_cache_17_amd as pkv
    from paged_kv_cache_17_amd import binding as B
    L = np.random.default_rng(47).integers(1, 301, size=700)
    wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=47)
    say("decode step, workspace too small, 8-bit =", quantized)
    c = _history_only_cache(wl, quantized=quantized)
    q = raw_to_torch(wl.q, wl.dtype)
    kn, vn = wl.packed_new_kv()
    kn, vn = raw_to_torch(kn, wl.dtype), raw_to_torch(vn, wl.dtype)
    need = B.paged_attn_workspace_size(wl.num_seqs, wl.n_q, wl.n_kv, 128, 16, wl.max_seq_len, 0)
    big = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lens = i32(wl.seq_lens)

    def decode(nbytes):
        try:
            if quantized:
                pkv.paged_attn_decode_q8(out, None, q, c.k_cache, c.v_cache, c.k_scale, c.v_scale, c.table_dev,
                                         lens, wl.max_seq_len, wl.scale, big[:nbytes])
            else:
                pkv.paged_attn_decode(out, None, q, c.k_cache, c.v_cache, c.table_dev, lens, wl.max_seq_len,
                                      wl.scale, big[:nbytes])
            return 0
        except pkv.PagedKVError as e:
            return e.status

    exact = _smallest_accepted(decode, need)
    torch.cuda.synchronize()
    say(f"  step needs {exact} of the {need} bytes paged_attn_workspace_size reports")
    for ws, status in ((big[:exact - 1], -6), (big[1:exact + 1], -2)):
        with pytest.raises(pkv.PagedKVError) as e:
            if quantized:
                pkv.paged_attn_decode_q8_append(out, None, q, c.k_cache, c.v_cache, c.k_scale, c.v_scale, kn, vn,
                                                c.table_dev, lens, wl.max_seq_len, wl.scale, ws)
            else:
                pkv.paged_attn_decode_append(out, None, q, c.k_cache, c.v_cache, kn, vn, c.table_dev, lens,
                                             wl.max_seq_len, wl.scale, ws)
        assert e.value.status == status
    torch.cuda.synchronize()
    assert all(_slot_is_poison(c, wl, s, quantized) for s in range(wl.num_seqs))
    # with exactly the bytes it needs the step runs and writes every new slot
    if quantized:
        pkv.paged_attn_decode_q8_append(out, None, q, c.k_cache, c.v_cache, c.k_scale, c.v_scale, kn, vn,
                                        c.table_dev, lens, wl.max_seq_len, wl.scale, big[:exact])
    else:
        pkv.paged_attn_decode_append(out, None, q, c.k_cache, c.v_cache, kn, vn, c.table_dev, lens,
                                     wl.max_seq_len, wl.scale, big[:exact])
    torch.cuda.synchronize()
    assert not any(_slot_is_poison(c, wl, s, quantized) for s in range(wl.num_seqs))


def test_chunk_step_too_small_workspace_writes_nothing():
    """A chunk step on the split path (split_tokens > 0) with a workspace one
    byte short is rejected before its append."""
    import paged_kv_cache_17_amd as pkv
    from paged_kv_cache_17_amd import binding as B
    L = np.array([40, 57, 300, 90])
    C = np.array([40, 40, 40, 1])
    wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - C,
                        new_lens=C, seed=57)
    say("chunk step, workspace too small")
    c = _history_only_cache(wl)
    q = raw_to_torch(wl.q, wl.dtype)
    kn, vn = wl.packed_new_kv()
    need = B.paged_attn_workspace_size(q.shape[0], wl.n_q, wl.n_kv, 128, 16, wl.max_seq_len, 64)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attn_chunk_append(torch.empty_like(q), None, q, i32(wl.q_offsets), c.k_cache, c.v_cache,
                                    raw_to_torch(kn, wl.dtype), raw_to_torch(vn, wl.dtype), c.table_dev,
                                    i32(wl.seq_lens), wl.max_new, wl.max_seq_len, wl.scale, ws[:need - 1],
                                    split_tokens=64)
    assert e.value.status == -6
    torch.cuda.synchronize()
    for s in range(wl.num_seqs):
        for p in range(int(wl.hist_lens[s]), int(wl.seq_lens[s])):
            blk = int(c.table[s, p // 16])
            assert torch.isnan(c.k_cache[blk, :, p % 16].float()).all()
