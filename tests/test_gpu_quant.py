"""GPU parity of the 8-bit K/V path (kv_append_q8, paged_attn_decode_q8,
paged_attn_chunk_q8 on large chunks).

Bars: the pool's codes and scales bit-exact against the oracle's
quantiser (both take the integer decision in fp32 with correctly rounded
division, ties to even; unwritten slots keep code -128 and a NaN scale);
decode outputs per (row, head) within 2e-2 of the row maximum of the
oracle's attention over the same dequantised cache (bf16 output); lse
within 1e-2.
"""
import numpy as np
import pytest

import oracle
from workloads import BF16, F32, build_workload, config_workload

from gpu_harness import build_gpu_cache, check_lse, check_rows, i32, out_f64, raw_to_torch, run_chunk

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


def _pools_match(c, ora):
    assert np.array_equal(c.table, ora.tables())
    assert np.array_equal(c.k_cache.cpu().numpy(), ora.pool_k)
    assert np.array_equal(c.v_cache.cpu().numpy(), ora.pool_v)
    # scales bit for bit, NaN poison included
    assert np.array_equal(c.k_scale.cpu().numpy().view(np.uint32), ora.scale_k.view(np.uint32))
    assert np.array_equal(c.v_scale.cpu().numpy().view(np.uint32), ora.scale_v.view(np.uint32))


def _decode(c, wl):
    q = raw_to_torch(wl.q, BF16)
    lse = torch.empty((wl.num_seqs, wl.n_q), dtype=torch.float32, device="cuda")
    out = c.decode(q, i32(wl.seq_lens), wl.max_seq_len, wl.scale, lse=lse)
    torch.cuda.synchronize()
    return out_f64(out, BF16), lse.cpu().numpy().astype(np.float64)


RAGGED = [1, 2, 15, 16, 17, 31, 33, 255, 256, 257, 1000, 2049, 3000]


@pytest.mark.parametrize("n_q,n_kv", [(32, 8), (8, 8), (16, 8), (64, 8), (6, 3)])
def test_q8_append_and_decode_match_the_oracle(n_q, n_kv):
    L = np.array(RAGGED)
    wl = build_workload(n_q=n_q, n_kv=n_kv, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=41)
    say("q8 decode", n_q, n_kv)
    c = build_gpu_cache(wl, quantized=True)
    ora = oracle.build_quant_cache(wl)
    _pools_match(c, ora)
    got, got_lse = _decode(c, wl)
    ref, ref_lse = oracle.paged_attention_all(ora)
    err = check_rows(got, ref, BF16, f"q8 {n_q}/{n_kv}")
    check_lse(got_lse, ref_lse, BF16, "q8 lse")
    say(f"  worst row rel err {err:.2e}")
    got2, _ = _decode(c, wl)
    assert np.array_equal(got, got2), "repeat run not bit-identical"


@pytest.mark.parametrize("dtype,d,bs", [(F32, 128, 16), (F32, 8, 4), (BF16, 64, 8), (BF16, 5, 3),
                                         (BF16, 128, 16), (BF16, 128, 5)])
def test_q8_append_any_shape_is_bit_exact(dtype, d, bs):
    """The quantising append takes any head_dim / block_size and fp32 or
    bf16 inputs (bf16 rows of 128 take the 16-lanes-per-row kernel); codes
    and scales equal the oracle's bit for bit."""
    L = np.array([1, bs, bs + 1, 3 * bs + 2, 70])
    wl = build_workload(n_q=4, n_kv=2, head_dim=d, block_size=bs, dtype=dtype, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=42)
    say("q8 append", dtype, d, bs)
    c = build_gpu_cache(wl, quantized=True)
    _pools_match(c, oracle.build_quant_cache(wl))


@pytest.mark.parametrize("n_q,n_kv,hist,new", [
    (32, 8, [0, 300, 1000, 2049, 4000], [512, 64, 100, 37, 9]),   # G 4: 36..2048 rows per kv head
    (8, 8, [0, 33, 1500], [40, 100, 33]),                          # G 1: 33..100 rows
    (64, 8, [17, 2000], [5, 6]),                                   # G 8: 40, 48 rows
])
def test_q8_large_chunks_match_the_oracle(n_q, n_kv, hist, new):
    """Chunks past 32 (query, head) rows per kv head over an 8-bit pool: the
    sequences' blocks are staged as bf16 s * code and the matrix-core chunk
    kernel runs over them. Every row within tolerance of the oracle's
    attention over s * code; a sequence with a table entry outside the pool
    gets NaN rows and leaves the others unchanged."""
    hist, new = np.array(hist), np.array(new)
    wl = build_workload(n_q=n_q, n_kv=n_kv, head_dim=128, block_size=16, dtype=BF16, hist_lens=hist,
                        new_lens=new, seed=47)
    say("q8 large chunks", n_q, n_kv, hist.tolist(), new.tolist())
    c = build_gpu_cache(wl, quantized=True)
    ora = oracle.build_quant_cache(wl)
    _pools_match(c, ora)
    out, lse = run_chunk(c, wl)
    got = out_f64(out, BF16)
    ref, ref_lse = oracle.paged_attention_all(ora)
    err = check_rows(got, ref, BF16, "q8 large chunks")
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, BF16, "q8 large chunks lse")
    say(f"  worst row rel err {err:.2e}")
    out2, _ = run_chunk(c, wl)
    assert np.array_equal(got, out_f64(out2, BF16)), "repeat run not bit-identical"
    # one bad table entry in the last sequence's first block
    c.table_dev[wl.num_seqs - 1, 0] = 10 ** 6
    out3, lse3 = run_chunk(c, wl)
    got3 = out_f64(out3, BF16)
    lo = int(wl.q_offsets[-2])
    assert np.isnan(got3[lo:]).all() and np.isnan(lse3[lo:].cpu().numpy()).all()
    assert np.array_equal(got3[:lo], got[:lo])


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_q8_append_past_the_staged_sequence_prefix(dtype):
    """More sequences than the quantising append stages in LDS (4096), bf16
    rows of 128 (16 lanes per row) and fp32 rows (one wave per row): codes
    and scales bit-exact."""
    rng = np.random.default_rng(37)
    S = 4200
    wl = build_workload(n_q=2, n_kv=1, head_dim=128, block_size=16, dtype=dtype,
                        hist_lens=rng.integers(0, 40, size=S), new_lens=rng.integers(1, 4, size=S), seed=37)
    say("q8 append, 4200 sequences", dtype)
    c = build_gpu_cache(wl, quantized=True)
    _pools_match(c, oracle.build_quant_cache(wl))


@pytest.mark.parametrize("n_q,n_kv,hist,new", [
    (32, 8, [0, 17, 300, 2049], [5, 5, 3, 5]),          # verification-sized: the balanced pass
    (32, 8, [0, 300, 1000, 2049], [512, 64, 100, 9]),   # past 32 rows per kv head: blocks staged as bf16
    (8, 8, [5, 1500], [40, 33]),                        # one query head per kv head, staged
])
def test_q8_chunk_step_matches_the_two_calls(n_q, n_kv, hist, new):
    """paged_attn_chunk_q8_append from the history-only state: codes, scales
    and tables bit-exact against the oracle after the call, every row
    bit-identical to kv_append_q8 + paged_attn_chunk_q8 and within the bar
    of the oracle; a sequence with a table entry outside the pool gets NaN
    rows while its other tokens are still written."""
    hist, new = np.array(hist), np.array(new)
    wl = build_workload(n_q=n_q, n_kv=n_kv, head_dim=128, block_size=16, dtype=BF16, hist_lens=hist,
                        new_lens=new, seed=53)
    say("q8 chunk step", n_q, n_kv, hist.tolist(), new.tolist())
    c = build_gpu_cache(wl, quantized=True, with_new=False)
    q = raw_to_torch(wl.q, BF16)
    kn, vn = wl.packed_new_kv()
    kn, vn = raw_to_torch(kn, BF16), raw_to_torch(vn, BF16)
    lse = torch.empty((q.shape[0], wl.n_q), dtype=torch.float32, device="cuda")
    out = c.chunk_step(q, i32(wl.q_offsets), kn, vn, i32(wl.seq_lens), wl.max_new, wl.max_seq_len, wl.scale,
                       lse=lse)
    torch.cuda.synchronize()
    ora = oracle.build_quant_cache(wl)
    _pools_match(c, ora)
    c2 = build_gpu_cache(wl, quantized=True)
    out2, lse2 = run_chunk(c2, wl)
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "not bit-identical to the two calls"
    ref, ref_lse = oracle.paged_attention_all(ora)
    err = check_rows(out_f64(out, BF16), ref, BF16, "q8 chunk step")
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, BF16, "q8 chunk step lse")
    say(f"  worst row rel err {err:.2e}")
    # a bad table entry in the last sequence's first block: that sequence's
    # rows NaN, its new tokens in valid blocks written all the same
    c3 = build_gpu_cache(wl, quantized=True, with_new=False)
    c3.table_dev[wl.num_seqs - 1, 0] = 10 ** 6
    lse3 = torch.empty_like(lse)
    out3 = c3.chunk_step(q, i32(wl.q_offsets), kn, vn, i32(wl.seq_lens), wl.max_new, wl.max_seq_len, wl.scale,
                         lse=lse3)
    torch.cuda.synchronize()
    lo = int(wl.q_offsets[-2])
    got3 = out_f64(out3, BF16)
    assert np.isnan(got3[lo:]).all() and np.isnan(lse3[lo:].cpu().numpy()).all()
    assert torch.equal(out3[:lo], out[:lo])
    c3.table_dev[wl.num_seqs - 1, 0] = int(c3.table[wl.num_seqs - 1, 0])
    _pools_match(c3, ora)


def test_q8_invalid_rows_become_nan():
    L = np.array([40, 50, 60, 70, 80])
    wl = build_workload(n_q=8, n_kv=2, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=43)
    c = build_gpu_cache(wl, quantized=True)
    lens = wl.seq_lens.copy()
    lens[1] = 0
    lens[2] = 10 ** 6
    c.table_dev[3, 1] = 10 ** 6
    q = raw_to_torch(wl.q, BF16)
    lse = torch.empty((wl.num_seqs, wl.n_q), dtype=torch.float32, device="cuda")
    out = c.decode(q, i32(lens), wl.max_seq_len, wl.scale, lse=lse)
    torch.cuda.synchronize()
    got = out_f64(out, BF16)
    for s in (1, 2, 3):
        assert np.isnan(got[s]).all() and np.isnan(lse[s].cpu().numpy()).all()
    ref, _ = oracle.paged_attention_all(oracle.build_quant_cache(wl))
    check_rows(got[[0, 4]], ref[[0, 4]], BF16, "valid q8 rows next to invalid ones")


def test_q8_many_short_sequences():
    """700 sequences of 1..300 keys at four query heads per kv head: segments
    change every few tiles, so each wave reloads queries and writes partials
    between tiles whose loads are still in flight. Every row within
    tolerance; a repeat is bit-identical."""
    L = np.random.default_rng(23).integers(1, 301, size=700)
    wl = build_workload(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=23)
    say("q8, 700 short sequences")
    c = build_gpu_cache(wl, quantized=True)
    ora = oracle.build_quant_cache(wl)
    got, got_lse = _decode(c, wl)
    ref, ref_lse = oracle.paged_attention_all(ora)
    err = check_rows(got, ref, BF16, "q8 700 short")
    check_lse(got_lse, ref_lse, BF16, "q8 700 short lse")
    say(f"  worst row rel err {err:.2e}")
    got2, _ = _decode(c, wl)
    assert np.array_equal(got, got2), "repeat run not bit-identical"


def test_q8_full_size_decode_batch_every_row():
    """The 64-sequence decode batch (lengths 512..4096) through the 8-bit
    path: whole pools (codes and scales) bit-exact, every row within
    tolerance of the oracle's attention over s * code."""
    wl = config_workload(2)
    say(f"q8 config 2: {wl.num_seqs} seqs, {int(wl.seq_lens.sum())} keys")
    c = build_gpu_cache(wl, quantized=True)
    ora = oracle.build_quant_cache(wl)
    _pools_match(c, ora)
    got, got_lse = _decode(c, wl)
    ref, ref_lse = oracle.paged_attention_all(ora)
    worst = check_rows(got, ref, BF16, "q8 cfg2")
    check_lse(got_lse, ref_lse, BF16, "q8 cfg2")
    say(f"  {wl.num_seqs} rows, worst row rel err {worst:.2e}")
