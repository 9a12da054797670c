"""Pins of the oracle's 8-bit K/V quantiser (chapter 5, section 4).

The chapter fixes symmetric absmax quantisation: s = max|w| / q_max with
q_max = 2^(b-1) - 1, codes round(w / s) clamped to [-q_max, q_max], values
read back as s * code, and the group-wise variant with one scale per group
of consecutive elements; exercise 5.4 prints the memory each variant takes
for a 256 x 512 matrix with FP16 scales. Its printed error percentages come
from a seeded torch run that this environment does not reproduce, so the
errors are pinned by their mathematical bound instead: every value is
within half a step (s / 2) of its input.
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import BF16, F32, build_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_byte_counts_of_the_exercise():
    g = _golden("foundations_ch5_quantization.json")
    n = g["matrix"]["rows"] * g["matrix"]["cols"]
    assert n * 2 / 1024 == g["matrix"]["fp16_kib"]
    for row in g["printed"]:
        groups = 1 if row["group"] is None else n // row["group"]
        nbytes = oracle.quant_bytes(n, row["bits"], groups, g["scale_bytes"])
        assert round(nbytes / 1024, 1) == row["kib"], row
        assert round(g["matrix"]["fp16_kib"] * 1024 / nbytes, 2) == row["ratio"], row
    assert g["q_max"]["int8"] == 2 ** 7 - 1 and g["q_max"]["int4"] == 2 ** 3 - 1


def test_half_step_bound_on_random_rows():
    rng = np.random.default_rng(1)
    for g in (1, 4, 64, 128):
        for mag in (1e-6, 1e-2, 1.0, 1e3):
            x = (rng.standard_normal((200, g)) * mag).astype(np.float32)
            codes, s = oracle.quantize_absmax(x)
            assert codes.dtype == np.int8 and np.abs(codes.astype(int)).max() <= 127
            back = oracle.dequantize(codes, s)
            step = s.astype(np.float64)[:, None]
            # half a step, plus the float32 rounding of x / s (a relative 2^-24 of <= 127 steps)
            assert (np.abs(back - x.astype(np.float64)) <= step * (0.5 + 127 * 2.0 ** -23)).all()
            # the largest element of each row lands on +-127 (unless the row's
            # maximum is below the 1e-8 floor of the scale)
            big = np.abs(x).argmax(axis=1)
            ok = np.abs(x).max(axis=1) >= 1e-8
            assert (np.abs(codes[np.arange(len(x)), big])[ok] == 127).all()


def test_exact_grids_symmetry_ties_and_zero():
    rng = np.random.default_rng(2)
    k = rng.integers(-127, 128, size=(50, 128))
    k[:, 7] = 127 * np.where(rng.random(50) < 0.5, 1, -1)
    for e in (-10, 0, 3):
        x = (k * 2.0 ** e).astype(np.float32)           # s = 2^e exactly
        codes, s = oracle.quantize_absmax(x)
        assert (s == np.float32(2.0 ** e)).all() and (codes == k).all()
        assert np.array_equal(oracle.dequantize(codes, s), x.astype(np.float64))
    x = rng.standard_normal((20, 32)).astype(np.float32)
    c1, s1 = oracle.quantize_absmax(x)
    c2, s2 = oracle.quantize_absmax(-x)
    assert np.array_equal(c2, -c1) and np.array_equal(s1, s2)
    # ties go to even: with s = 1, 2.5 -> 2, 3.5 -> 4, -2.5 -> -2
    t = np.array([[127.0, 2.5, 3.5, -2.5, 0.5, -0.5]], dtype=np.float32)
    codes, s = oracle.quantize_absmax(t)
    assert s[0] == 1.0 and codes.tolist() == [[127, 2, 4, -2, 0, 0]]
    codes, s = oracle.quantize_absmax(np.zeros((1, 8), dtype=np.float32))
    assert (codes == 0).all() and s[0] == np.float32(np.float32(1e-8) / np.float32(127))


def test_group_wise_scales_protect_against_outlier_channels():
    """The chapter's point about outliers: one scale per group confines an
    outlier's damage to its group, so group-wise error is far below
    per-tensor error when a few columns are 6-8x larger."""
    rng = np.random.default_rng(123)
    W = (rng.standard_normal((256, 512)) * 0.08).astype(np.float32)
    W[:, 17] *= 8.5
    W[:, 203] *= 6.0
    X = rng.standard_normal((16, 512))
    Y = X @ W.T.astype(np.float64)

    def err(group):
        Wg = W.reshape(1, -1) if group is None else W.reshape(-1, group)
        c, s = oracle.quantize_absmax(Wg)
        Wh = oracle.dequantize(c, s).reshape(W.shape)
        return np.linalg.norm(Y - X @ Wh.T) / np.linalg.norm(Y)

    assert err(64) < err(None) / 2


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_quantised_cache_reads_back_the_quantised_rows(dtype):
    """Through the pool and tables, a sequence's dequantised K/V equal its
    contiguous rows quantised row by row (paged = contiguous for the 8-bit
    format), and unwritten slots keep the poison."""
    L = np.array([1, 5, 16, 17, 40])
    wl = build_workload(n_q=4, n_kv=2, head_dim=8, block_size=4, dtype=dtype, hist_lens=L - 1,
                        new_lens=np.ones_like(L), seed=11)
    c = oracle.build_quant_cache(wl)
    for s in range(wl.num_seqs):
        K, V = c.sequence_kv(s)
        k, v = wl.rows(s, 0, int(wl.seq_lens[s]))
        ck, sk = oracle.quantize_absmax(oracle.widen(k, dtype))
        cv, sv = oracle.quantize_absmax(oracle.widen(v, dtype))
        assert np.array_equal(K, oracle.dequantize(ck, sk).transpose(1, 0, 2))
        assert np.array_equal(V, oracle.dequantize(cv, sv).transpose(1, 0, 2))
    used = {b for sq in c.seqs for b in sq.blocks}
    unused = [b for b in range(wl.num_blocks) if b not in used]
    assert (c.pool_k[unused] == -128).all() and np.isnan(c.scale_k[unused]).all()
