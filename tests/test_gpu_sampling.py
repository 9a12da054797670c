"""GPU parity of sample_tokens against the sampling oracle.

The sampled token and the kept counts are integers decided by floating
point: the oracle takes the z = logit / T decision in the same fp32 (so the
order, top-k and greedy agree exactly), and both sides evaluate the masses
exp(z - max z) and their sums in float64, so they differ only by the order
of the additions (a relative 1e-12 at most over these vocabularies). Where
the two may legitimately differ - the draw's u, or the top-p boundary
share, within 1e-9 of a step - the GPU's answer is checked to be one of the
valid neighbours; everywhere else tokens and kept counts are exact.

Rows take one of three device paths (top-k of at most 256 tokens with
chunks x k <= 8192: per-chunk candidates; top-k off on rows of at most 64
chunks: per-chunk mass histograms and per-chunk lists around each chunk's
own top-p boundary, unless more than 12288 tokens share the row's boundary
bin; otherwise one workgroup over the whole row); the cases below put rows
on every side of those lines.
"""
import numpy as np
import pytest

from oracle import sampling as S
from workloads import build_sample_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

EPS = 1e-9


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_17_amd as pkv
    pkv.load_library()


def _run(sw):
    import paged_kv_cache_17_amd as pkv
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kept = torch.empty((len(sw.u), 2), dtype=torch.int32, device="cuda")
    tok = pkv.sample_tokens(dev(sw.logits), dev(sw.temperature), dev(sw.top_k), dev(sw.top_p), dev(sw.u), kept=kept)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), kept.cpu().numpy()


def _top_p_ambiguous(x, T, k, tp):
    """True when the top-p cut falls within EPS of a cumulative share."""
    if tp >= 1.0 or T == 0:
        return False
    z = S.scaled_logits(x, T)
    order = S.desc_order(z)
    keep = order if (k <= 0 or k >= len(z)) else order[:k]
    m = np.exp(z[keep] - z.max())
    share = np.cumsum(m) / m.sum()
    return bool(np.any(np.abs(share - tp) < EPS))


def _check(sw):
    tok, kept = _run(sw)
    exact = 0
    for i in range(len(sw.u)):
        x, T, k, tp, u = sw.logits[i], float(sw.temperature[i]), int(sw.top_k[i]), float(sw.top_p[i]), float(sw.u[i])
        t, kk, kp, f = S.sample(x, T, k, tp, u)
        assert kept[i, 0] == kk, (i, kept[i], kk)
        if _top_p_ambiguous(x, T, k, tp):
            assert abs(int(kept[i, 1]) - kp) <= 1 and tok[i] >= 0
            continue
        assert kept[i, 1] == kp, (i, kept[i], kp, T, k, tp)
        if tok[i] == t:
            exact += 1
        else:
            assert f[tok[i]] > 0 and S.cdf_margin(f, u, t) < EPS, (i, tok[i], t)
    return exact


@pytest.mark.parametrize("vocab", [1, 2, 4, 10, 1000, 8192, 8193, 50257, 128256])
def test_sampling_matches_the_oracle(vocab):
    sw = build_sample_workload(rows=48, vocab=vocab, seed=vocab)
    exact = _check(sw)
    print(f"vocab {vocab}: {exact} of 48 tokens exact", flush=True)
    assert exact >= 46


def test_sampling_with_ties_and_equal_rows():
    sw = build_sample_workload(rows=64, vocab=3000, seed=5, tie_grid=0.5)
    sw.logits[:4] = 1.25          # rows of identical logits: ties everywhere
    _check(sw)


def test_ties_across_chunks():
    """Coarse logits over three 8192-wide chunks: the k-th key is tied in
    several chunks, so each chunk keeps its ties by index and the finishing
    sort keeps the lowest indices overall."""
    sw = build_sample_workload(rows=32, vocab=20000, seed=11, tie_grid=1.0, ks=(1, 5, 50, 256),
                               temps=(0.5, 1.0), ps=(1.0, 0.9, 0.3))
    sw.logits[:2] = 0.75
    _check(sw)


def test_path_boundary_on_a_wide_vocabulary():
    """300000 logits = 37 chunks: k = 221 (37 x 221 = 8177 candidates) is the
    largest on the candidate path, 222 and 257 go to the whole-row path."""
    sw = build_sample_workload(rows=16, vocab=300000, seed=3, ks=(200, 221, 222, 256, 257),
                               temps=(0.7, 1.2), ps=(1.0, 0.9))
    exact = _check(sw)
    assert exact >= 15


def test_top_k_off_rows():
    """Top-k off on a 128256-entry vocabulary (16 chunks): smooth rows of
    several spreads, a row of identical logits (its boundary bin holds every
    token, beyond what the histogram path gathers: whole-row path), rows on
    coarse grids (large tied bins, ties at the boundary) and a row whose top
    half is one tied value."""
    sw = build_sample_workload(rows=24, vocab=128256, seed=21, ks=(0,), temps=(0.5, 1.0, 2.0),
                               ps=(1.0, 0.99, 0.9, 0.5, 0.1), sigmas=(0.5, 2.0, 6.0))
    sw.logits[0] = 0.5
    sw.logits[1] = np.round(sw.logits[1] * 4.0) / 4.0
    sw.logits[2] = np.round(sw.logits[2] * 64.0) / 64.0
    sw.logits[3, ::2] = 3.0
    sw.top_p[:4] = (0.5, 0.9, 0.9, 0.3)
    exact = _check(sw)
    assert exact >= 22


def test_quotients_below_the_normal_range():
    """Logits whose quotients by T fall at or below the smallest normal fp32
    value, where the fp64 product does not round like the division (exact
    midpoints exist among subnormals), so the kernels divide for those
    values; some rows are tiny throughout, others carry a few tiny values
    among normal ones, so waves mix both cases. Candidate path (k = 5, 50),
    histogram path (k off, top-p 0.9 and 1) and both vocabulary widths."""
    for vocab, seed in ((1000, 41), (50257, 42)):
        sw = build_sample_workload(rows=16, vocab=vocab, seed=seed, ks=(0, 5, 50), temps=(0.8, 1.5, 3.0),
                                   ps=(1.0, 0.9))
        rng = np.random.default_rng(seed + 100)
        tiny = (rng.standard_normal((8, vocab)) * 2e-38).astype(np.float32)
        sw.logits[:8] = tiny                               # every quotient near or below 2^-126
        sw.top_k[:8] = (0, 5, 0, 50, 0, 5, 0, 50)          # both paths on the tiny rows
        idx = rng.integers(0, vocab, size=(8, 64))
        for r in range(8, 16):
            sw.logits[r, idx[r - 8]] = tiny[r - 8, idx[r - 8]]   # a few tiny values in normal rows
        assert np.any(np.abs(sw.logits[:8] / sw.temperature[:8, None]) < np.float32(2.0 ** -126))
        exact = _check(sw)
        assert exact >= 15, (vocab, exact)


def test_top_k_off_chunk_windows():
    """Rows built so that chunks fall on every side of the histogram path's
    per-chunk lists (each chunk lists its tokens in a few bins around its own
    top-p boundary, and the row's boundary bin is taken from those lists):
    an outlier that holds nearly all the mass (its bin is the boundary, every
    other chunk lies below it), outliers that move the row's boundary a few
    bins above most chunks' own (their lists miss it: those chunks are
    scanned again), a chunk with thousands of tied logits at the boundary
    (its list overflows: scanned), and a chunk far below the rest."""
    sw = build_sample_workload(rows=8, vocab=128256, seed=31, ks=(0,), temps=(0.8,), ps=(0.9,), sigmas=(2.0,))
    c = (128256 + 15) // 16
    sw.logits[0, 7 * c + 5] = 25.0
    sw.logits[1, 7 * c + 5] = 10.0
    sw.logits[2, 3 * c:3 * c + 3000] = 2.5
    sw.logits[3, 5 * c:6 * c] = -50.0
    sw.logits[4, 2 * c + 9] = 11.0
    sw.logits[4, 12 * c + 9] = 11.0
    sw.logits[5, 9 * c:9 * c + 6000] = 3.0
    sw.top_p[6:] = (0.5, 0.99)
    sw.logits[6, 1 * c + 1] = 10.5
    sw.logits[7, 14 * c + 77] = 9.5
    exact = _check(sw)
    assert exact >= 7


def test_top_k_off_beyond_the_histogram_rows():
    """65 chunks (one more than the histogram path merges) and 64 chunks
    exactly, top-k off: the whole-row path and the widest histogram row."""
    for vocab in (65 * 8192, 64 * 8192):
        sw = build_sample_workload(rows=6, vocab=vocab, seed=vocab % 1000, ks=(0,), temps=(0.7, 1.3),
                                   ps=(1.0, 0.9, 0.6))
        exact = _check(sw)
        assert exact >= 5, vocab


def test_invalid_temperature_gives_no_token():
    import paged_kv_cache_17_amd as pkv
    x = torch.randn(3, 5000, device="cuda")
    T = torch.tensor([-1.0, float("nan"), 1.0], device="cuda")
    k = torch.tensor([5, 0, 5], dtype=torch.int32, device="cuda")
    p = torch.ones(3, device="cuda")
    u = torch.full((3,), 0.5, device="cuda")
    kept = torch.empty((3, 2), dtype=torch.int32, device="cuda")
    tok = pkv.sample_tokens(x, T, k, p, u, kept=kept).cpu().tolist()
    assert tok[:2] == [-1, -1] and kept.cpu().tolist()[:2] == [[0, 0], [0, 0]]
    assert 0 <= tok[2] < 5000


def test_workspace_is_checked():
    import paged_kv_cache_17_amd as pkv
    x = torch.randn(2, 20000, device="cuda")
    T = torch.ones(2, device="cuda")
    k = torch.full((2,), 5, dtype=torch.int32, device="cuda")
    p = torch.ones(2, device="cuda")
    u = torch.full((2,), 0.5, device="cuda")
    need = pkv.sample_workspace_size(2, 20000)
    # per chunk: histogram, header, group sums, list of tokens near its boundary, tally
    assert need == 2 * 3 * (16384 + 16 + 512 + 4096 * 8 + 120)
    small = torch.empty(need - 8, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PagedKVError):
        pkv.sample_tokens(x, T, k, p, u, workspace=small)


def test_page_examples_on_the_device():
    import paged_kv_cache_17_amd as pkv
    rows = [np.log([0.4, 0.3, 0.2, 0.1]), np.log([0.45, 0.30, 0.15, 0.10]), np.array([1.0, 3.0, 3.0, 2.0])]
    x = torch.tensor(np.array(rows, dtype=np.float32), device="cuda")
    T = torch.tensor([1.0, 1.0, 0.0], device="cuda")
    k = torch.tensor([0, 3, 0], dtype=torch.int32, device="cuda")
    p = torch.tensor([0.65, 0.8, 1.0], device="cuda")
    u = torch.tensor([0.99, 0.99, 0.5], device="cuda")
    kept = torch.empty((3, 2), dtype=torch.int32, device="cuda")
    tok = pkv.sample_tokens(x, T, k, p, u, kept=kept).cpu().numpy()
    kept = kept.cpu().numpy()
    assert kept[0, 1] == 2 and tok[0] == 1          # top-p 0.65 keeps {0, 1}; u = 0.99 draws the last
    assert kept[1].tolist() == [3, 2] and tok[1] == 1   # top-k 3 then top-p 0.8 keeps {0, 1}
    assert tok[2] == 1                              # greedy: lowest index among tied maxima
