"""The balanced decode pass's work split and partial-slot rule, checked on the CPU.

The device code hands wave w < W' = min(W, T) the tiles
[floor(w T / W'), floor((w+1) T / W')), writes the partial of wave w for
segment sigma to slot w + sigma, and the merge pass looks for a segment's
partials at w + sigma for w from wave_of(first tile) to wave_of(last tile),
wave_of(t) = ceil((t + 1) W' / T) - 1. These integer formulas are restated
here and checked for: every tile covered once, no empty wave, slots unique
and below W + #segments, and the merge reading exactly the written slots.
"""
import random


def wave_range(w, W, T):
    return (w * T) // W, ((w + 1) * T) // W


def wave_of(t, W, T):
    return ((t + 1) * W + T - 1) // T - 1


def _check(seg_lengths, W_grid):
    T = sum(seg_lengths)
    W = min(W_grid, T)
    starts = [0]
    for n in seg_lengths:
        starts.append(starts[-1] + n)
    seg_of = []
    for sgm, n in enumerate(seg_lengths):
        seg_of += [sgm] * n
    written = {}
    covered = [0] * T
    for w in range(W):
        lo, hi = wave_range(w, W, T)
        assert hi > lo, "empty wave"
        for t in range(lo, hi):
            covered[t] += 1
            assert wave_of(t, W, T) == w
        for sgm in sorted({seg_of[t] for t in range(lo, hi)}):
            slot = w + sgm
            assert slot not in written
            assert slot < W_grid + len(seg_lengths)
            written[slot] = (w, sgm)
    assert covered == [1] * T
    for sgm, n in enumerate(seg_lengths):
        if n == 0:
            continue
        w_lo = wave_of(starts[sgm], W, T)
        w_hi = wave_of(starts[sgm] + n - 1, W, T)
        reads = [w + sgm for w in range(w_lo, w_hi + 1)]
        assert all(written.get(r, (None, None))[1] == sgm for r in reads)
        assert sorted(r for r, (_, s2) in written.items() if s2 == sgm) == reads


def test_partition_rules_hold():
    rng = random.Random(0)
    for _ in range(400):
        n_seg = rng.randint(1, 40)
        lengths = [rng.choice([1, 1, 2, 3, 8, 40, 200]) for _ in range(n_seg)]
        W = rng.choice([1, 2, 3, 7, 64, 100, 2048])
        _check(lengths, W)


def test_fewer_tiles_than_waves():
    _check([1, 1, 1], 8)
    _check([5, 2, 3], 2048)
