"""Seeded synthetic workloads shaped like the paged-KV decode configurations.

Everything here is input preparation: lengths drawn from the stated
distributions, a permutation that fixes the pool's allocation order, K/V
histories and queries drawn from N(0, 1). bf16 data is produced from fp32
draws by round-to-nearest-even and kept as raw uint16 bit patterns, so a
consumer decides itself how to widen it.

Draw order for one workload: lengths, then the pool permutation, from
``numpy.random.default_rng(seed)``; sequence ``s``'s K rows then V rows
(history and new tokens together) from ``default_rng([seed, 1, s])``; all
query rows from ``default_rng([seed, 2])``. Per-sequence streams make the
draw independent of how many threads fill the arrays.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np

F32 = "f32"
BF16 = "bf16"

CONFIG_NAMES = {
    1: "tiny-lab-mha-d4-b4-fp32",
    2: "decode-64seq-L512..4096-32q8kv-d128-b16-bf16",
    3: "decode-256seq-L128..8192log-32q8kv-d128-b16-bf16",
    4: "decode-8seq-L32768-32q8kv-d128-b16-bf16",
    5: "mix-48decode-L256..4096+16chunk512-P0..2048-32q8kv-d128-b16-bf16",
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    bits = t.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        bits[nan] = np.uint16(0x7FC0)
    return bits


def poison_bits(dtype: str):
    """Quiet-NaN bit pattern used to fill pool slots nobody wrote."""
    return np.uint16(0x7FC0) if dtype == BF16 else np.uint32(0x7FC00000)


def storage_dtype(dtype: str):
    return np.uint16 if dtype == BF16 else np.float32


@dataclasses.dataclass
class Workload:
    """One batch of sequences for a single decode (or chunk) step.

    Sequence ``s`` already holds ``hist_lens[s]`` cached tokens and appends
    ``new_lens[s]`` tokens in the step, so it attends over
    ``seq_lens[s] = hist_lens[s] + new_lens[s]`` keys. ``k_seq``/``v_seq`` hold
    every token of every sequence, packed: rows ``kv_offsets[s]`` to
    ``kv_offsets[s+1]`` are sequence ``s`` in position order, each row
    ``[n_kv, d]``. ``q`` holds one row ``[n_q, d]`` per new token, packed by
    ``q_offsets``. Raw storage: uint16 bf16 bits or float32.
    """

    name: str
    n_q: int
    n_kv: int
    head_dim: int
    block_size: int
    dtype: str
    scale: float
    hist_lens: np.ndarray
    new_lens: np.ndarray
    num_blocks: int
    table_stride: int
    alloc_order: np.ndarray
    kv_offsets: np.ndarray
    k_seq: np.ndarray
    v_seq: np.ndarray
    q_offsets: np.ndarray
    q: np.ndarray
    seed: int = 7

    @property
    def num_seqs(self) -> int:
        return int(len(self.hist_lens))

    @property
    def seq_lens(self) -> np.ndarray:
        return self.hist_lens + self.new_lens

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_new(self) -> int:
        return int(self.new_lens.max()) if self.num_seqs else 0

    def rows(self, s: int, lo: int, hi: int):
        """K and V rows of sequence ``s`` for positions ``lo..hi-1``."""
        a = int(self.kv_offsets[s])
        return self.k_seq[a + lo:a + hi], self.v_seq[a + lo:a + hi]

    def hist_rows(self, s: int):
        return self.rows(s, 0, int(self.hist_lens[s]))

    def new_rows(self, s: int):
        h = int(self.hist_lens[s])
        return self.rows(s, h, h + int(self.new_lens[s]))

    def packed_new_kv(self):
        """New-token K/V rows of all sequences packed in sequence order."""
        ks, vs = [], []
        for s in range(self.num_seqs):
            k, v = self.new_rows(s)
            ks.append(k)
            vs.append(v)
        shape = (0, self.n_kv, self.head_dim)
        sd = storage_dtype(self.dtype)
        return (np.concatenate(ks) if ks else np.zeros(shape, sd),
                np.concatenate(vs) if vs else np.zeros(shape, sd))

    def packed_hist_kv(self):
        ks, vs = [], []
        for s in range(self.num_seqs):
            k, v = self.hist_rows(s)
            ks.append(k)
            vs.append(v)
        shape = (0, self.n_kv, self.head_dim)
        sd = storage_dtype(self.dtype)
        return (np.concatenate(ks) if ks else np.zeros(shape, sd),
                np.concatenate(vs) if vs else np.zeros(shape, sd))

    def ideal_kv_bytes(self) -> int:
        """K+V bytes the step must read: every cached key of every kv head once."""
        b = 2 if self.dtype == BF16 else 4
        return int(self.seq_lens.sum()) * self.n_kv * self.head_dim * 2 * b


def _draw(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == BF16 else x


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def build_workload(*, n_q, n_kv, head_dim, block_size, dtype, hist_lens, new_lens,
                   num_blocks=None, table_stride=None, order="random", seed=7,
                   rng=None, name="custom", scale=None) -> Workload:
    """Draw K/V histories and queries for explicitly given lengths.

    ``num_blocks`` defaults to 1.25x the blocks the sequences need;
    ``table_stride`` to the longest sequence's block count. ``order`` is
    "random" (seeded permutation of block ids) or "identity".
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    hist = np.asarray(hist_lens, dtype=np.int64)
    new = np.asarray(new_lens, dtype=np.int64)
    assert hist.shape == new.shape and (hist >= 0).all() and (new >= 0).all()
    total = hist + new
    need = int(sum(-(-int(L) // block_size) for L in total))
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(1.25 * need)))
    if table_stride is None:
        table_stride = max(1, max((-(-int(L) // block_size) for L in total), default=1))
    if isinstance(order, str) and order == "random":
        alloc_order = rng.permutation(num_blocks).astype(np.int32)
    elif isinstance(order, str) and order == "identity":
        alloc_order = np.arange(num_blocks, dtype=np.int32)
    else:
        alloc_order = np.asarray(order, dtype=np.int32)
        assert sorted(alloc_order.tolist()) == list(range(num_blocks))
    kv_offsets = np.zeros(len(total) + 1, dtype=np.int64)
    np.cumsum(total, out=kv_offsets[1:])
    sd = storage_dtype(dtype)
    k_seq = np.empty((int(kv_offsets[-1]), n_kv, head_dim), dtype=sd)
    v_seq = np.empty_like(k_seq)
    def fill(s):
        a, b = int(kv_offsets[s]), int(kv_offsets[s + 1])
        srng = np.random.default_rng([seed, 1, s])
        k_seq[a:b] = _draw(srng, (b - a, n_kv, head_dim), dtype)
        v_seq[a:b] = _draw(srng, (b - a, n_kv, head_dim), dtype)

    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(total))))
    q_offsets = np.zeros(len(new) + 1, dtype=np.int64)
    np.cumsum(new, out=q_offsets[1:])
    q = _draw(np.random.default_rng([seed, 2]), (int(q_offsets[-1]), n_q, head_dim), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Workload(name=name, n_q=n_q, n_kv=n_kv, head_dim=head_dim, block_size=block_size,
                    dtype=dtype, scale=float(scale), hist_lens=hist, new_lens=new,
                    num_blocks=int(num_blocks), table_stride=int(table_stride),
                    alloc_order=alloc_order, kv_offsets=kv_offsets, k_seq=k_seq, v_seq=v_seq,
                    q_offsets=q_offsets, q=q, seed=seed)


def _uniform(rng, lo, hi, n):
    return rng.integers(lo, hi + 1, size=n).astype(np.int64)


def _loguniform(rng, lo, hi, n):
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    return np.clip(np.round(x), lo, hi).astype(np.int64)


def config_workload(cfg: int, seed: int = 7, batch_scale: float = 1.0) -> Workload:
    """The five workload shapes, drawn from ``seed``.

    ``batch_scale`` < 1 keeps every distribution but draws fewer sequences
    (used only to make CPU-side checks fast; timing uses 1.0).
    """
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[cfg]
    if cfg == 1:
        # Tiny lab scale: 2 MHA heads of width 4, blocks of 4 tokens, a 12-block
        # pool, three sequences with 9, 7 and 5 cached tokens plus one new token.
        return build_workload(n_q=2, n_kv=2, head_dim=4, block_size=4, dtype=F32,
                              hist_lens=[9, 7, 5], new_lens=[1, 1, 1], num_blocks=12,
                              table_stride=6, order="random", rng=rng, seed=seed, name=name)
    gqa = dict(n_q=32, n_kv=8, head_dim=128, block_size=16, dtype=BF16)

    def n(k):
        return max(1, int(round(k * batch_scale)))

    if cfg == 2:
        L = _uniform(rng, 512, 4096, n(64))
        return build_workload(**gqa, hist_lens=L - 1, new_lens=np.ones_like(L),
                              table_stride=4096 // 16, rng=rng, seed=seed, name=name)
    if cfg == 3:
        L = _loguniform(rng, 128, 8192, n(256))
        return build_workload(**gqa, hist_lens=L - 1, new_lens=np.ones_like(L),
                              table_stride=8192 // 16, rng=rng, seed=seed, name=name)
    if cfg == 4:
        L = np.full(n(8), 32768, dtype=np.int64)
        return build_workload(**gqa, hist_lens=L - 1, new_lens=np.ones_like(L),
                              table_stride=32768 // 16, rng=rng, seed=seed, name=name)
    if cfg == 5:
        Ld = _uniform(rng, 256, 4096, n(48))
        P = _uniform(rng, 0, 2048, n(16))
        hist = np.concatenate([Ld - 1, P])
        new = np.concatenate([np.ones_like(Ld), np.full_like(P, 512)])
        return build_workload(**gqa, hist_lens=hist, new_lens=new,
                              table_stride=4096 // 16, rng=rng, seed=seed, name=name)
    raise ValueError(f"unknown config {cfg}")
