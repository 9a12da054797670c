"""CPU oracle for paged-KV decode attention (float64, NumPy).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it. It shares no code, table or constant with the
HIP library and imports nothing from it.

What it states, in plain slow code, is what the pages define:

* the block pool and its allocator: fixed-size blocks handed out on demand,
  lowest-ranked free block first, returned on release with no double free
  (Inference Engineering lab page, class ``KVPool`` of its listing;
  LLM inference serving tutorial, sections 1.7 and 4.2);
* appending a token's K/V into slot ``pos % B`` of the block the sequence's
  table maps ``pos // B`` to (lab page, ``KVPool.write``);
* gathering a sequence's cache by concatenating its blocks and truncating to
  its length (lab page, ``KVPool.gather``);
* attention: scaled dot products, a causal mask allowing key ``j`` for a query
  at absolute position ``t`` iff ``j <= t``, max-subtracted softmax, weighted
  sum of V (lab page, function ``forward``; foundations-of-llms chapter 5,
  section 2.1), with query head ``h`` reading kv head
  ``h // (n_q / n_kv)`` (chapter 5, section 3.1, grouped-query attention);
* the split-and-merge form of the same softmax (chapter 5, section 4.1,
  online softmax), used only to pin that splitting is exact.

Parity status of each function is listed in its docstring.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# Raw storage -> float64
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64.

    A bf16 value is the top half of an IEEE binary32 value, so placing the 16
    bits in the high half of a 32-bit word gives the same number exactly.
    Pinned by known bit patterns (1.0, -2.0, inf, smallest subnormal).
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def widen(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Stored K/V/q values (uint16 bf16 bits or float32) as float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    return np.asarray(raw, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Block allocator
# --------------------------------------------------------------------------


class OracleError(Exception):
    pass


class OutOfBlocks(OracleError):
    pass


class InvalidFree(OracleError):
    pass


class BlockAllocator:
    """Free set of block ids handed out lowest rank first, with holder counts.

    The lab's pool keeps a sorted free list, pops index 0 when a sequence
    needs a block and re-sorts after a release, so it always hands out the
    smallest free id (lab page, ``KVPool.__init__``, ``write``, ``release``).
    Here "smallest" is by rank, where ``order[i]`` has rank ``i``; the
    identity order is exactly the lab's policy, a permutation scatters the
    tables while staying deterministic.

    The lab asserts on exhaustion; here ``alloc`` raises ``OutOfBlocks`` and
    changes nothing. The serving tutorial (section 1.7) requires reclaim to
    be free of double frees, so ``free`` validates every id (in range,
    currently allocated, no duplicates) before returning any of them.

    Shared blocks (serving tutorial, section 4.2: a common prefix or beam
    branches point at the same physical block, counted by reference;
    section 1.7: the block goes back only when its last holder lets go):
    ``alloc`` gives a block one holder, ``share`` adds one, ``free`` drops
    one and returns the block to the free set when none is left.
    Pinned against the tutorial's block-slot and sharing demos, the lab's
    7-of-12 peak and a brute-force model of the sorted list.
    """

    def __init__(self, num_blocks: int, order=None):
        self.num_blocks = int(num_blocks)
        if order is None:
            order = list(range(self.num_blocks))
        order = [int(x) for x in order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("order must be a permutation of 0..num_blocks-1")
        self.rank = {blk: i for i, blk in enumerate(order)}
        self.free_ranks = sorted(range(self.num_blocks))   # ranks of free ids
        self.order = order
        self.refs = {}                                      # allocated id -> holders

    @property
    def num_free(self) -> int:
        return len(self.free_ranks)

    def free_ids(self) -> list:
        """Free ids in the order they would be handed out."""
        return [self.order[r] for r in self.free_ranks]

    def refcount(self, blk: int) -> int:
        return self.refs.get(int(blk), 0)

    def alloc(self, n: int) -> list:
        if n < 0:
            raise ValueError("negative count")
        if n > len(self.free_ranks):
            raise OutOfBlocks(f"need {n} blocks, {len(self.free_ranks)} free")
        taken, self.free_ranks = self.free_ranks[:n], self.free_ranks[n:]
        ids = [self.order[r] for r in taken]
        for b in ids:
            self.refs[b] = 1
        return ids

    def _check_held(self, ids, exc):
        if len(set(ids)) != len(ids):
            raise exc("duplicate id in one call")
        for b in ids:
            if not (0 <= b < self.num_blocks):
                raise exc(f"id {b} out of range")
            if self.refs.get(b, 0) == 0:
                raise exc(f"id {b} is free")

    def free(self, ids) -> None:
        ids = [int(x) for x in ids]
        self._check_held(ids, InvalidFree)
        back = []
        for b in ids:
            self.refs[b] -= 1
            if self.refs[b] == 0:
                del self.refs[b]
                back.append(self.rank[b])
        self.free_ranks = sorted(self.free_ranks + back)

    def share(self, ids) -> None:
        ids = [int(x) for x in ids]
        self._check_held(ids, InvalidBlock)
        for b in ids:
            self.refs[b] += 1


class InvalidBlock(OracleError):
    pass


class SequenceBlocks:
    """One sequence's block table row (the lab's ``seq["blocks"]``).

    ``ensure(L)`` grows the row to ceil(L / B) blocks, taking one new block
    each time a position reaches ``len(blocks) * B``; taking them in one
    ``alloc`` call gives the same ids as the lab's one-at-a-time pops.
    ``release`` drops the row's hold on its blocks and empties it, so a
    second release is a no-op (serving tutorial, section 1.7: reclaim must
    be idempotent).

    ``fork`` and ``cow`` are the sharing side (serving tutorial, section
    4.2): a new row points at another row's first ceil(L / B) blocks; before
    a row writes positions in a block that other rows also hold, it swaps in
    a fresh block (lowest rank first, in row order) holding a copy, and the
    others keep the original.
    """

    def __init__(self, block_size: int):
        self.block_size = int(block_size)
        self.blocks = []

    def ensure(self, allocator: BlockAllocator, length: int) -> None:
        need = -(-int(length) // self.block_size)
        if need > len(self.blocks):
            self.blocks += allocator.alloc(need - len(self.blocks))

    def release(self, allocator: BlockAllocator) -> None:
        blocks, self.blocks = self.blocks, []
        allocator.free(blocks)

    def truncate(self, allocator: BlockAllocator, length: int) -> None:
        """Roll the row back to ``length`` tokens: keep ceil(length / B) blocks
        and let go of the rest (chapter 5 section 5: drafts after the first
        rejected one are discarded; serving tutorial, question on speculative
        decoding: their KV is rolled back, not committed)."""
        keep = -(-int(length) // self.block_size)
        if keep < len(self.blocks):
            tail, self.blocks = self.blocks[keep:], self.blocks[:keep]
            allocator.free(tail)

    def fork(self, allocator: BlockAllocator, src: "SequenceBlocks", length: int) -> None:
        if self.blocks:
            raise ValueError("fork into a non-empty row")
        need = -(-int(length) // self.block_size)
        if need > len(src.blocks):
            raise ValueError("fork past the source's blocks")
        allocator.share(src.blocks[:need])
        self.blocks = list(src.blocks[:need])

    def cow(self, allocator: BlockAllocator, start: int, count: int) -> list:
        """Make the blocks holding positions [start, start + count) private to
        this row; returns the (old, new) pairs whose contents must be copied."""
        if count <= 0 or not self.blocks:
            return []
        first = int(start) // self.block_size
        last = min((int(start) + int(count) - 1) // self.block_size, len(self.blocks) - 1)
        shared = [i for i in range(first, last + 1) if allocator.refcount(self.blocks[i]) > 1]
        if len(shared) > allocator.num_free:
            raise OutOfBlocks("no room for the copies")
        pairs = []
        for i in shared:
            old = self.blocks[i]
            new = allocator.alloc(1)[0]
            allocator.refs[old] -= 1
            self.blocks[i] = new
            pairs.append((old, new))
        return pairs


def copy_blocks(pool_k, pool_v, pairs) -> None:
    """Copy-on-write's data side: block ``new`` receives block ``old``'s K and V."""
    for old, new in pairs:
        pool_k[new] = pool_k[old]
        pool_v[new] = pool_v[old]


# --------------------------------------------------------------------------
# Byte and slot counts (pinned by the serving tutorial's demos D06/D07 and
# the lab's HBM budget block)
# --------------------------------------------------------------------------


def kv_bytes_per_token(n_layer: int, n_kv_head: int, d_head: int, bytes_per_elem: int) -> int:
    """Ideal K+V payload of one token: 2 (K and V) x layers x kv heads x width x bytes.

    Serving tutorial, section 4.1 (m_token); lab page, block 10.
    """
    return 2 * n_layer * n_kv_head * d_head * bytes_per_elem


def block_alloc_slots(lengths, block_size: int):
    """(logical slots, allocated slots) when each sequence holds ceil(L/B) blocks.

    Serving tutorial, section 4.2 and demo D07: the last block of each
    sequence is only partly filled (internal fragmentation).
    """
    logical = sum(int(L) for L in lengths)
    allocated = sum(-(-int(L) // block_size) * block_size for L in lengths)
    return logical, allocated


# --------------------------------------------------------------------------
# Append and gather (raw storage, bit-exact copies)
# --------------------------------------------------------------------------


def token_slots(blocks, positions, block_size: int):
    """(block id, slot) of each position through a table row: position ``p``
    lives in slot ``p % B`` of block ``blocks[p // B]`` (lab page, the
    ``KVPool`` class: the rule its write and gather both follow)."""
    positions = np.asarray(positions, dtype=np.int64)
    row = np.asarray(blocks, dtype=np.int64)
    return row[positions // block_size], positions % block_size


def append(pool_k, pool_v, blocks, start: int, k_new, v_new, block_size: int) -> None:
    """Write tokens ``start .. start+T-1`` into the pool through a table row.

    ``pool_*`` are ``[num_blocks, n_kv, B, d]`` raw arrays; ``k_new``/``v_new``
    are ``[T, n_kv, d]``. Every kv head of a token goes to the token's slot
    (``token_slots``). Nothing else in the pool changes.
    """
    blk, slot = token_slots(blocks, start + np.arange(len(k_new)), block_size)
    pool_k[blk, :, slot, :] = k_new
    pool_v[blk, :, slot, :] = v_new


def gather(pool, blocks, length: int, block_size: int) -> np.ndarray:
    """A sequence's cache as ``[n_kv, L, d]``: for each position 0..L-1 the
    row held in its slot (lab page, ``KVPool.gather``: the sequence's blocks
    read in table order, cut to its length)."""
    blk, slot = token_slots(blocks, np.arange(length), block_size)
    return pool[blk, :, slot, :].transpose(1, 0, 2)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------


def attention(q, K, V, scale: float, q_pos):
    """Causal scaled-dot-product attention with grouped kv heads, float64.

    ``q``: ``[T, n_q, d]``; ``K``, ``V``: ``[n_kv, L, d]``; ``q_pos[t]`` is the
    absolute position of query ``t``. Query head ``h`` uses kv head
    ``h // (n_q // n_kv)``. For each (t, h):
    ``s_j = scale * q.k_j`` for ``j <= q_pos[t]`` (others masked),
    ``p = exp(s - max s) / sum``, ``o = sum_j p_j v_j``,
    ``lse = max s + ln(sum exp(s - max s))``.
    Returns ``(out [T, n_q, d], lse [T, n_q], p [n_q, T, L])``.
    Lab page, ``forward`` (scores, causal mask, softmax, weighted sum);
    chapter 5, sections 2.1 and 3.1. Pinned by brute force, closed forms,
    a library SDPA and paged-vs-contiguous equality.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    T, n_q, d = q.shape
    n_kv, L, _ = K.shape
    if n_q % n_kv:
        raise ValueError("n_q must be a multiple of n_kv")
    group = n_q // n_kv
    # heads g*group .. g*group + group - 1 read kv head g: one product per kv head
    qg = q.reshape(T, n_kv, group, d).transpose(1, 2, 0, 3)          # [n_kv, group, T, d]
    scores = np.matmul(qg, K.transpose(0, 2, 1)[:, None]) * scale     # [n_kv, group, T, L]
    scores = scores.reshape(n_q, T, L)
    allow = np.arange(L)[None, :] <= np.asarray(q_pos)[:, None]       # [T, L]
    scores = np.where(allow[None], scores, -np.inf)
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    z = e.sum(axis=-1, keepdims=True)
    p = e / z
    out = np.matmul(p.reshape(n_kv, group, T, L), V[:, None])         # [n_kv, group, T, d]
    out = out.reshape(n_q, T, d).transpose(1, 0, 2)
    lse = (m[..., 0] + np.log(z[..., 0])).T             # [T, n_q]
    return out, lse, p


def attention_split_merge(q, K, V, scale: float, q_pos, bounds):
    """The same attention computed split by split and merged.

    ``bounds`` partitions ``[0, L)`` into key ranges. For range ``j`` the
    partial state is its own max ``m_j``, sum ``l_j = sum exp(s - m_j)`` and
    normalised output ``o_j`` (chapter 5, section 4.1: m, l and O of the
    first tile). States combine with weights ``w_j = l_j exp(m_j - M)``,
    ``M = max m_j``: ``o = sum w_j o_j / sum w_j``, ``lse = M + ln sum w_j``.
    A range with no allowed key has ``l_j = 0`` and weight 0.
    The page states the result is exact; that is the pin (equality with
    ``attention`` up to rounding).
    """
    q = np.asarray(q, dtype=np.float64)
    T, n_q, d = q.shape
    parts = []
    for lo, hi in bounds:
        if hi <= lo:
            continue
        Kj, Vj = np.asarray(K)[:, lo:hi], np.asarray(V)[:, lo:hi]
        group = n_q // K.shape[0]
        kv_of_head = np.arange(n_q) // group
        s = np.einsum("thd,hjd->htj", q, Kj[kv_of_head].astype(np.float64)) * scale
        allow = (np.arange(lo, hi)[None, :] <= np.asarray(q_pos)[:, None])
        s = np.where(allow[None], s, -np.inf)
        m = s.max(axis=-1)                                   # [n_q, T]
        has = np.isfinite(m)
        e = np.where(has[..., None], np.exp(s - np.where(has, m, 0.0)[..., None]), 0.0)
        l = e.sum(axis=-1)
        o = np.einsum("htj,hjd->htd", e, Vj[kv_of_head].astype(np.float64))
        o = np.where(has[..., None], o / np.where(has, l, 1.0)[..., None], 0.0)
        parts.append((m, l, o))
    M = np.max(np.stack([m for m, _, _ in parts]), axis=0)
    num = np.zeros((n_q, T, d))
    den = np.zeros((n_q, T))
    for m, l, o in parts:
        w = np.where(np.isfinite(m), l * np.exp(np.where(np.isfinite(m), m - M, 0.0)), 0.0)
        num += w[..., None] * o
        den += w
    out = (num / den[..., None]).transpose(1, 0, 2)
    lse = (M + np.log(den)).T
    return out, lse


# --------------------------------------------------------------------------
# Whole-step drivers
# --------------------------------------------------------------------------


class OracleCache:
    """The oracle's own pool, allocator and table rows for one workload.

    Built by replaying the step as a serving loop would: first every
    sequence's history (table grown, tokens appended, in sequence order),
    then the step itself (tables grown for the new tokens, new tokens
    appended, in sequence order). Unwritten slots keep the caller's fill
    value (NaN poison in the tests).
    """

    def __init__(self, wl, fill=None):
        self.wl = wl
        sd = np.uint16 if wl.dtype == "bf16" else np.float32
        shape = (wl.num_blocks, wl.n_kv, wl.block_size, wl.head_dim)
        if fill is None:
            fill = np.uint16(0x7FC0) if wl.dtype == "bf16" else np.float32(np.nan)
        if sd is np.float32:
            self.pool_k = np.full(shape, fill, dtype=np.float32)
        else:
            self.pool_k = np.full(shape, fill, dtype=np.uint16)
        self.pool_v = self.pool_k.copy()
        self.allocator = BlockAllocator(wl.num_blocks, wl.alloc_order)
        self.seqs = [SequenceBlocks(wl.block_size) for _ in range(wl.num_seqs)]

    def fill_history(self):
        wl = self.wl
        for s in range(wl.num_seqs):
            h = int(wl.hist_lens[s])
            self.seqs[s].ensure(self.allocator, h)
            k, v = wl.hist_rows(s)
            append(self.pool_k, self.pool_v, self.seqs[s].blocks, 0, k, v, wl.block_size)

    def append_step(self):
        wl = self.wl
        for s in range(wl.num_seqs):
            self.seqs[s].ensure(self.allocator, int(wl.seq_lens[s]))
            k, v = wl.new_rows(s)
            append(self.pool_k, self.pool_v, self.seqs[s].blocks, int(wl.hist_lens[s]), k, v,
                   wl.block_size)

    def tables(self) -> np.ndarray:
        wl = self.wl
        t = np.full((wl.num_seqs, wl.table_stride), -1, dtype=np.int32)
        for s, sb in enumerate(self.seqs):
            t[s, :len(sb.blocks)] = sb.blocks
        return t

    def sequence_kv(self, s: int):
        """Widened gathered cache of sequence ``s`` (``[n_kv, L, d]`` each)."""
        wl = self.wl
        L = int(wl.seq_lens[s])
        K = gather(self.pool_k, self.seqs[s].blocks, L, wl.block_size)
        V = gather(self.pool_v, self.seqs[s].blocks, L, wl.block_size)
        return widen(K, wl.dtype), widen(V, wl.dtype)

    def attend(self, s: int, heads=None):
        """Outputs for sequence ``s``'s new-token queries through the pool.

        Returns ``(out [C, n_q, d], lse [C, n_q])``; ``heads`` restricts the
        computation to a subset of query heads (others are NaN).
        """
        wl = self.wl
        K, V = self.sequence_kv(s)
        return _attend_rows(wl, s, K, V, heads)


def _attend_rows(wl, s, K, V, heads):
    L = int(wl.seq_lens[s])
    C = int(wl.new_lens[s])
    a, b = int(wl.q_offsets[s]), int(wl.q_offsets[s + 1])
    q = widen(wl.q[a:b], wl.dtype)
    pos = np.arange(L - C, L)
    if heads is None:
        out, lse, _ = attention(q, K, V, wl.scale, pos)
        return out, lse
    group = wl.n_q // wl.n_kv
    out = np.full((C, wl.n_q, wl.head_dim), np.nan)
    lse = np.full((C, wl.n_q), np.nan)
    for h in heads:
        g = h // group
        o, l, _ = attention(q[:, h:h + 1], K[g:g + 1], V[g:g + 1], wl.scale, pos)
        out[:, h] = o[:, 0]
        lse[:, h] = l[:, 0]
    return out, lse


def contiguous_attend(wl, s: int, heads=None):
    """Attention for sequence ``s`` straight from its contiguous history, with
    no pool or table: the "recompute" side of the lab's cache-vs-recompute
    check."""
    k, v = wl.rows(s, 0, int(wl.seq_lens[s]))
    K = widen(k, wl.dtype).transpose(1, 0, 2)
    V = widen(v, wl.dtype).transpose(1, 0, 2)
    return _attend_rows(wl, s, K, V, heads)


# --------------------------------------------------------------------------
# 8-bit cache (symmetric absmax quantisation, one scale per token and kv head)
# --------------------------------------------------------------------------

QUANT_POISON_CODE = np.int8(-128)   # outside the code range: marks unwritten slots


def quantize_absmax(x, q_max: int = 127, eps: float = 1e-8):
    """Symmetric absmax quantisation of each row (last axis) of ``x``.

    Chapter 5, section 4: scale ``s = max|x| / q_max`` (the exercise clamps
    ``max|x|`` below at 1e-8), code ``clamp(round(x / s), -q_max, q_max)``,
    value read back as ``s * code``; group-wise form with one scale per group
    of consecutive elements - here a row is one token's head_dim values for
    one kv head. The scale and the codes are computed in float32 (the
    exercise's precision), rounding ties to even, so the integer decision is
    the one a float32 implementation with correctly rounded division makes.
    Returns ``(codes int8 [..., g], scales float32 [...])``. Pinned by the
    half-step bound, exact grids, symmetry and the chapter's byte counts.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1, keepdims=True)
    s = np.maximum(amax, np.float32(eps)) / np.float32(q_max)
    codes = np.clip(np.rint(x / s), -q_max, q_max).astype(np.int8)
    return codes, s[..., 0]


def dequantize(codes, scales) -> np.ndarray:
    """``s * code`` in float64 (exact: an 8-bit code times a float32 scale)."""
    return np.asarray(codes).astype(np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def quant_bytes(n_elements: int, bits: int, groups: int, scale_bytes: int) -> int:
    """Storage of a quantised tensor: ``bits`` per element plus one scale per
    group (chapter 5, section 4: the exercise's memory column counts the
    codes and FP16 scales the same way)."""
    return n_elements * bits // 8 + groups * scale_bytes


def append_quantized(codes_k, codes_v, scale_k, scale_v, blocks, start: int, k_new, v_new, block_size: int,
                     dtype: str) -> None:
    """Quantise tokens ``start .. start+T-1`` (raw ``[T, n_kv, d]`` rows of
    ``dtype``) row by row with ``quantize_absmax`` and write codes and scales
    into their slots through a table row (the append rule of ``append``)."""
    ck, sk = quantize_absmax(widen(k_new, dtype))
    cv, sv = quantize_absmax(widen(v_new, dtype))
    blk, slot = token_slots(blocks, start + np.arange(len(k_new)), block_size)
    codes_k[blk, :, slot, :] = ck
    codes_v[blk, :, slot, :] = cv
    scale_k[blk, :, slot] = sk
    scale_v[blk, :, slot] = sv


def quantized_rows(rows, dtype: str) -> np.ndarray:
    """Raw ``[..., d]`` rows as the 8-bit cache reads them back: ``s * code``
    of their absmax quantisation, float64."""
    codes, scales = quantize_absmax(widen(rows, dtype))
    return dequantize(codes, scales)


class QuantOracleCache(OracleCache):
    """The oracle's 8-bit pool: codes ``[num_blocks, n_kv, B, d]`` and one
    float32 scale per (block, kv head, slot), for K and for V. Tokens are
    quantised row by row (``quantize_absmax``) as they are appended, through
    the same allocator and table replay as ``OracleCache``; attention reads
    ``s * code``. Unwritten codes hold -128 and unwritten scales NaN."""

    def __init__(self, wl):
        self.wl = wl
        shape = (wl.num_blocks, wl.n_kv, wl.block_size, wl.head_dim)
        self.pool_k = np.full(shape, QUANT_POISON_CODE, dtype=np.int8)
        self.pool_v = self.pool_k.copy()
        self.scale_k = np.full(shape[:3], np.nan, dtype=np.float32)
        self.scale_v = self.scale_k.copy()
        self.allocator = BlockAllocator(wl.num_blocks, wl.alloc_order)
        self.seqs = [SequenceBlocks(wl.block_size) for _ in range(wl.num_seqs)]

    def _append(self, s, start, k, v):
        append_quantized(self.pool_k, self.pool_v, self.scale_k, self.scale_v, self.seqs[s].blocks, start, k, v,
                         self.wl.block_size, self.wl.dtype)

    def fill_history(self):
        wl = self.wl
        for s in range(wl.num_seqs):
            self.seqs[s].ensure(self.allocator, int(wl.hist_lens[s]))
            k, v = wl.hist_rows(s)
            self._append(s, 0, k, v)

    def append_step(self):
        wl = self.wl
        for s in range(wl.num_seqs):
            self.seqs[s].ensure(self.allocator, int(wl.seq_lens[s]))
            k, v = wl.new_rows(s)
            self._append(s, int(wl.hist_lens[s]), k, v)

    def sequence_kv(self, s: int):
        wl = self.wl
        L = int(wl.seq_lens[s])
        B = wl.block_size
        blocks = self.seqs[s].blocks
        K = gather(self.pool_k, blocks, L, B)
        V = gather(self.pool_v, blocks, L, B)
        blk, slot = token_slots(blocks, np.arange(L), B)
        sk = self.scale_k[blk, :, slot].T
        sv = self.scale_v[blk, :, slot].T
        return dequantize(K, sk), dequantize(V, sv)


def build_quant_cache(wl) -> QuantOracleCache:
    c = QuantOracleCache(wl)
    c.fill_history()
    c.append_step()
    return c


def build_tables(wl) -> np.ndarray:
    """Only the allocation side of ``build_cache``: the table rows the
    history-then-step replay produces (no K/V storage)."""
    alloc = BlockAllocator(wl.num_blocks, wl.alloc_order)
    seqs = [SequenceBlocks(wl.block_size) for _ in range(wl.num_seqs)]
    for s in range(wl.num_seqs):
        seqs[s].ensure(alloc, int(wl.hist_lens[s]))
    for s in range(wl.num_seqs):
        seqs[s].ensure(alloc, int(wl.seq_lens[s]))
    t = np.full((wl.num_seqs, wl.table_stride), -1, dtype=np.int32)
    for s, sb in enumerate(seqs):
        t[s, :len(sb.blocks)] = sb.blocks
    return t


def build_cache(wl, fill=None) -> OracleCache:
    c = OracleCache(wl, fill)
    c.fill_history()
    c.append_step()
    return c


def paged_attention_all(cache: OracleCache):
    """Every sequence's outputs, packed like the queries: ``[sum C, n_q, d]``."""
    wl = cache.wl
    outs, lses = [], []
    for s in range(wl.num_seqs):
        o, l = cache.attend(s)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)
