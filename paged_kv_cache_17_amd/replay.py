"""Fill a ``PagedKVCache`` from a seeded workload through the library's own
calls: tables grown by ``kvpool_ensure`` in sequence order, K/V written by
``kv_append`` (8-bit caches: ``kv_append_q8``), forks and copy-on-write
through ``kvpool_fork`` / ``kvpool_cow`` / ``kv_copy_blocks``, speculative
cycles through ``paged_attn_chunk`` and ``kvpool_truncate``.

A workload is any object with the attributes these functions read (the
sequence lengths, the allocation order, the packed K/V rows and queries as
raw storage: uint16 bf16 bits or float32). Only argument marshalling
happens here; every step runs in the library.
"""
from __future__ import annotations

import numpy as np

from . import binding as _B
from .cache import PagedKVCache

torch = _B.torch
BF16 = "bf16"


def torch_dtype(dtype):
    return torch.bfloat16 if dtype == BF16 else torch.float32


def raw_to_torch(raw, dtype, device="cuda"):
    raw = np.ascontiguousarray(raw)
    if dtype == BF16:
        return torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(raw.astype(np.float32, copy=False)).to(device)


def torch_to_raw(t, dtype):
    t = t.detach().cpu().contiguous()
    if dtype == BF16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def i32(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def build_gpu_cache(wl, fill_nan=True, alloc_order=None, quantized=False, with_new=True):
    """Replay history then step through the library: tables grown by
    ``kvpool_ensure`` in sequence order, K/V written by ``kv_append`` (or
    quantised by ``kv_append_q8`` into an 8-bit cache). With
    ``with_new=False`` the tables cover the step's new tokens but only the
    history is written (the state a decode step starts from)."""
    order = wl.alloc_order if alloc_order is None else alloc_order
    c = PagedKVCache(wl.num_blocks, wl.n_kv, wl.head_dim, wl.block_size,
                     torch.int8 if quantized else torch_dtype(wl.dtype),
                     wl.num_seqs, wl.table_stride, alloc_order=order, fill_nan=fill_nan,
                     poison_workspace=fill_nan)
    for s in range(wl.num_seqs):
        c.ensure(s, int(wl.hist_lens[s]))
    c.upload_table()
    kh, vh = wl.packed_hist_kv()
    if len(kh):
        hs = np.zeros(wl.num_seqs + 1, dtype=np.int64)
        np.cumsum(wl.hist_lens, out=hs[1:])
        c.append(raw_to_torch(kh, wl.dtype), raw_to_torch(vh, wl.dtype),
                 i32(np.zeros(wl.num_seqs)), i32(hs))
    for s in range(wl.num_seqs):
        c.ensure(s, int(wl.seq_lens[s]))
    c.upload_table()
    kn, vn = wl.packed_new_kv()
    if len(kn) and with_new:
        c.append(raw_to_torch(kn, wl.dtype), raw_to_torch(vn, wl.dtype), i32(wl.hist_lens), i32(wl.q_offsets))
    torch.cuda.synchronize()
    return c


def build_gpu_fork_cache(fw, fill_nan=True, share=True, quantized=False):
    """Forked sequences through the library: prompts written once (rows
    0..P-1), each forked into its branches (rows P..P+n*P-1), the prompt rows
    released, then for every branch copy-on-write of the shared tail block
    and its own tokens appended. Returns (cache, number of block copies).
    With share=False every branch row instead gets a private copy of its
    prompt (the no-sharing baseline). quantized: an 8-bit pool (codes and
    scales written by kv_append_q8, copied by kv_copy_blocks_q8)."""
    NP, NB = fw.num_prompts, fw.num_branches
    c = PagedKVCache(fw.num_blocks, fw.n_kv, fw.head_dim, fw.block_size,
                     torch.int8 if quantized else torch_dtype(fw.dtype), NP + NB, fw.table_stride,
                     alloc_order=fw.alloc_order, fill_nan=fill_nan, poison_workspace=fill_nan)
    if not share:
        lens = fw.branch_lens()
        for b in range(NB):
            c.ensure(NP + b, int(lens[b]))
        c.upload_table()
        counts = np.concatenate([np.zeros(NP, dtype=np.int64), lens])
        starts = np.zeros(NP + NB + 1, dtype=np.int64)
        np.cumsum(counts, out=starts[1:])
        ks = np.concatenate([np.concatenate([fw.prompt_k[fw.prompt_of(b)], fw.own_k[b]]) for b in range(NB)])
        vs = np.concatenate([np.concatenate([fw.prompt_v[fw.prompt_of(b)], fw.own_v[b]]) for b in range(NB)])
        c.append(raw_to_torch(ks, fw.dtype), raw_to_torch(vs, fw.dtype), i32(np.zeros(NP + NB)), i32(starts))
        torch.cuda.synchronize()
        return c, 0
    for p, P in enumerate(fw.prompt_lens):
        c.ensure(p, int(P))
    c.upload_table()
    counts = np.concatenate([fw.prompt_lens, np.zeros(NB, dtype=np.int64)])
    starts = np.zeros(NP + NB + 1, dtype=np.int64)
    np.cumsum(counts, out=starts[1:])
    c.append(raw_to_torch(np.concatenate(fw.prompt_k), fw.dtype), raw_to_torch(np.concatenate(fw.prompt_v), fw.dtype),
             i32(np.zeros(NP + NB)), i32(starts))
    for b in range(NB):
        c.fork(fw.prompt_of(b), NP + b, int(fw.prompt_lens[fw.prompt_of(b)]))
    for p in range(NP):
        c.release(p)
    copies = 0
    for b in range(NB):
        P, g = int(fw.prompt_lens[fw.prompt_of(b)]), int(fw.own_lens[b])
        copies += c.unshare_for_write(NP + b, P, g)
        c.ensure(NP + b, P + g)
    c.upload_table()
    counts = np.concatenate([np.zeros(NP, dtype=np.int64), fw.own_lens])
    starts = np.zeros(NP + NB + 1, dtype=np.int64)
    np.cumsum(counts, out=starts[1:])
    pos = np.concatenate([np.zeros(NP, dtype=np.int64), [fw.prompt_lens[fw.prompt_of(b)] for b in range(NB)]])
    c.append(raw_to_torch(np.concatenate(fw.own_k), fw.dtype), raw_to_torch(np.concatenate(fw.own_v), fw.dtype),
             i32(pos), i32(starts))
    torch.cuda.synchronize()
    return c, copies


class GpuSpec:
    """Speculative-decoding cycles through the library: history appended
    once, then per cycle gamma + 1 tokens appended (kv_append; an 8-bit pool:
    kv_append_q8), verified as one causal chunk (paged_attn_chunk /
    paged_attn_chunk_q8) and rolled back to the committed length
    (kvpool_truncate)."""

    def __init__(self, sw, fill_nan=True, quantized=False):
        self.sw = sw
        S = sw.num_seqs
        self.c = PagedKVCache(sw.num_blocks, sw.n_kv, sw.head_dim, sw.block_size,
                              torch.int8 if quantized else torch_dtype(sw.dtype), S, sw.table_stride,
                              alloc_order=sw.alloc_order, fill_nan=fill_nan, poison_workspace=fill_nan)
        self.lens = np.array(sw.hist_lens, dtype=np.int64)
        for s in range(S):
            self.c.ensure(s, int(self.lens[s]))
        self.c.upload_table()
        starts = np.zeros(S + 1, dtype=np.int64)
        np.cumsum(self.lens, out=starts[1:])
        self.c.append(raw_to_torch(np.concatenate(sw.hist_k), sw.dtype), raw_to_torch(np.concatenate(sw.hist_v), sw.dtype),
                      i32(np.zeros(S)), i32(starts))
        g1 = sw.gamma + 1
        self.q_start = i32(np.arange(S + 1) * g1)
        self.cyc = [(raw_to_torch(np.concatenate(sw.cyc_k[c]), sw.dtype), raw_to_torch(np.concatenate(sw.cyc_v[c]), sw.dtype),
                     raw_to_torch(sw.cyc_q[c], sw.dtype)) for c in range(sw.cycles)]
        torch.cuda.synchronize()

    def append_cycle(self, c, stream=None):
        sw = self.sw
        g1 = sw.gamma + 1
        for s in range(sw.num_seqs):
            self.c.ensure(s, int(self.lens[s]) + g1)
        self.c.upload_table()
        k, v, _ = self.cyc[c]
        self.c.append(k, v, i32(self.lens), self.q_start, stream=stream)

    def verify(self, c, split_tokens=0, stream=None):
        sw = self.sw
        g1 = sw.gamma + 1
        lens = self.lens + g1
        return self.c.chunk(self.cyc[c][2], self.q_start, i32(lens), g1, int(lens.max()), sw.scale,
                            split_tokens=split_tokens, stream=stream)

    def rollback(self, c):
        sw = self.sw
        for s in range(sw.num_seqs):
            keep = int(sw.accepted[c, s]) + 1
            self.c.truncate(s, int(self.lens[s]) + keep)
            self.lens[s] += keep
        self.c.upload_table()
