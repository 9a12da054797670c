"""A paged KV cache object built on the C ABI.

Holds the device K/V pools (torch tensors used as plain device memory), a
host block table with per-sequence block counts maintained by the
library's ``kvpool_*`` allocator, its device mirror, and a reusable
attention workspace. Every method only marshals arguments into
``libpagedkv.so`` calls.
"""
from __future__ import annotations

import numpy as np

from . import binding as B

torch = B.torch


class PagedKVCache:
    def __init__(self, num_blocks: int, n_kv: int, head_dim: int, block_size: int, dtype,
                 num_seqs: int, table_stride: int, alloc_order=None, device="cuda", fill_nan=False,
                 poison_workspace=False):
        self.num_blocks, self.n_kv, self.head_dim, self.block_size = num_blocks, n_kv, head_dim, block_size
        self.dtype = dtype
        self.device = device
        shape = (num_blocks, n_kv, block_size, head_dim)
        # dtype torch.int8: 8-bit codes plus one fp32 scale per (block, kv head,
        # slot) for K and for V (kv_append_q8 / paged_attn_decode_q8)
        self.quantized = dtype == torch.int8
        if self.quantized:
            # poison: code -128 (outside the code range) and NaN scales
            self.k_cache = torch.full(shape, -128, dtype=torch.int8, device=device)
            self.v_cache = torch.full(shape, -128, dtype=torch.int8, device=device)
            fill = float("nan") if fill_nan else 0.0
            self.k_scale = torch.full(shape[:3], fill, dtype=torch.float32, device=device)
            self.v_scale = torch.full(shape[:3], fill, dtype=torch.float32, device=device)
        elif fill_nan:
            self.k_cache = torch.full(shape, float("nan"), dtype=dtype, device=device)
            self.v_cache = torch.full(shape, float("nan"), dtype=dtype, device=device)
        else:
            self.k_cache = torch.empty(shape, dtype=dtype, device=device)
            self.v_cache = torch.empty(shape, dtype=dtype, device=device)
        self.pool = B.KVPool(num_blocks, block_size, alloc_order)
        self.table = np.full((num_seqs, table_stride), -1, dtype=np.int32)
        self.held = np.zeros(num_seqs, dtype=np.int32)
        self.table_dev = torch.from_numpy(self.table).to(device)
        self._ws = None
        # Debug aid: fill the workspace with 0xFF bytes (NaN floats) before
        # every call, so a partial slot the first pass failed to write shows
        # up as NaN output instead of reading stale memory.
        self.poison_workspace = poison_workspace

    # ---- host bookkeeping -------------------------------------------------
    def ensure(self, s: int, length: int) -> None:
        self.pool.kvpool_ensure(self.table, self.held, s, length)

    def release(self, s: int) -> None:
        self.pool.kvpool_release(self.table, self.held, s)

    def truncate(self, s: int, length: int) -> None:
        """Roll row ``s`` back to ``length`` tokens (rejected speculative drafts);
        call ``upload_table`` before the next device call that reads the table."""
        self.pool.kvpool_truncate(self.table, self.held, s, length)

    def fork(self, src: int, dst: int, length: int) -> None:
        """Row ``dst`` (empty) shares row ``src``'s blocks for its first ``length`` tokens."""
        self.pool.kvpool_fork(self.table, self.held, src, dst, length)

    def unshare_for_write(self, s: int, start: int, count: int, stream=None) -> int:
        """Copy-on-write before appending ``count`` tokens at ``start`` to row ``s``:
        shared blocks in that range are replaced by private copies (host table
        updated, contents copied on the device). Returns the number of copies;
        call ``upload_table`` before the next device call that reads the table."""
        src, dst = self.pool.kvpool_cow(self.table, self.held, s, start, count)
        if len(src):
            src_d, dst_d = torch.from_numpy(src).to(self.device), torch.from_numpy(dst).to(self.device)
            if self.quantized:
                B.kv_copy_blocks_q8(self.k_cache, self.v_cache, self.k_scale, self.v_scale, src_d, dst_d,
                                    stream=stream)
            else:
                B.kv_copy_blocks(self.k_cache, self.v_cache, src_d, dst_d, stream=stream)
        return len(src)

    def upload_table(self, stream=None) -> None:
        self.table_dev.copy_(torch.from_numpy(self.table), non_blocking=False)

    # ---- device calls -----------------------------------------------------
    def append(self, k_new, v_new, start_pos, new_start, stream=None) -> None:
        if self.quantized:
            B.kv_append_q8(self.k_cache, self.v_cache, self.k_scale, self.v_scale, k_new, v_new, self.table_dev,
                           start_pos, new_start, stream=stream)
            return
        B.kv_append(self.k_cache, self.v_cache, k_new, v_new, self.table_dev, start_pos, new_start,
                    stream=stream)

    def workspace(self, num_q_rows: int, n_q: int, max_seq_len: int, split_tokens: int = 0, chunk=None):
        if chunk is None:
            need = B.paged_attn_workspace_size(num_q_rows, n_q, self.n_kv, self.head_dim, self.block_size,
                                               max_seq_len, split_tokens)
        elif self.quantized:   # (num_seqs, max_q_len) of a chunk call over the 8-bit cache
            need = B.paged_attn_chunk_q8_workspace_size(chunk[0], num_q_rows, chunk[1], n_q, self.n_kv,
                                                        self.head_dim, self.block_size, max_seq_len)
        else:   # (num_seqs, max_q_len) of a chunk call
            need = B.paged_attn_chunk_workspace_size(chunk[0], num_q_rows, chunk[1], n_q, self.n_kv, self.head_dim,
                                                     self.block_size, max_seq_len, split_tokens)
        need = max(need, 256)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        if self.poison_workspace:
            self._ws.fill_(0xFF)
        return self._ws

    def decode(self, q, seq_lens, max_seq_len: int, scale: float, out=None, lse=None,
               split_tokens: int = 0, stream=None):
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace(q.shape[0], q.shape[1], max_seq_len, split_tokens)
        if self.quantized:
            if split_tokens:
                raise ValueError("the 8-bit decode uses the balanced partition only (split_tokens=0)")
            B.paged_attn_decode_q8(out, lse, q, self.k_cache, self.v_cache, self.k_scale, self.v_scale,
                                   self.table_dev, seq_lens, max_seq_len, scale, ws, stream=stream)
            return out
        B.paged_attn_decode(out, lse, q, self.k_cache, self.v_cache, self.table_dev, seq_lens,
                            max_seq_len, scale, ws, split_tokens=split_tokens, stream=stream)
        return out

    def decode_step(self, q, k_new, v_new, seq_lens, max_seq_len: int, scale: float, out=None, lse=None,
                    stream=None):
        """Append one token per sequence (``k_new``/``v_new`` ``[S, n_kv, d]`` bf16 at position
        ``seq_lens - 1``; quantised for an 8-bit cache) and attend, in one call (d 128, block 16)."""
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace(q.shape[0], q.shape[1], max_seq_len, 0)
        if self.quantized:
            B.paged_attn_decode_q8_append(out, lse, q, self.k_cache, self.v_cache, self.k_scale, self.v_scale,
                                          k_new, v_new, self.table_dev, seq_lens, max_seq_len, scale, ws,
                                          stream=stream)
            return out
        B.paged_attn_decode_append(out, lse, q, self.k_cache, self.v_cache, k_new, v_new, self.table_dev,
                                   seq_lens, max_seq_len, scale, ws, stream=stream)
        return out

    def chunk(self, q, q_start, seq_lens, max_q_len: int, max_seq_len: int, scale: float, out=None,
              lse=None, split_tokens: int = 0, stream=None):
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace(q.shape[0], q.shape[1], max_seq_len, split_tokens,
                            chunk=(q_start.shape[0] - 1, max_q_len))
        if self.quantized:
            if split_tokens:
                raise ValueError("chunks over an 8-bit cache use the balanced partition only (split_tokens=0)")
            B.paged_attn_chunk_q8(out, lse, q, q_start, self.k_cache, self.v_cache, self.k_scale, self.v_scale,
                                  self.table_dev, seq_lens, max_q_len, max_seq_len, scale, ws, stream=stream)
            return out
        B.paged_attn_chunk(out, lse, q, q_start, self.k_cache, self.v_cache, self.table_dev, seq_lens,
                           max_q_len, max_seq_len, scale, ws, split_tokens=split_tokens, stream=stream)
        return out

    def chunk_step(self, q, q_start, k_new, v_new, seq_lens, max_q_len: int, max_seq_len: int, scale: float,
                   out=None, lse=None, split_tokens: int = 0, stream=None):
        """Append each sequence's chunk (``k_new``/``v_new`` ``[sum C, n_kv, d]``, the last C_s of
        ``seq_lens``; bf16 and quantised for an 8-bit cache) and attend it, in one call
        (``paged_attn_chunk_append`` / ``paged_attn_chunk_q8_append``)."""
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace(q.shape[0], q.shape[1], max_seq_len, split_tokens,
                            chunk=(q_start.shape[0] - 1, max_q_len))
        if self.quantized:
            if split_tokens:
                raise ValueError("chunks over an 8-bit cache use the balanced partition only (split_tokens=0)")
            B.paged_attn_chunk_q8_append(out, lse, q, q_start, self.k_cache, self.v_cache, self.k_scale, self.v_scale,
                                         k_new, v_new, self.table_dev, seq_lens, max_q_len, max_seq_len, scale, ws,
                                         stream=stream)
            return out
        B.paged_attn_chunk_append(out, lse, q, q_start, self.k_cache, self.v_cache, k_new, v_new, self.table_dev,
                                  seq_lens, max_q_len, max_seq_len, scale, ws, split_tokens=split_tokens,
                                  stream=stream)
        return out
