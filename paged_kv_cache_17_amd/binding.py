"""ctypes binding of ``libpagedkv.so`` (argument marshalling only).

Each function has the name of the C entry point it calls and turns torch
tensors into the pointers, sizes and stream the C ABI takes. All work runs
in the library's HIP kernels; there is no Python or CPU fallback, and every
call raises if the library is missing or returns an error.

torch is imported before the library is opened so the process uses one HIP
runtime (the library's libamdhip64 dependency resolves to the one torch
already loaded).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

try:  # torch first: see module docstring
    import torch
except ImportError:  # pragma: no cover - the pool API works without torch
    torch = None

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_F32 = 0
PKV_BF16 = 1

_i32 = ctypes.c_int32
_p = ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)
_size_t = ctypes.c_size_t

_SIGNATURES = {
    "pkv_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "kvpool_create": ([_i32, _i32, _pi32, ctypes.POINTER(_p)], ctypes.c_int),
    "kvpool_destroy": ([_p], ctypes.c_int),
    "kvpool_alloc": ([_p, _i32, _pi32], ctypes.c_int),
    "kvpool_free": ([_p, _i32, _pi32], ctypes.c_int),
    "kvpool_num_free": ([_p, _pi32], ctypes.c_int),
    "kvpool_free_ids": ([_p, _pi32, _pi32], ctypes.c_int),
    "kvpool_ensure": ([_p, _pi32, _pi32, _i32, _i32], ctypes.c_int),
    "kvpool_release": ([_p, _pi32, _pi32], ctypes.c_int),
    "kvpool_truncate": ([_p, _pi32, _pi32, _i32], ctypes.c_int),
    "kvpool_share": ([_p, _i32, _pi32], ctypes.c_int),
    "kvpool_refcount": ([_p, _i32, _pi32], ctypes.c_int),
    "kvpool_fork": ([_p, _pi32, _i32, _pi32, _pi32, _i32, _i32], ctypes.c_int),
    "kvpool_cow": ([_p, _pi32, _i32, _i32, _i32, _pi32, _pi32, _i32, _pi32], ctypes.c_int),
    "kv_copy_blocks_q8": ([_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p], ctypes.c_int),
    "paged_attn_chunk_q8": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                             _i32, _i32, ctypes.c_float, _p, _size_t, _p], ctypes.c_int),
    "paged_attn_chunk_q8_append": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _p, _size_t, _p], ctypes.c_int),
    "kv_copy_blocks": ([_p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p], ctypes.c_int),
    "kv_append_q8": ([_p, _p, _p, _p, _p, _p, _i32, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p],
                     ctypes.c_int),
    "paged_attn_decode_q8": ([_p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                              ctypes.c_float, _p, _size_t, _p], ctypes.c_int),
    "kv_append": ([_p, _p, _p, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p],
                  ctypes.c_int),
    "paged_attn_split_tokens": ([_i32, _i32, _i32, _i32, _i32, _pi32], ctypes.c_int),
    "paged_attn_chunk_q8_workspace_size": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_size_t)],
                                           ctypes.c_int),
    "paged_attn_chunk_workspace_size": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                         ctypes.POINTER(_size_t)], ctypes.c_int),
    "paged_attn_workspace_size": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_size_t)],
                                  ctypes.c_int),
    "paged_attn_decode": ([_p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                           ctypes.c_float, _i32, _i32, _p, _size_t, _p], ctypes.c_int),
    "paged_attn_decode_append": ([_p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                  _i32, ctypes.c_float, _i32, _p, _size_t, _p], ctypes.c_int),
    "paged_attn_decode_append_noalloc": ([_p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32,
                                          _i32, _i32, ctypes.c_float, _i32, _p], ctypes.c_int),
    "paged_attn_decode_q8_append": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32,
                                     _i32, _i32, _i32, ctypes.c_float, _p, _size_t, _p], ctypes.c_int),
    "paged_attn_chunk_append": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32,
                                 _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _i32, _p, _size_t, _p],
                                ctypes.c_int),
    "paged_attn_chunk": ([_p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                          _i32, _i32, ctypes.c_float, _i32, _i32, _p, _size_t, _p], ctypes.c_int),
    "pkv_set_profile_events": ([_p, _p], ctypes.c_int),
    "pkv_stream_read": ([_p, _p, _size_t, _p, _i32, _i32, _i32, _p, _p], ctypes.c_int),
    "sample_workspace_size": ([_i32, _i32, ctypes.POINTER(_size_t)], ctypes.c_int),
    "sample_tokens": ([_p, _p, _p, _i32, _i32, ctypes.c_int64, _p, _p, _p, _p, _p, _size_t, _p], ctypes.c_int),
}

EXPORTED = tuple(_SIGNATURES)

_LIB = None


class PagedKVError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {message} (status {status})")
        self.status = status


def load_library():
    """Open the library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_17_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _LIB = lib
    return _LIB


def _check(fn: str, status: int):
    if status != 0:
        msg = load_library().pkv_strerror(status).decode()
        raise PagedKVError(fn, status, msg)


def strerror(status: int) -> str:
    return load_library().pkv_strerror(status).decode()


# --------------------------------------------------------------------------
# Block pool (host)
# --------------------------------------------------------------------------


def _i32_ptr(a: np.ndarray, offset: int = 0):
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return ctypes.cast(a.ctypes.data + 4 * offset, _pi32)


class KVPool:
    """Owner of one ``kvpool_t`` (block ids only; storage is the caller's)."""

    def __init__(self, num_blocks: int, block_size: int, alloc_order=None):
        lib = load_library()
        self._h = _p()
        order = None
        if alloc_order is not None:
            self._order = np.ascontiguousarray(alloc_order, dtype=np.int32)
            order = _i32_ptr(self._order)
        _check("kvpool_create", lib.kvpool_create(int(num_blocks), int(block_size), order,
                                                  ctypes.byref(self._h)))
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if self._h:
            load_library().kvpool_destroy(self._h)
            self._h = _p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def kvpool_alloc(self, n: int) -> np.ndarray:
        out = np.zeros(max(int(n), 1), dtype=np.int32)
        _check("kvpool_alloc", load_library().kvpool_alloc(self._h, int(n), _i32_ptr(out)))
        return out[:int(n)]

    def kvpool_free(self, ids) -> None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        _check("kvpool_free", load_library().kvpool_free(self._h, int(len(ids)), _i32_ptr(ids)))

    def kvpool_num_free(self) -> int:
        n = _i32()
        _check("kvpool_num_free", load_library().kvpool_num_free(self._h, ctypes.byref(n)))
        return n.value

    def kvpool_free_ids(self) -> np.ndarray:
        out = np.zeros(self.num_blocks, dtype=np.int32)
        n = _i32()
        _check("kvpool_free_ids", load_library().kvpool_free_ids(self._h, _i32_ptr(out), ctypes.byref(n)))
        return out[:n.value]

    def kvpool_ensure(self, table: np.ndarray, held: np.ndarray, s: int, length: int) -> None:
        """Grow row ``s`` of a host table ``[S, stride]`` (held counts in ``held[S]``)."""
        stride = table.shape[1]
        _check("kvpool_ensure", load_library().kvpool_ensure(
            self._h, _i32_ptr(table, s * stride), _i32_ptr(held, s), int(stride), int(length)))

    def kvpool_release(self, table: np.ndarray, held: np.ndarray, s: int) -> None:
        stride = table.shape[1]
        _check("kvpool_release", load_library().kvpool_release(
            self._h, _i32_ptr(table, s * stride), _i32_ptr(held, s)))

    def kvpool_truncate(self, table: np.ndarray, held: np.ndarray, s: int, length: int) -> None:
        """Roll row ``s`` back to ``length`` tokens (blocks past it are released)."""
        stride = table.shape[1]
        _check("kvpool_truncate", load_library().kvpool_truncate(
            self._h, _i32_ptr(table, s * stride), _i32_ptr(held, s), int(length)))

    def kvpool_share(self, ids) -> None:
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        _check("kvpool_share", load_library().kvpool_share(self._h, int(len(ids)), _i32_ptr(ids)))

    def kvpool_refcount(self, block: int) -> int:
        n = _i32()
        _check("kvpool_refcount", load_library().kvpool_refcount(self._h, int(block), ctypes.byref(n)))
        return n.value

    def kvpool_fork(self, table: np.ndarray, held: np.ndarray, src: int, dst: int, length: int) -> None:
        """Row ``dst`` (empty) shares the blocks of row ``src`` covering ``length`` tokens."""
        stride = table.shape[1]
        _check("kvpool_fork", load_library().kvpool_fork(
            self._h, _i32_ptr(table, src * stride), int(held[src]), _i32_ptr(table, dst * stride),
            _i32_ptr(held, dst), int(stride), int(length)))

    def kvpool_cow(self, table: np.ndarray, held: np.ndarray, s: int, start: int, count: int):
        """Unshare row ``s``'s blocks covering ``[start, start + count)``; returns the
        ``(src, dst)`` id arrays of the block copies the caller must make."""
        stride = table.shape[1]
        cap = -(-int(count) // self.block_size) + 1
        src = np.zeros(cap, dtype=np.int32)
        dst = np.zeros(cap, dtype=np.int32)
        n = _i32()
        _check("kvpool_cow", load_library().kvpool_cow(
            self._h, _i32_ptr(table, s * stride), int(held[s]), int(start), int(count), _i32_ptr(src),
            _i32_ptr(dst), int(cap), ctypes.byref(n)))
        return src[:n.value], dst[:n.value]


# --------------------------------------------------------------------------
# Device entry points
# --------------------------------------------------------------------------


def _ptr(t):
    return None if t is None else _p(t.data_ptr())


def _dtype_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return _p(stream.cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("device tensors required")
            if not t.is_contiguous():
                raise ValueError("contiguous tensors required")


def kv_append(k_cache, v_cache, k_new, v_new, block_table, start_pos, new_start, stream=None):
    """Append ``k_new``/``v_new`` ``[T, n_kv, d]`` into the pool through ``block_table``."""
    _dev(k_cache, v_cache, k_new, v_new, block_table, start_pos, new_start)
    num_blocks, n_kv, bs, d = k_cache.shape
    lib = load_library()
    _check("kv_append", lib.kv_append(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(block_table),
        int(block_table.shape[1]), _ptr(start_pos), _ptr(new_start), int(start_pos.shape[0]),
        int(k_new.shape[0]), int(num_blocks), int(n_kv), int(d), int(bs), _dtype_code(k_cache),
        _stream(stream)))


def kv_copy_blocks(k_cache, v_cache, src_ids, dst_ids, stream=None):
    """Copy whole blocks ``src_ids[i] -> dst_ids[i]`` (device int32) in both pools."""
    _dev(k_cache, v_cache, src_ids, dst_ids)
    num_blocks, n_kv, bs, d = k_cache.shape
    _check("kv_copy_blocks", load_library().kv_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(src_ids), _ptr(dst_ids), int(src_ids.shape[0]), int(num_blocks),
        int(n_kv), int(d), int(bs), _dtype_code(k_cache), _stream(stream)))


def kv_append_q8(k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_table, start_pos, new_start, stream=None):
    """Quantise ``k_new``/``v_new`` ``[T, n_kv, d]`` (bf16 or fp32) into the 8-bit pool."""
    _dev(k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_table, start_pos, new_start)
    num_blocks, n_kv, bs, d = k_codes.shape
    _check("kv_append_q8", load_library().kv_append_q8(
        _ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
        _ptr(block_table), int(block_table.shape[1]), _ptr(start_pos), _ptr(new_start), int(start_pos.shape[0]),
        int(k_new.shape[0]), int(num_blocks), int(n_kv), int(d), int(bs), _stream(stream)))


def paged_attn_decode_q8(out, lse, q, k_codes, v_codes, k_scale, v_scale, block_table, seq_lens, max_seq_len,
                         scale, workspace, stream=None):
    """Decode attention over the 8-bit pool: ``q``/``out`` bf16 ``[S, n_q, d]``."""
    _dev(out, lse, q, k_codes, v_codes, k_scale, v_scale, block_table, seq_lens, workspace)
    num_blocks, n_kv, bs, d = k_codes.shape
    S, n_q, _ = q.shape
    _check("paged_attn_decode_q8", load_library().paged_attn_decode_q8(
        _ptr(out), _ptr(lse), _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), int(S), int(max_seq_len), int(num_blocks),
        int(n_q), int(n_kv), int(d), int(bs), float(scale), _ptr(workspace),
        int(workspace.numel() * workspace.element_size()), _stream(stream)))


def paged_attn_split_tokens(num_q_rows, n_kv, block_size, max_seq_len, requested=0) -> int:
    out = _i32()
    _check("paged_attn_split_tokens", load_library().paged_attn_split_tokens(
        int(num_q_rows), int(n_kv), int(block_size), int(max_seq_len), int(requested), ctypes.byref(out)))
    return out.value


def paged_attn_chunk_workspace_size(num_seqs, total_q, max_q_len, n_q, n_kv, head_dim, block_size, max_seq_len,
                                    split_tokens=0) -> int:
    """Workspace bytes for paged_attn_chunk on any of its paths."""
    n = _size_t(0)
    _check("paged_attn_chunk_workspace_size", load_library().paged_attn_chunk_workspace_size(
        int(num_seqs), int(total_q), int(max_q_len), int(n_q), int(n_kv), int(head_dim), int(block_size),
        int(max_seq_len), int(split_tokens), ctypes.byref(n)))
    return int(n.value)


def paged_attn_chunk_q8_workspace_size(num_seqs, total_q, max_q_len, n_q, n_kv, head_dim, block_size,
                                       max_seq_len) -> int:
    """Workspace bytes for paged_attn_chunk_q8 on either of its paths."""
    n = _size_t(0)
    _check("paged_attn_chunk_q8_workspace_size", load_library().paged_attn_chunk_q8_workspace_size(
        int(num_seqs), int(total_q), int(max_q_len), int(n_q), int(n_kv), int(head_dim), int(block_size),
        int(max_seq_len), ctypes.byref(n)))
    return int(n.value)


def paged_attn_workspace_size(num_q_rows, n_q, n_kv, head_dim, block_size, max_seq_len, split_tokens=0) -> int:
    out = _size_t()
    _check("paged_attn_workspace_size", load_library().paged_attn_workspace_size(
        int(num_q_rows), int(n_q), int(n_kv), int(head_dim), int(block_size), int(max_seq_len),
        int(split_tokens), ctypes.byref(out)))
    return out.value


def paged_attn_decode(out, lse, q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale,
                      workspace, split_tokens=0, stream=None):
    """Decode attention: ``q``/``out`` ``[S, n_q, d]``, ``lse`` ``[S, n_q]`` float32 or None."""
    _dev(out, lse, q, k_cache, v_cache, block_table, seq_lens, workspace)
    num_blocks, n_kv, bs, d = k_cache.shape
    S, n_q, _ = q.shape
    _check("paged_attn_decode", load_library().paged_attn_decode(
        _ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        int(block_table.shape[1]), _ptr(seq_lens), int(S), int(max_seq_len), int(num_blocks),
        int(n_q), int(n_kv), int(d), int(bs), float(scale), _dtype_code(k_cache), int(split_tokens),
        _ptr(workspace), int(workspace.numel() * workspace.element_size()), _stream(stream)))


def paged_attn_decode_append(out, lse, q, k_cache, v_cache, k_new, v_new, block_table, seq_lens, max_seq_len,
                             scale, workspace, stream=None):
    """Decode step in one call: append ``k_new``/``v_new`` ``[S, n_kv, d]`` at position
    ``seq_lens - 1`` of each sequence, then decode attention as :func:`paged_attn_decode`."""
    _dev(out, lse, q, k_cache, v_cache, k_new, v_new, block_table, seq_lens, workspace)
    num_blocks, n_kv, bs, d = k_cache.shape
    S, n_q, _ = q.shape
    _check("paged_attn_decode_append", load_library().paged_attn_decode_append(
        _ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
        _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), int(S), int(max_seq_len),
        int(num_blocks), int(n_q), int(n_kv), int(d), int(bs), float(scale), _dtype_code(k_cache),
        _ptr(workspace), int(workspace.numel() * workspace.element_size()), _stream(stream)))


def paged_attn_decode_append_noalloc(out, lse, q, k_cache, v_cache, k_new, v_new, block_table, seq_lens,
                                     max_seq_len, scale, stream=None):
    """:func:`paged_attn_decode_append` with the split-K workspace in the library's
    static device array (no workspace argument; nothing is allocated)."""
    _dev(out, lse, q, k_cache, v_cache, k_new, v_new, block_table, seq_lens)
    num_blocks, n_kv, bs, d = k_cache.shape
    S, n_q, _ = q.shape
    _check("paged_attn_decode_append_noalloc", load_library().paged_attn_decode_append_noalloc(
        _ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
        _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), int(S), int(max_seq_len),
        int(num_blocks), int(n_q), int(n_kv), int(d), int(bs), float(scale), _dtype_code(k_cache),
        _stream(stream)))


def paged_attn_decode_q8_append(out, lse, q, k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_table,
                                seq_lens, max_seq_len, scale, workspace, stream=None):
    """Decode step in one call over an 8-bit pool: quantise and append ``k_new``/``v_new``
    ``[S, n_kv, d]`` (bf16) at ``seq_lens - 1``, then :func:`paged_attn_decode_q8`."""
    _dev(out, lse, q, k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_table, seq_lens, workspace)
    num_blocks, n_kv, bs, d = k_codes.shape
    S, n_q, _ = q.shape
    _check("paged_attn_decode_q8_append", load_library().paged_attn_decode_q8_append(
        _ptr(out), _ptr(lse), _ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale), _ptr(k_new),
        _ptr(v_new), _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), int(S), int(max_seq_len),
        int(num_blocks), int(n_q), int(n_kv), int(d), int(bs), float(scale), _ptr(workspace),
        int(workspace.numel() * workspace.element_size()), _stream(stream)))


def paged_attn_chunk(out, lse, q, q_start, k_cache, v_cache, block_table, seq_lens, max_q_len,
                     max_seq_len, scale, workspace, split_tokens=0, stream=None):
    """Chunk attention: ``q``/``out`` ``[sum C, n_q, d]`` packed by ``q_start``."""
    _dev(out, lse, q, q_start, k_cache, v_cache, block_table, seq_lens, workspace)
    num_blocks, n_kv, bs, d = k_cache.shape
    total_q, n_q, _ = q.shape
    _check("paged_attn_chunk", load_library().paged_attn_chunk(
        _ptr(out), _ptr(lse), _ptr(q), _ptr(q_start), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        int(block_table.shape[1]), _ptr(seq_lens), int(seq_lens.shape[0]), int(total_q), int(max_q_len),
        int(max_seq_len), int(num_blocks), int(n_q), int(n_kv), int(d), int(bs), float(scale),
        _dtype_code(k_cache), int(split_tokens),
        _ptr(workspace) if workspace is not None else None,
        int(workspace.numel() * workspace.element_size()) if workspace is not None else 0,
        _stream(stream)))


def paged_attn_chunk_append(out, lse, q, q_start, k_cache, v_cache, k_new, v_new, block_table, seq_lens,
                            max_q_len, max_seq_len, scale, workspace, split_tokens=0, stream=None):
    """Chunk step in one call: append ``k_new``/``v_new`` ``[sum C, n_kv, d]`` as the last C_s keys of
    each sequence, then chunk attention as :func:`paged_attn_chunk`."""
    _dev(out, lse, q, q_start, k_cache, v_cache, k_new, v_new, block_table, seq_lens, workspace)
    num_blocks, n_kv, bs, d = k_cache.shape
    total_q, n_q, _ = q.shape
    _check("paged_attn_chunk_append", load_library().paged_attn_chunk_append(
        _ptr(out), _ptr(lse), _ptr(q), _ptr(q_start), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
        _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), int(seq_lens.shape[0]), int(total_q),
        int(max_q_len), int(max_seq_len), int(num_blocks), int(n_q), int(n_kv), int(d), int(bs), float(scale),
        _dtype_code(k_cache), int(split_tokens),
        _ptr(workspace) if workspace is not None else None,
        int(workspace.numel() * workspace.element_size()) if workspace is not None else 0,
        _stream(stream)))


def sample_workspace_size(rows, vocab) -> int:
    """Bytes of device workspace sample_tokens needs for ``rows`` x ``vocab``."""
    n = _size_t(0)
    _check("sample_workspace_size", load_library().sample_workspace_size(int(rows), int(vocab), ctypes.byref(n)))
    return int(n.value)


def sample_tokens(logits, temperature, top_k, top_p, u, token=None, kept=None, workspace=None, stream=None):
    """Next token per row of ``logits`` ``[rows, vocab]`` (float32); per-row
    ``temperature``, ``top_k`` (int32), ``top_p``, ``u`` device tensors.
    ``workspace``: device uint8 tensor of at least sample_workspace_size
    bytes (allocated here when omitted). Returns the int32 token tensor (and
    fills ``kept`` [rows, 2] if given)."""
    rows, vocab = logits.shape
    if token is None:
        token = torch.empty(rows, dtype=torch.int32, device=logits.device)
    if workspace is None:
        workspace = torch.empty(max(1, sample_workspace_size(rows, vocab)), dtype=torch.uint8, device=logits.device)
    _dev(logits, temperature, top_k, top_p, u, token, kept, workspace)
    if logits.dtype != torch.float32 or top_k.dtype != torch.int32:
        raise TypeError("float32 logits and int32 top_k required")
    _check("sample_tokens", load_library().sample_tokens(
        _ptr(token), _ptr(kept), _ptr(logits), int(rows), int(vocab), int(logits.stride(0)), _ptr(temperature),
        _ptr(top_k), _ptr(top_p), _ptr(u), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
        _stream(stream)))
    return token


def pkv_set_profile_events(before, after):
    """Time the decode split kernel alone (torch.cuda.Event objects or None)."""
    b = _p(before.cuda_event) if before is not None else None
    a = _p(after.cuda_event) if after is not None else None
    _check("pkv_set_profile_events", load_library().pkv_set_profile_events(b, a))


def pkv_stream_read(a, b, order, workgroups, sink, tile_bytes=4096, stream=None):
    """Read-only streaming probe (measurement only): ``order`` None reads all of
    ``a`` contiguously; otherwise the tiles of ``tile_bytes`` (4096 or 2048) that
    ``order`` names in ``a`` and ``b``, in the decode pass's per-wave pattern.
    ``sink`` receives a checksum per lane."""
    _dev(a, sink)
    if order is not None:
        _dev(b, order)
    nbytes = a.numel() * a.element_size()
    _check("pkv_stream_read", load_library().pkv_stream_read(
        _ptr(a), _ptr(b) if b is not None else None, int(nbytes), _ptr(order) if order is not None else None,
        int(order.numel()) if order is not None else 0, int(tile_bytes), int(workgroups), _ptr(sink),
        _stream(stream)))


def kv_copy_blocks_q8(k_codes, v_codes, k_scale, v_scale, src_ids, dst_ids, stream=None):
    """Copy whole blocks of an 8-bit pool (codes and scales): ``src_ids[i]`` onto ``dst_ids[i]``."""
    _dev(k_codes, v_codes, k_scale, v_scale, src_ids, dst_ids)
    num_blocks, n_kv, bs, d = k_codes.shape
    _check("kv_copy_blocks_q8", load_library().kv_copy_blocks_q8(
        _ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale), _ptr(src_ids), _ptr(dst_ids),
        int(src_ids.numel()), int(num_blocks), int(n_kv), int(d), int(bs), _stream(stream)))


def paged_attn_chunk_q8(out, lse, q, q_start, k_codes, v_codes, k_scale, v_scale, block_table, seq_lens, max_q_len,
                        max_seq_len, scale, workspace, stream=None):
    """Chunk attention over an 8-bit pool: ``q``/``out`` bf16 ``[total_q, n_q, d]``; ``workspace``
    of paged_attn_chunk_q8_workspace_size bytes."""
    _dev(out, lse, q, q_start, k_codes, v_codes, k_scale, v_scale, block_table, seq_lens, workspace)
    num_blocks, n_kv, bs, d = k_codes.shape
    total_q, n_q, _ = q.shape
    _check("paged_attn_chunk_q8", load_library().paged_attn_chunk_q8(
        _ptr(out), _ptr(lse), _ptr(q), _ptr(q_start), _ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens), int(seq_lens.shape[0]), int(total_q),
        int(max_q_len), int(max_seq_len), int(num_blocks), int(n_q), int(n_kv), int(d), int(bs), float(scale),
        _ptr(workspace), int(workspace.numel() * workspace.element_size()), _stream(stream)))


def paged_attn_chunk_q8_append(out, lse, q, q_start, k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_table,
                               seq_lens, max_q_len, max_seq_len, scale, workspace, stream=None):
    """Chunk step over an 8-bit pool in one call: ``k_new``/``v_new`` bf16 ``[sum C, n_kv, d]``
    quantised into the pool as the last C_s keys of each sequence, then :func:`paged_attn_chunk_q8`."""
    _dev(out, lse, q, q_start, k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_table, seq_lens, workspace)
    num_blocks, n_kv, bs, d = k_codes.shape
    total_q, n_q, _ = q.shape
    _check("paged_attn_chunk_q8_append", load_library().paged_attn_chunk_q8_append(
        _ptr(out), _ptr(lse), _ptr(q), _ptr(q_start), _ptr(k_codes), _ptr(v_codes), _ptr(k_scale), _ptr(v_scale),
        _ptr(k_new), _ptr(v_new), _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens),
        int(seq_lens.shape[0]), int(total_q), int(max_q_len), int(max_seq_len), int(num_blocks), int(n_q),
        int(n_kv), int(d), int(bs), float(scale), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
        _stream(stream)))
