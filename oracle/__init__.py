"""CPU oracle for the paged-KV decode path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library. It is
plain float64 NumPy (plus a pure-Python brute force for tiny inputs) and
shares no code with the HIP path.
"""
from .paged_attention import (  # noqa: F401
    BlockAllocator,
    InvalidBlock,
    InvalidFree,
    copy_blocks,
    OracleCache,
    OutOfBlocks,
    QuantOracleCache,
    SequenceBlocks,
    QUANT_POISON_CODE,
    append,
    append_quantized,
    attention,
    attention_split_merge,
    bf16_bits_to_f64,
    block_alloc_slots,
    build_cache,
    build_quant_cache,
    build_tables,
    contiguous_attend,
    dequantize,
    gather,
    kv_bytes_per_token,
    paged_attention_all,
    quant_bytes,
    quantize_absmax,
    quantized_rows,
    token_slots,
    widen,
)
from . import sampling  # noqa: F401,E402
