"""Ragged paged attention for AMD Instinct MI355X (gfx950).

The compute lives in ``librpa.so`` (hand-written HIP kernels behind the C ABI declared in
``include/rpa.h``); this package only marshals PyTorch tensors into that ABI.  There is no
CPU fallback: every call fails loudly if the library or a gfx950 device is missing.

    write_kv(k_new, v_new, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, ...)
    attention(q, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, scale, ...)
    attention_noalloc(...)   # the same without a workspace (static device scratch)
    build_union_tables(mask, base_tables, past, kv_len, page_size)
    rotary_write_kv(q, k, v, k_cache, v_cache, ...)   # rotary + packed-QKV split + scatter
    GraphAttention(...)   # device-planned call that a HIP graph can capture

Caches are bf16, or FP8 E4M3 codes (uint8 / float8_e4m3fn storage) with per-cache scales
passed as k_scale / v_scale.
"""
from ._rpa import (  # noqa: F401
    GraphAttention,
    KERNEL_AUTO,
    KERNEL_DECODE,
    KERNEL_MIXED,
    KERNEL_PREFILL,
    KV_BF16,
    KV_FP8_E4M3,
    LAYOUT_HEAD_MAJOR,
    LAYOUT_SEQ_MAJOR,
    PreparedAttention,
    PreparedWriteKV,
    RpaError,
    NOALLOC_SCRATCH_BYTES,
    attention,
    attention_noalloc,
    build_union_tables,
    kv_dtype_of,
    library_path,
    load_library,
    rotary_write_kv,
    select_kernel,
    split_packed_qkv,
    workspace_size,
    write_kv,
)
