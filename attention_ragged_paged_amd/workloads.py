"""Seeded synthetic inputs for ragged paged attention.

This module only draws inputs: lengths, page permutations, block tables, block
masks and N(0, 1) values rounded once to bfloat16.  It holds none of the
method's arithmetic, and both the GPU path's tests and the CPU oracle consume
what it returns (as numpy arrays of bf16 bit patterns, ``uint16``).

Draw order for every batch, from ``numpy.random.default_rng(seed)``:
  1. lengths that are random (integer uniform, both ends inclusive);
  2. one permutation of the page pool, consumed in sequence order, then logical
     block order (per (sequence, KV head) in the KV-head-major layout);
  3. K cache values, then V cache values (every pool page is filled);
  4. q, then k_new, then v_new;
  5. the block mask, for the block-sparse workload.

FP8 caches (``kv_dtype="fp8"``) hold E4M3 codes (``uint8``) drawn directly, not
quantized from values, with the cache scales ``FP8_SCALE`` = 1/4: half of the codes
field by field (sign uniform, exponent field ~ round(N(9, 0.8)) clipped to [1, 10],
mantissa uniform: values of order one, below 4 in magnitude, like the N(0, 1) bf16
caches), half uniformly over every finite code (zero, subnormals, up to +-448, i.e.
values up to 112 in magnitude).  Poisoned slots of an FP8 cache hold the NaN code 0x7F.

Named workloads (shapes of Llama-3-8B attention: 32 query heads, 8 KV heads,
head dim 128) follow the five configurations the path is built for; see
``WORKLOADS``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SEQ_MAJOR = 0
HEAD_MAJOR = 1

BF16_NAN = 0x7FC0
FP8_NAN = 0x7F
FP8_SCALE = 1.0 / 4.0


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(
        np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 26) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16, generated in chunks to bound memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def _fp8_codes(rng: np.random.Generator, shape, chunk: int = 1 << 26) -> np.ndarray:
    """E4M3 codes (see the module docstring), in chunks: each code is, with probability 1/2,
    drawn field by field around values of order one, else uniformly over all 254 finite codes
    (zero, subnormals and +-448 included)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        m = e - s
        sign = rng.integers(0, 2, size=m, dtype=np.uint8)
        expo = np.clip(np.rint(rng.normal(9.0, 0.8, size=m)), 1, 10).astype(np.uint8)
        mant = rng.integers(0, 8, size=m, dtype=np.uint8)
        typical = (sign << 7) | (expo << 3) | mant
        anycode = rng.integers(0, 254, size=m, dtype=np.uint8)
        anycode = np.where(anycode >= 0x7F, anycode + 1, anycode).astype(np.uint8)  # skip 0x7F
        out[s:e] = np.where(rng.random(m) < 0.5, typical, anycode)
    return out.reshape(shape)


@dataclass
class RaggedBatch:
    name: str
    q: np.ndarray            # uint16 [T, Hq, D]
    k_new: np.ndarray        # uint16 [T, Hkv, D]
    v_new: np.ndarray        # uint16 [T, Hkv, D]
    k_cache: np.ndarray      # uint16 [P, S, Hkv, D] (seq-major) or [P, S, D] (head-major)
    v_cache: np.ndarray
    block_tables: np.ndarray  # int32 [B, max_pages] or [B, Hkv, max_pages]; -1 = unused
    cu_q_lens: np.ndarray    # int32 [B + 1]
    kv_lens: np.ndarray      # int32 [B] or [B, Hkv]; includes the new tokens
    scale: float
    page_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    layout: int
    seed: int
    extra: dict = field(default_factory=dict)
    k_scale: float = 1.0     # FP8 caches: cached K value = code value * k_scale
    v_scale: float = 1.0

    @property
    def kv_fp8(self) -> bool:
        return self.k_cache.dtype == np.uint8

    @property
    def num_seqs(self) -> int:
        return self.cu_q_lens.shape[0] - 1

    @property
    def total_q(self) -> int:
        return int(self.cu_q_lens[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_q_lens)

    @property
    def num_pages(self) -> int:
        return self.k_cache.shape[0]

    @property
    def max_pages(self) -> int:
        return self.block_tables.shape[-1]


def ragged_batch(name, q_lens, kv_lens, num_q_heads, num_kv_heads, head_dim, page_size,
                 pool_pages, seed, layout=SEQ_MAJOR, scale=None, max_pages=None, rng=None,
                 poison_unused=False, kv_dtype="bf16"):
    """A batch of sequences with the given new-token and total lengths.

    Pages come from one permutation of ``pool_pages`` physical pages.  With
    ``poison_unused`` every cache slot that no sequence owns (unused pages and
    the tail slots of each sequence's last page) holds NaN.  ``kv_dtype`` "fp8" gives
    caches of E4M3 codes with scales FP8_SCALE (drawn in place of the bf16 caches).  In the
    KV-head-major layout ``kv_lens`` may also be given per (sequence, KV head),
    shape [B, Hkv] (each head with its own past, as over compacted tables).
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    B = q_lens.shape[0]
    Hq, Hkv, D, S = num_q_heads, num_kv_heads, head_dim, page_size
    if kv_lens.ndim == 1:
        assert kv_lens.shape == (B,)
        kv_head = np.repeat(kv_lens[:, None], Hkv, axis=1)
    else:
        assert layout == HEAD_MAJOR and kv_lens.shape == (B, Hkv)
        kv_head = kv_lens
    assert np.all(kv_head >= q_lens[:, None])
    n_blocks_h = (kv_head + S - 1) // S            # [B, Hkv]
    n_blocks = n_blocks_h.max(axis=1)             # per sequence (its longest head)
    if max_pages is None:
        max_pages = int(max(1, n_blocks.max(initial=1)))
    need = int(n_blocks.sum()) if layout == SEQ_MAJOR else int(n_blocks_h.sum())
    assert need <= pool_pages, f"pool of {pool_pages} pages < {need} needed"
    perm = rng.permutation(pool_pages).astype(np.int32)
    if layout == SEQ_MAJOR:
        tables = np.full((B, max_pages), -1, dtype=np.int32)
    else:
        tables = np.full((B, Hkv, max_pages), -1, dtype=np.int32)
    cur = 0
    for b in range(B):
        nb = int(n_blocks[b])
        if layout == SEQ_MAJOR:
            tables[b, :nb] = perm[cur:cur + nb]
            cur += nb
        else:
            for g in range(Hkv):
                nbg = int(n_blocks_h[b, g])
                tables[b, g, :nbg] = perm[cur:cur + nbg]
                cur += nbg
    cache_shape = (pool_pages, S, Hkv, D) if layout == SEQ_MAJOR else (pool_pages, S, D)
    assert kv_dtype in ("bf16", "fp8")
    fp8 = kv_dtype == "fp8"
    draw_cache = _fp8_codes if fp8 else _normal_bf16
    k_cache = draw_cache(rng, cache_shape)
    v_cache = draw_cache(rng, cache_shape)
    T = int(q_lens.sum())
    q = _normal_bf16(rng, (T, Hq, D))
    k_new = _normal_bf16(rng, (T, Hkv, D))
    v_new = _normal_bf16(rng, (T, Hkv, D))
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    if layout == SEQ_MAJOR:
        kvl = kv_lens.astype(np.int32)
    else:
        kvl = np.ascontiguousarray(kv_head.astype(np.int32))
    if poison_unused:
        owned = np.zeros((pool_pages, S), dtype=bool)
        for b in range(B):
            rows = tables[b][None] if layout == SEQ_MAJOR else tables[b]
            for gi, row in enumerate(rows):
                L = int(kv_head[b, gi])
                for i in range((L + S - 1) // S):
                    n = min(S, L - i * S)
                    owned[row[i], :n] = True
        k_cache[~owned] = FP8_NAN if fp8 else BF16_NAN
        v_cache[~owned] = FP8_NAN if fp8 else BF16_NAN
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    cs = FP8_SCALE if fp8 else 1.0
    return RaggedBatch(name, q, k_new, v_new, k_cache, v_cache, tables, cu, kvl, float(scale),
                       S, Hq, Hkv, D, layout, seed, k_scale=cs, v_scale=cs)


# --------------------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------------------

def tiny_ragged(seed=1, **kw):
    """3 sequences, q_lens [1,1,7], kv_lens [17,40,23]; 4/2 heads, D 64; page 16; 16 pages."""
    return ragged_batch("tiny_ragged", [1, 1, 7], [17, 40, 23], 4, 2, 64, 16, 16, seed,
                        scale=1.0 / 8.0, **kw)


def llama3_decode(seed=2, num_seqs=64, lo=512, hi=4096, pool_pages=20000, **kw):
    """64 decode sequences (q_len 1), kv_len ~ U[512, 4096]; 32/8/128; page 16; 20k-page pool."""
    rng = np.random.default_rng(seed)
    kv = rng.integers(lo, hi + 1, size=num_seqs)
    return ragged_batch("llama3_decode", np.ones(num_seqs, np.int64), kv, 32, 8, 128, 16,
                        pool_pages, seed, rng=rng, **kw)


def llama3_decode_fp8(seed=2, **kw):
    """llama3_decode with E4M3 K/V caches (same lengths, pages and queries)."""
    b = llama3_decode(seed=seed, kv_dtype="fp8", **kw)
    b.name = "llama3_decode_fp8"
    return b


def llama3_prefill(seed=3, num_seqs=4, seq_len=2048, **kw):
    """4 sequences of 2048 new tokens, no prior context; 32/8/128; page 64."""
    S = 64
    pool = num_seqs * ((seq_len + S - 1) // S)
    return ragged_batch("llama3_prefill", [seq_len] * num_seqs, [seq_len] * num_seqs, 32, 8,
                        128, S, pool, seed, **kw)


def mixed_chunked(seed=4, chunk=512, context=8192, num_decode=96, lo=1024, hi=8192,
                  pool_pages=50000, **kw):
    """A 512-token chunk at context 8192 (kv 8704) first, then 96 decodes, kv ~ U[1024, 8192]."""
    rng = np.random.default_rng(seed)
    kv_dec = rng.integers(lo, hi + 1, size=num_decode)
    q_lens = np.concatenate([[chunk], np.ones(num_decode, np.int64)])
    kv_lens = np.concatenate([[context + chunk], kv_dec])
    return ragged_batch("mixed_chunked", q_lens, kv_lens, 32, 8, 128, 16, pool_pages, seed,
                        rng=rng, **kw)


def mixed_chunked_fp8(seed=4, **kw):
    """mixed_chunked with E4M3 K/V caches."""
    b = mixed_chunked(seed=seed, kv_dtype="fp8", **kw)
    b.name = "mixed_chunked_fp8"
    return b


def block_union_sparse(seed=5, context=131072, chunk=4096, density=0.1, column_shared=False,
                       num_q_heads=32, num_kv_heads=8, head_dim=128, **kw):
    """One sequence: a 4096-query chunk ending at context 131072 (past 126976), KV-head-major
    64-token pages, and a per-head block mask [Hq][chunk/64][context/64].

    Mask: for query block qb the diagonal block is past/64 + qb; blocks after it are 0; block 0
    and the diagonal are 1; every other block is Bernoulli(density), drawn per (head, qb, kb),
    or per (head, kb) shared by all query blocks when ``column_shared``.
    """
    S = 64
    rng = np.random.default_rng(seed)
    past = context - chunk
    n_kb = context // S
    pool = num_kv_heads * n_kb
    batch = ragged_batch("block_union_sparse" + ("_colshared" if column_shared else ""),
                         [chunk], [context], num_q_heads, num_kv_heads, head_dim, S, pool, seed,
                         layout=HEAD_MAJOR, rng=rng, **kw)
    n_qb = chunk // S
    if column_shared:
        cols = rng.random((num_q_heads, 1, n_kb)) < density
        mask = np.broadcast_to(cols, (num_q_heads, n_qb, n_kb)).copy()
    else:
        mask = rng.random((num_q_heads, n_qb, n_kb)) < density
    diag = past // S + np.arange(n_qb)
    kb = np.arange(n_kb)
    mask &= kb[None, None, :] <= diag[None, :, None]
    mask[:, :, 0] = True
    mask[:, np.arange(n_qb), diag] = True
    batch.extra.update(mask=mask.astype(np.uint8), past=past, context=context, chunk=chunk)
    return batch


def block_union_sparse_colshared(seed=5, **kw):
    """block_union_sparse with the column-shared mask: one Bernoulli(0.1) draw per (head, KV
    block) shared by all query blocks, so the union over Q-blocks stays sparse (about 34% of
    the blocks per KV head after the union over the 4 heads of a group)."""
    return block_union_sparse(seed=seed, column_shared=True, **kw)


WORKLOADS = {
    "tiny_ragged": tiny_ragged,
    "llama3_decode": llama3_decode,
    "llama3_prefill": llama3_prefill,
    "mixed_chunked": mixed_chunked,
    "block_union_sparse": block_union_sparse,
    "block_union_sparse_colshared": block_union_sparse_colshared,
    "llama3_decode_fp8": llama3_decode_fp8,
    "mixed_chunked_fp8": mixed_chunked_fp8,
}
