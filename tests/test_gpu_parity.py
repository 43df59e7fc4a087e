"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Cache writes and union tables must match bit for bit; attention outputs within max-abs 2e-2
(bf16 inputs, fp32 accumulation, bf16 output).  Small cases compare every output element;
the full-size workloads compare sampled rows that the oracle computes one by one.
"""
import itertools

import numpy as np
import pytest
import torch

import attention_ragged_paged_amd as rpa
import oracle
from attention_ragged_paged_amd import workloads as wl
from tests.gpu_util import (Dev, bf16_dev, compare, i32_dev, oracle_after_write, sample_rows, say,
                            to_host_bits, to_host_f32)

pytestmark = pytest.mark.gpu

KERNELS = [rpa.KERNEL_AUTO, rpa.KERNEL_DECODE, rpa.KERNEL_PREFILL, rpa.KERNEL_MIXED]


def _full_check(b, kernel=rpa.KERNEL_AUTO, fused=True, label="", typical=None):
    d = Dev(b)
    if not fused:
        d.write()
    out = d.attention(fused_write=fused, kernel=kernel)
    kc, vc = oracle_after_write(b)
    assert np.array_equal(to_host_bits(d.k_cache), kc), f"{label}: K cache differs"
    assert np.array_equal(to_host_bits(d.v_cache), vc), f"{label}: V cache differs"
    ref = oracle.attention(b.q, kc, vc, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale,
                           b.page_size, b.num_kv_heads, layout=b.layout)
    return compare(to_host_f32(out), ref, label, typical=typical)


# ------------------------------------------------------------------------------ write ----

@pytest.mark.parametrize("layout", [wl.SEQ_MAJOR, wl.HEAD_MAJOR])
@pytest.mark.parametrize("D", [64, 128])
def test_write_kv_bit_exact(layout, D):
    say(f"write_kv layout={layout} D={D}")
    b = wl.ragged_batch("w", [1, 7, 0, 33, 16], [17, 23, 5, 100, 16], 8, 2, D, 16, 40, 21,
                        layout=layout)
    d = Dev(b)
    d.write()
    kc, vc = oracle_after_write(b)
    assert np.array_equal(to_host_bits(d.k_cache), kc)
    assert np.array_equal(to_host_bits(d.v_cache), vc)


# ------------------------------------------------------------------- tiny ragged batch ---

@pytest.mark.parametrize("kernel", KERNELS)
def test_tiny_ragged_every_kernel(kernel):
    say(f"tiny_ragged kernel={kernel}")
    _full_check(wl.tiny_ragged(), kernel=kernel, label=f"tiny kernel={kernel}")


def test_tiny_ragged_separate_write():
    say("tiny_ragged separate write")
    _full_check(wl.tiny_ragged(), fused=False, label="tiny write-then-attend")


def _matrix():
    cases = []
    q_sets = [[1], [4], [16], [32], [48], [1, 4], [0, 16, 1], [32, 1, 0, 3], [48, 16, 1, 4]]
    heads = [(4, 4), (8, 2), (14, 2), (32, 8)]
    pages = [16, 32, 64, 128, 256]
    rng = np.random.default_rng(99)
    for i, (qs, (Hq, Hkv), S, D) in enumerate(itertools.product(q_sets, heads, pages, [64, 128])):
        if rng.random() > 0.12:
            continue
        past = [int(rng.integers(0, 300)) for _ in qs]
        cases.append((qs, past, Hq, Hkv, S, D, i))
    return cases


@pytest.mark.parametrize("qs,past,Hq,Hkv,S,D,i", _matrix())
def test_ragged_matrix(qs, past, Hq, Hkv, S, D, i):
    kv = [q + p for q, p in zip(qs, past)]
    pool = sum((k + S - 1) // S for k in kv) + 3
    scale = 0.05 + 0.01 * (i % 7)   # explicit non-default scales
    b = wl.ragged_batch("m", qs, kv, Hq, Hkv, D, S, pool, 1000 + i, scale=scale)
    for kernel in KERNELS:
        say(f"matrix case {i}: q={qs} past={past} heads={Hq}/{Hkv} S={S} D={D} kernel={kernel}")
        _full_check(b, kernel=kernel, label=f"case {i} kernel {kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_nan_in_unowned_slots_does_not_leak(kernel):
    """Unused pages and the tail slots past each sequence's kv_len hold NaN."""
    say(f"nan poison kernel={kernel}")
    b = wl.ragged_batch("nan", [1, 5, 40, 1], [33, 21, 75, 250], 8, 2, 128, 16, 40, 31,
                        poison_unused=True)
    _full_check(b, kernel=kernel, label=f"nan kernel={kernel}")


def test_mixed_order_does_not_matter():
    """Reordering the sequences of a mixed batch permutes per-sequence results only."""
    say("mixed order")
    b = wl.ragged_batch("ord", [200, 1, 1, 3], [700, 90, 300, 40], 32, 8, 128, 16, 120, 41)
    _full_check(b, label="mixed order A")
    perm = [2, 0, 3, 1]
    qs = np.diff(b.cu_q_lens)
    b2 = wl.ragged_batch("ord2", qs[perm], b.kv_lens[perm], 32, 8, 128, 16, 120, 41)
    _full_check(b2, label="mixed order B")


def test_long_decode_sequence_many_chunks():
    """One decode sequence long enough that a wave walks more than 64 chunks of its split."""
    say("long decode 300k")
    b = wl.ragged_batch("long", [1, 2], [300000, 5000], 4, 1, 128, 16, 19100, 51)
    d = Dev(b)
    out = d.attention()
    kc, vc = oracle_after_write(b)
    rows = np.array([[0, 0], [0, 3], [1, 1], [2, 2]], np.int32)
    ref = oracle.attention(b.q, kc, vc, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale, 16, 1,
                           rows=rows)
    got = to_host_f32(out)[rows[:, 0], rows[:, 1]]
    compare(got, ref, "long decode", typical=(1e-3, 1e-4))


# --------------------------------------------------------------- full-size workloads ----

def _sampled(b, n_rows, label, kernel=rpa.KERNEL_AUTO, check_cache=True, typical=None):
    d = Dev(b)
    out = d.attention(kernel=kernel)
    kc, vc = oracle_after_write(b)
    if check_cache:
        assert np.array_equal(to_host_bits(d.k_cache), kc), f"{label}: K cache differs"
        assert np.array_equal(to_host_bits(d.v_cache), vc), f"{label}: V cache differs"
    rows = sample_rows(b, n_rows)
    ref = oracle.attention(b.q, kc, vc, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale,
                           b.page_size, b.num_kv_heads, layout=b.layout, rows=rows)
    got = to_host_f32(out)[rows[:, 0], rows[:, 1]]
    return compare(got, ref, label, typical=typical)


def test_llama3_decode_full_size():
    say("llama3_decode full size (64 seqs, kv U[512,4096], 20k-page pool)")
    _sampled(wl.llama3_decode(), 512, "llama3 decode", typical=(3e-3, 3e-4))


def test_llama3_prefill_full_size():
    say("llama3_prefill full size (4 x 2048, page 64)")
    _sampled(wl.llama3_prefill(), 256, "llama3 prefill", typical=(1e-2, 5e-4))


def test_mixed_chunked_full_size():
    say("mixed_chunked full size (512 @ 8192 + 96 decodes, page 16)")
    b = wl.mixed_chunked()
    d = Dev(b)
    assert rpa.select_kernel(d.q, d.k_cache, d.tables, d.cu_h, d.kvl_h) == rpa.KERNEL_MIXED
    del d
    _sampled(b, 400, "mixed chunked", typical=(2e-3, 2e-4))


# ------------------------------------------------------------------ union tables -------

@pytest.mark.parametrize("seed,Hq,Hkv,nQB,nKB,S,past,kv_len,dens", [
    (0, 8, 2, 4, 24, 16, 320, 370, 0.2),
    (1, 4, 4, 3, 100, 32, 1000, 1070, 0.05),   # G = 1, unaligned block count
    (2, 32, 8, 64, 2048, 64, 126976, 131072, 0.1),
    (3, 28, 4, 5, 4096, 16, 65000, 65536, 0.0),
])
def test_union_tables_bit_exact(seed, Hq, Hkv, nQB, nKB, S, past, kv_len, dens):
    say(f"union tables seed={seed}")
    rng = np.random.default_rng(seed)
    mask = (rng.random((Hq, nQB, nKB)) < dens).astype(np.uint8)
    base = rng.permutation(Hkv * nKB).astype(np.int32).reshape(Hkv, nKB)
    t, c, k = rpa.build_union_tables(torch.from_numpy(mask).cuda(), i32_dev(base), past, kv_len, S)
    torch.cuda.synchronize()
    et, ec, ek, _ = oracle.union_tables(mask, base, past, kv_len, S)
    assert np.array_equal(t.cpu().numpy(), et)
    assert np.array_equal(c.cpu().numpy(), ec)
    assert np.array_equal(k.cpu().numpy(), ek)


@pytest.mark.parametrize("column_shared,fused", [(False, False), (True, True)])
def test_block_union_sparse_full_size(column_shared, fused):
    """Union tables built on the GPU, then causal attention over the selected KV-head-major
    pages; the chunk's K/V are written either by the separate scatter through the base tables
    or inside the attention launch through the compacted tables (whose last blocks are the
    chunk's own pages).  Caches bit-exact, sampled rows against the oracle's position-wise
    sparse attention."""
    say(f"block_union_sparse full size column_shared={column_shared} fused={fused}")
    b = wl.block_union_sparse(column_shared=column_shared)
    past, ctx = b.extra["past"], b.extra["context"]
    d = Dev(b)
    mask_d = torch.from_numpy(b.extra["mask"]).cuda()
    t, c, kvl = rpa.build_union_tables(mask_d, d.tables[0], past, ctx, b.page_size)
    torch.cuda.synchronize()
    et, ec, ek, sel = oracle.union_tables(b.extra["mask"], b.block_tables[0], past, ctx,
                                          b.page_size)
    assert np.array_equal(t.cpu().numpy(), et) and np.array_equal(kvl.cpu().numpy(), ek)
    say(f"  union density per KV head: {np.round(ec / (ctx // b.page_size), 3).tolist()}")
    if not fused:
        d.write()
    out = d.attention(fused_write=fused, tables=t[None].contiguous(),
                      kv_lens=kvl[None].contiguous(),
                      kv_lens_host=torch.from_numpy(ek[None].copy()))
    kc, vc = oracle_after_write(b)
    assert np.array_equal(to_host_bits(d.k_cache), kc), "K cache differs"
    assert np.array_equal(to_host_bits(d.v_cache), vc), "V cache differs"
    rows = sample_rows(b, 96)
    ref = oracle.attention(b.q, kc, vc, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale,
                           b.page_size, b.num_kv_heads, layout=wl.HEAD_MAJOR,
                           block_allowed=sel[None], rows=rows)
    got = to_host_f32(out)[rows[:, 0], rows[:, 1]]
    compare(got, ref, f"sparse column_shared={column_shared} fused={fused}", typical=(5e-4, 6e-5))


# --------------------------------------------------------------- layouts and extremes ----

@pytest.mark.parametrize("kernel", KERNELS)
def test_head_major_per_head_lengths(kernel):
    """KV-head-major pages with a different kv_len (and so a different past) per KV head,
    as over compacted tables: decode-class and prefill-class sequences, fused write."""
    say(f"head-major per-head lengths kernel={kernel}")
    qs = [1, 40, 3]
    kv = np.array([[70, 33], [40, 95], [3, 130]])
    pool = int(((kv + 15) // 16).sum()) + 4
    b = wl.ragged_batch("hm", qs, kv, 8, 2, 128, 16, pool, 77, layout=wl.HEAD_MAJOR)
    _full_check(b, kernel=kernel, label=f"head-major kernel={kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_group_of_64_heads(kernel):
    """G = 64 query heads per KV head: every sequence is prefill-class (2 tokens per 128-row
    tile); forcing the decode kernel still gives the same result."""
    say(f"G=64 kernel={kernel}")
    b = wl.ragged_batch("g64", [1, 3, 20], [101, 503, 57], 64, 1, 64, 32, 30, 78)
    _full_check(b, kernel=kernel, label=f"G=64 kernel={kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_page_size_1024(kernel):
    say(f"page 1024 kernel={kernel}")
    b = wl.ragged_batch("p1024", [1, 30], [3001, 2030], 8, 2, 128, 1024, 8, 79)
    _full_check(b, kernel=kernel, label=f"page 1024 kernel={kernel}")


def test_long_context_prefill_splits():
    """Prefill-only batch whose long contexts are cut into many KV splits (merged in-kernel)."""
    say("long-context prefill splits")
    b = wl.ragged_batch("lcp", [200, 64], [30200, 5064], 32, 8, 128, 16, 2300, 80)
    d = Dev(b)
    assert rpa.select_kernel(d.q, d.k_cache, d.tables, d.cu_h, d.kvl_h) == rpa.KERNEL_PREFILL
    del d
    _sampled(b, 160, "long-context prefill", typical=(1.5e-3, 1.2e-4))


@pytest.mark.parametrize("Hq,Hkv,D", [(24, 8, 64), (16, 2, 64), (8, 8, 128), (12, 4, 128)])
def test_prefill_split_rows_every_group_size(Hq, Hkv, D):
    """A lone chunk at a long context, prefill-only, so its few items are cut into KV splits
    whose partials are written and merged as whole rows: group sizes 1, 3 and 8 (rows of a
    128-row item that fall past the group or the chunk stay unwritten), both head dims, every
    output element against the oracle."""
    say(f"prefill split rows Hq={Hq} Hkv={Hkv} D={D}")
    b = wl.ragged_batch("psr", [90], [6090], Hq, Hkv, D, 32, 200, 82 + Hq)
    d = Dev(b)
    assert rpa.select_kernel(d.q, d.k_cache, d.tables, d.cu_h, d.kvl_h) == rpa.KERNEL_PREFILL
    del d
    _full_check(b, label=f"prefill split rows {Hq}/{Hkv}/{D}", typical=(2e-3, 2e-4))


def test_long_context_mixed_splits():
    """Mixed batch with a chunk at a 40k context and decodes up to 70k keys."""
    say("long-context mixed splits")
    b = wl.ragged_batch("lcm", [300, 1, 1, 1], [40300, 9001, 101, 70001], 32, 8, 128, 16, 7500, 81)
    _sampled(b, 160, "long-context mixed", typical=(8e-3, 1e-4))


@pytest.mark.parametrize("n_seqs", [160, 161, 300])
def test_many_decode_sequences_order_and_scan(n_seqs):
    """Up to 160 decode-class sequences the decode items follow a host-built longest-first
    order carried in the kernel arguments; beyond that the in-kernel scan maps them.  Both
    sides of the limit, and a mixed batch, against the oracle on sampled rows."""
    say(f"{n_seqs} decode sequences")
    rng = np.random.default_rng(n_seqs)
    kv = rng.integers(1, 700, size=n_seqs)
    q = np.ones(n_seqs, np.int64)
    pool = int(((kv + 15) // 16).sum()) + 48
    b = wl.ragged_batch("many", q, kv, 8, 2, 128, 16, pool, 71, max_pages=48)
    _sampled(b, 300, f"{n_seqs} decodes")
    q[0], kv[0] = 40, 640   # one prefill chunk makes it a mixed batch
    b2 = wl.ragged_batch("many_mixed", q, kv, 8, 2, 128, 16, pool, 72, max_pages=48)
    _sampled(b2, 300, f"{n_seqs} mixed")


@pytest.mark.parametrize("nsplit_ctx", [0, 6000])
def test_uniform_prefill_batch_rank_by_rank(nsplit_ctx):
    """Prefill-only batches whose sequences share q_len and kv_len run q-tile rank by rank
    across the sequences; with and without KV splits (a long shared context), group size 4,
    fused write, every output element against the oracle."""
    say(f"uniform prefill batch, context {nsplit_ctx}")
    q = [96, 96, 96]
    kv = [96 + nsplit_ctx] * 3
    pool = sum((k + 15) // 16 for k in kv) + 4
    b = wl.ragged_batch("uni", q, kv, 8, 2, 64, 16, pool, 83 + nsplit_ctx)
    d = Dev(b)
    assert rpa.select_kernel(d.q, d.k_cache, d.tables, d.cu_h, d.kvl_h) == rpa.KERNEL_PREFILL
    del d
    _full_check(b, label=f"uniform prefill context {nsplit_ctx}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_bad_table_entry_is_never_stored_through(kernel):
    """A block-table entry outside [0, num_pages) where only new tokens land (the precondition
    broken): the fused write skips those stores, every other cache byte is as the oracle
    writes it, and the outputs are exact (readers take new keys from k_new, never from the
    cache).  rpa_write_kv skips them the same way."""
    say(f"bad table entry kernel={kernel}")
    b = wl.ragged_batch("bad", [1, 3, 20], [40, 35, 80], 8, 2, 128, 16, 20, 95)
    page = int(b.block_tables[1, 2])          # sequence 1: past 32, new tokens in block 2
    kc, vc = oracle_after_write(b)
    ref = oracle.attention(b.q, kc, vc, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale, 16, 2)
    kc_want, vc_want = kc.copy(), vc.copy()
    kc_want[page], vc_want[page] = b.k_cache[page], b.v_cache[page]   # never written
    for bad in (b.num_pages + 7, -1):
        bb = wl.RaggedBatch(**{**b.__dict__})
        bb.block_tables = b.block_tables.copy()
        bb.block_tables[1, 2] = bad
        d = Dev(bb)
        out = d.attention(kernel=kernel)
        assert np.array_equal(to_host_bits(d.k_cache), kc_want), f"entry {bad}: K cache differs"
        assert np.array_equal(to_host_bits(d.v_cache), vc_want), f"entry {bad}: V cache differs"
        compare(to_host_f32(out), ref, f"bad entry {bad} kernel={kernel}")
        w = Dev(bb)
        w.write()
        assert np.array_equal(to_host_bits(w.k_cache), kc_want), f"entry {bad}: rpa_write_kv K"
        assert np.array_equal(to_host_bits(w.v_cache), vc_want), f"entry {bad}: rpa_write_kv V"
