"""The structured long-context checks (tests/structured.py) on the CPU oracle: they pass on the
oracle's own output and fail when the oracle reads one page wrongly, so the GPU tests that use
them can see a missing, duplicated or misplaced page that the 2e-2 contract cannot."""
import numpy as np
import pytest

import oracle
from attention_ragged_paged_amd import workloads as wl
from tests import structured as st


def _batch(layout=wl.SEQ_MAJOR):
    kv = [900, 333, 1000] if layout == wl.SEQ_MAJOR else [[900, 700], [333, 400], [1000, 111]]
    kv_arr = np.array(kv)
    pool = int(((kv_arr + 15) // 16).sum()) + 6
    return wl.ragged_batch("st", [1, 5, 40], kv, 8, 2, 64, 16, pool, 9, layout=layout)


def _oracle_bf16(b, tables, **kw):
    """The oracle after its write, rounded to bf16 as the GPU's output is."""
    kc, vc = oracle.write_kv(b.cu_q_lens, b.kv_lens, b.block_tables, b.k_new, b.v_new,
                             b.k_cache, b.v_cache, b.page_size, layout=b.layout)
    out = oracle.attention(b.q, kc, vc, tables, b.cu_q_lens, b.kv_lens, b.scale, b.page_size,
                           b.num_kv_heads, layout=b.layout, **kw)
    return wl.bf16_to_f32(wl.bf16_bits(out.astype(np.float32))).astype(np.float64)


def _moved(tables, layout, how):
    """A copy of the tables with pages read wrongly: 'dup' reads block 21's page for block
    20 of sequence 0 (page 20 dropped, 21 twice); 'far' reads block 53's page for block 21
    (same parity, differ in bits 5 and 1); 'swap_at_limit' swaps the pages of blocks 60 and 61
    of sequence 2, whose rows' causal limits run through them (a swap of two pages that every
    row sees changes no output: attention is a function of the set of visible keys)."""
    t = tables.copy()
    row = t[0] if layout == wl.SEQ_MAJOR else t[0, 0]
    if how == "dup":
        row[20] = row[21]
    elif how == "far":
        row[21] = row[53]
    else:
        r2 = t[2] if layout == wl.SEQ_MAJOR else t[2, 0]
        r2[60], r2[61] = r2[61], r2[60]
    return t


@pytest.mark.parametrize("layout", [wl.SEQ_MAJOR, wl.HEAD_MAJOR])
def test_equal_scores_exact_on_oracle(layout):
    b = _batch(layout)
    sb, expected = st.equal_scores_batch(b)
    ok, msg = st.bf16_ulp_check(_oracle_bf16(sb, sb.block_tables), expected, "oracle")
    assert ok, msg


@pytest.mark.parametrize("how", ["dup", "far", "swap_at_limit"])
@pytest.mark.parametrize("layout", [wl.SEQ_MAJOR, wl.HEAD_MAJOR])
def test_equal_scores_see_a_moved_page(layout, how):
    b = _batch(layout)
    sb, expected = st.equal_scores_batch(b)
    # the duplicated page holds data, so only the pattern (not the NaN poison) can expose it
    got = _oracle_bf16(sb, _moved(sb.block_tables, layout, how))
    ok, msg = st.bf16_ulp_check(got, expected, "oracle with a moved page")
    assert not ok, "a moved page went unnoticed"


def test_equal_scores_see_a_dropped_tail_key():
    """Reading one key fewer in the last page (causal limit off by one) is caught too."""
    b = _batch()
    sb, expected = st.equal_scores_batch(b)
    kv = sb.kv_lens.copy()
    kv[2] -= 1   # sequence 2 one key short: its rows see one key less
    sb2 = wl.RaggedBatch(**{**sb.__dict__})
    sb2.kv_lens = kv
    kc, vc = oracle.write_kv(sb.cu_q_lens, sb.kv_lens, sb.block_tables, sb.k_new, sb.v_new,
                             sb.k_cache, sb.v_cache, 16)
    out = oracle.attention(sb.q, kc, vc, sb.block_tables, sb.cu_q_lens, kv, sb.scale, 16, 2)
    got = wl.bf16_to_f32(wl.bf16_bits(out.astype(np.float32))).astype(np.float64)
    ok, _ = st.bf16_ulp_check(got, expected, "oracle, one key short")
    assert not ok


def _run_dominant_on_oracle(b, tables, launches):
    bad = 0
    for edits in launches:
        pb = st.plant_host(b, edits)
        rows = np.array([[e.token, e.head] for e in edits], np.int32)
        kc, vc = oracle.write_kv(pb.cu_q_lens, pb.kv_lens, pb.block_tables, pb.k_new, pb.v_new,
                                 pb.k_cache, pb.v_cache, pb.page_size, layout=pb.layout)
        out = oracle.attention(pb.q, kc, vc, tables, pb.cu_q_lens, pb.kv_lens, pb.scale,
                               pb.page_size, pb.num_kv_heads, layout=pb.layout, rows=rows)
        got = wl.bf16_to_f32(wl.bf16_bits(out.astype(np.float32))).astype(np.float64)
        ok, _ = st.dominant_check(got, edits, "oracle")
        bad += not ok
    return bad


@pytest.mark.parametrize("layout", [wl.SEQ_MAJOR, wl.HEAD_MAJOR])
def test_dominant_sweep_on_oracle(layout):
    """Every boundary position of sequence 0 returns its V row through the right table, and
    not through a table that never reads block 20's page (block 21's read in its place)."""
    b = _batch(layout)
    L = int(b.kv_lens[0] if layout == wl.SEQ_MAJOR else b.kv_lens[0, 0])
    ps = st.boundary_positions(L, step=16)
    targets = [(0, 0, p) for p in ps]
    launches = st.dominant_launches(b, targets)
    assert _run_dominant_on_oracle(b, b.block_tables, launches) == 0
    assert _run_dominant_on_oracle(b, _moved(b.block_tables, layout, "dup"), launches) > 0


def test_pattern_prefix_sums_stay_small():
    """The property the equal-score check rests on: |sum over keys 0..n-1| <= 2 S per column."""
    for S in (16, 64):
        pat = st.pattern(np.arange(50000), S, 5, 128)
        assert np.abs(np.cumsum(pat, axis=0)).max() <= 2 * S
