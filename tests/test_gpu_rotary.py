"""GPU parity of the fused rotary + packed-QKV scatter (rpa_rotary_write_kv) against the oracle.

Rotated Q and the caches bit for bit (both sides evaluate the same fp32 fused multiply-adds
and round to bf16 to nearest even); then attention over the updated caches within max-abs 2e-2.
"""
import numpy as np
import pytest
import torch

import attention_ragged_paged_amd as rpa
import oracle
from attention_ragged_paged_amd import workloads as wl
from tests.gpu_util import (Dev, bf16_dev, cache_host, compare, oracle_attention, say,
                            to_host_bits, to_host_f32, visible_vmax)

pytestmark = pytest.mark.gpu


def _tables(max_pos, rd, seed):
    rng = np.random.default_rng(seed)
    theta = rng.uniform(-np.pi, np.pi, size=(max_pos, max(rd, 2) // 2))
    return np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)


def _run(b, rd, interleaved, packed, max_pos=None):
    d = Dev(b)
    max_pos = max_pos or int(np.max(b.kv_lens)) + 3
    cos, sin = _tables(max_pos, rd, 11)
    if packed:
        qkv = torch.cat([d.q, d.k_new, d.v_new], dim=1).reshape(b.total_q, -1).contiguous()
        q, k, v = rpa.split_packed_qkv(qkv, b.num_q_heads, b.num_kv_heads)
    else:
        q, k, v = d.q, d.k_new, d.v_new
    q_out = rpa.rotary_write_kv(q, k, v, d.k_cache, d.v_cache, d.tables, d.cu, d.kvl,
                                cos_cache=torch.from_numpy(cos).cuda(),
                                sin_cache=torch.from_numpy(sin).cuda(), rotary_dim=rd,
                                interleaved=interleaved, cu_q_lens_host=d.cu_h,
                                kv_lens_host=d.kvl_h, k_scale=b.k_scale, v_scale=b.v_scale)
    torch.cuda.synchronize()
    qo, kc, vc = oracle.rotary_qkv(b.cu_q_lens, b.kv_lens, b.block_tables, b.q, b.k_new, b.v_new,
                                   b.k_cache, b.v_cache, b.page_size, cos, sin, rd, interleaved,
                                   layout=b.layout, k_scale=b.k_scale, v_scale=b.v_scale)
    return d, q_out, qo, kc, vc


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("layout", [wl.SEQ_MAJOR, wl.HEAD_MAJOR])
@pytest.mark.parametrize("D,rd,interleaved,packed", [
    (128, 128, False, True), (128, 128, True, False), (128, 64, False, False),
    (128, 32, True, True), (64, 64, False, True), (64, 16, True, False), (128, 0, False, True),
])
def test_rotary_write_bit_exact(kv_dtype, layout, D, rd, interleaved, packed):
    say(f"rotary write {kv_dtype} layout={layout} D={D} rd={rd} interleaved={interleaved} "
        f"packed={packed}")
    pool = 60 if layout == wl.SEQ_MAJOR else 110
    b = wl.ragged_batch("rot", [1, 7, 0, 33, 16], [17, 23, 5, 100, 16], 8, 2, D, 16, pool, 21,
                        layout=layout, kv_dtype=kv_dtype)
    d, q_out, qo, kc, vc = _run(b, rd, interleaved, packed)
    assert np.array_equal(to_host_bits(q_out), qo), "rotated Q differs"
    assert np.array_equal(cache_host(d.k_cache), kc), "K cache differs"
    assert np.array_equal(cache_host(d.v_cache), vc), "V cache differs"


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_rotary_then_attention(kv_dtype):
    """The full path for a packed-QKV model: rotate + scatter, then attention over the caches
    with no new K/V in the call."""
    say(f"rotary then attention {kv_dtype}")
    b = wl.ragged_batch("rota", [1, 40, 1, 3], [60, 700, 120, 33], 16, 4, 128, 16, 70, 31,
                        kv_dtype=kv_dtype)
    d, q_out, qo, kc, vc = _run(b, 128, False, True)
    out = rpa.attention(q_out, d.k_cache, d.v_cache, d.tables, d.cu, d.kvl, b.scale,
                        cu_q_lens_host=d.cu_h, kv_lens_host=d.kvl_h, k_scale=b.k_scale,
                        v_scale=b.v_scale)
    torch.cuda.synchronize()
    ref = oracle.attention(qo, kc, vc, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale,
                           b.page_size, b.num_kv_heads, k_scale=b.k_scale, v_scale=b.v_scale)
    compare(to_host_f32(out), ref, f"rotary + attention {kv_dtype}",
            row_scale=visible_vmax(b, vc) if kv_dtype == "fp8" else None)


def test_rotary_llama3_prefill_size():
    """4 x 2048 tokens of packed QKV with full-head split rotary (Llama-3 style)."""
    say("rotary llama3 prefill size")
    b = wl.llama3_prefill()
    d, q_out, qo, kc, vc = _run(b, 128, False, True, max_pos=8192)
    assert np.array_equal(to_host_bits(q_out), qo)
    assert np.array_equal(cache_host(d.k_cache), kc)
    assert np.array_equal(cache_host(d.v_cache), vc)
