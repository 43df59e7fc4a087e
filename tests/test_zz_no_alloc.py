"""rpa_attention_noalloc (split partials in the library's static device scratch, no workspace)
through the C ABI, against rpa_attention with a workspace on the same batches: outputs and
caches bit-identical (same kernels and plan), both within the contract of the oracle.  Two
calls in a row, the second on a smaller batch (the scratch keeps the first call's contents),
and a batch too large for the scratch is refused without a launch."""
import numpy as np
import pytest
import torch

import attention_ragged_paged_amd as rpa
import oracle
from attention_ragged_paged_amd import workloads as wl
from tests.gpu_util import Dev, compare, oracle_after_write, say, to_host_bits, to_host_f32

pytestmark = pytest.mark.gpu


def _noalloc(d, out):
    b = d.b
    return rpa.attention_noalloc(d.q, d.k_cache, d.v_cache, d.tables, d.cu, d.kvl, b.scale,
                                 out=out, k_new=d.k_new, v_new=d.v_new, cu_q_lens_host=d.cu_h,
                                 kv_lens_host=d.kvl_h)


def test_noalloc_matches_workspace_call_twice_in_a_row():
    big = wl.ragged_batch("na1", [1, 1, 100, 3, 1], [5000, 3000, 6000, 40, 900], 32, 8, 128, 16,
                          1100, 91)
    small = wl.ragged_batch("na2", [1, 30], [2000, 900], 32, 8, 128, 16, 220, 92)
    for b in (big, small):   # both split some sequences, so the scratch is used
        d = Dev(b)
        need = rpa.workspace_size(d.q, d.k_cache, d.tables, d.cu_h, d.kvl_h)
        assert 0 < need <= rpa.NOALLOC_SCRATCH_BYTES, need
    outs = {}
    for name, b in (("big", big), ("small", small)):
        say(f"no-alloc call on the {name} batch: q_lens {np.diff(b.cu_q_lens).tolist()}")
        ref_dev = Dev(b)
        ref = ref_dev.attention()            # rpa_attention with a workspace, fused write
        d = Dev(b)
        out = torch.full_like(d.q, 5.0)
        got = _noalloc(d, out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), \
            f"{name}: rpa_attention_noalloc differs from rpa_attention"
        assert torch.equal(d.k_cache.view(torch.int16), ref_dev.k_cache.view(torch.int16))
        assert torch.equal(d.v_cache.view(torch.int16), ref_dev.v_cache.view(torch.int16))
        kc, vc = oracle_after_write(b)
        assert np.array_equal(to_host_bits(d.k_cache), kc)
        ref_o = oracle.attention(b.q, kc, vc, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale,
                                 b.page_size, b.num_kv_heads)
        compare(to_host_f32(got), ref_o, f"no-alloc {name}")
        outs[name] = got
    # the big batch again, after the small one, still equals its first result
    d = Dev(big)
    again = _noalloc(d, torch.empty_like(d.q))
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), outs["big"].view(torch.int16))


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    b = wl.ragged_batch("na3", [300, 1, 1, 1], [40300, 9001, 101, 70001], 32, 8, 128, 16, 7500,
                        93)
    d = Dev(b)
    need = rpa.workspace_size(d.q, d.k_cache, d.tables, d.cu_h, d.kvl_h)
    assert need > rpa.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(d.q, 5.0)
    with pytest.raises(rpa.RpaError) as ei:
        _noalloc(d, out)
    assert ei.value.status == 3 and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out.float() == 5.0).all()), "a refused call must launch nothing"
