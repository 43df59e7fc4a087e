"""GPU parity of the FP8 (E4M3) KV cache against the CPU oracle.

Cache writes bit-exact: every stored code equals the oracle's encode of float32(x) * float32(1 /
scale) (clamped to +-448, nearest even).  Attention over the codes: both sides read the same
dequantized values (every E4M3 value is exact in bf16), so what remains is the bf16 rounding of
probabilities and outputs, which is relative to the values: each output row must lie within
2e-2 * max(1, max |V| over the keys the row sees) of the oracle.  The caches hold codes over the
whole E4M3 range (zero, subnormals, up to +-448: values up to 112 at the scale 1/4) beside
codes of order one.
"""
import numpy as np
import pytest
import torch

import attention_ragged_paged_amd as rpa
import oracle
from attention_ragged_paged_amd import workloads as wl
from tests.gpu_util import (Dev, bf16_dev, cache_host, compare, i32_dev, oracle_after_write,
                            oracle_attention, sample_rows, say, to_host_f32, visible_vmax)

pytestmark = pytest.mark.gpu

KERNELS = [rpa.KERNEL_AUTO, rpa.KERNEL_DECODE, rpa.KERNEL_PREFILL, rpa.KERNEL_MIXED]


def _batch(q_lens, kv_lens, Hq=8, Hkv=2, D=128, S=16, seed=0, layout=wl.SEQ_MAJOR, **kw):
    pool = kw.pop("pool", None)
    if pool is None:
        kvh = np.asarray(kv_lens)
        if layout == wl.HEAD_MAJOR and kvh.ndim == 1:   # one page set per KV head
            kvh = np.repeat(kvh[:, None], Hkv, axis=1)
        pool = int(((kvh + S - 1) // S).sum()) + 4
    return wl.ragged_batch("f8", q_lens, kv_lens, Hq, Hkv, D, S, pool, seed, layout=layout,
                           kv_dtype="fp8", **kw)


def _check(b, kernel=rpa.KERNEL_AUTO, fused=True, label=""):
    d = Dev(b)
    if not fused:
        d.write()
    out = d.attention(fused_write=fused, kernel=kernel)
    kc, vc = oracle_after_write(b)
    assert np.array_equal(cache_host(d.k_cache), kc), f"{label}: K cache differs"
    assert np.array_equal(cache_host(d.v_cache), vc), f"{label}: V cache differs"
    ref = oracle_attention(b, kc, vc)
    return compare(to_host_f32(out), ref, label, row_scale=visible_vmax(b, vc))


@pytest.mark.parametrize("layout", [wl.SEQ_MAJOR, wl.HEAD_MAJOR])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_write_kv_bit_exact(layout, D):
    say(f"fp8 write_kv layout={layout} D={D}")
    b = _batch([1, 7, 0, 33, 16], [17, 23, 5, 100, 16], D=D, seed=21, layout=layout)
    d = Dev(b)
    d.write()
    kc, vc = oracle_after_write(b)
    assert np.array_equal(cache_host(d.k_cache), kc)
    assert np.array_equal(cache_host(d.v_cache), vc)


def test_fp8_write_ties_saturation_and_odd_scales():
    """New values placed on every midpoint between neighbouring codes (ties go to the even
    code), beyond the largest finite value (saturation), in the subnormal range, and scales
    that are not powers of two."""
    say("fp8 write ties / saturation / odd scales")
    b = _batch([64, 1], [64, 30], Hq=4, Hkv=2, D=128, seed=5)
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = oracle.fp8_decode(codes)
    mids = (vals[1:] + vals[:-1]) / 2                       # 126 ties, exact in bf16
    special = np.array([448.0, 480.0, 1e6, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -12])
    pool = np.concatenate([mids, -mids, special, -special])
    rng = np.random.default_rng(3)
    for ks, vs, label in [(b.k_scale, b.v_scale, "power-of-two scales"), (0.37, 1.9, "odd scales")]:
        bb = wl.RaggedBatch(**{**b.__dict__})
        x = rng.choice(pool, size=b.k_new.shape) * ks       # x * (1/ks) lands on the ties
        bb.k_new = wl.bf16_bits(x.astype(np.float32))
        bb.v_new = wl.bf16_bits((rng.choice(pool, size=b.v_new.shape) * vs).astype(np.float32))
        bb.k_scale, bb.v_scale = ks, vs
        d = Dev(bb)
        d.write()
        kc, vc = oracle_after_write(bb)
        assert np.array_equal(cache_host(d.k_cache), kc), label
        assert np.array_equal(cache_host(d.v_cache), vc), label


@pytest.mark.parametrize("kernel", KERNELS)
def test_fp8_tiny_ragged_every_kernel(kernel):
    say(f"fp8 tiny ragged kernel={kernel}")
    b = wl.tiny_ragged(kv_dtype="fp8")
    _check(b, kernel=kernel, label=f"fp8 tiny kernel={kernel}")


def test_fp8_separate_write_then_attend():
    say("fp8 write then attend")
    _check(wl.tiny_ragged(kv_dtype="fp8"), fused=False, label="fp8 write-then-attend")


@pytest.mark.parametrize("qs,past,Hq,Hkv,S,D", [
    ([1, 4, 16], [40, 100, 7], 8, 2, 16, 128),
    ([48, 1, 3], [200, 75, 0], 32, 8, 64, 128),
    ([33, 1], [17, 300], 4, 4, 32, 64),
    ([100], [150], 14, 2, 16, 128),
    ([1, 1, 1, 1], [1000, 17, 64, 555], 32, 8, 16, 128),
    ([70, 2], [0, 90], 8, 1, 128, 64),
])
def test_fp8_ragged_cases(qs, past, Hq, Hkv, S, D):
    kv = [q + p for q, p in zip(qs, past)]
    b = _batch(qs, kv, Hq=Hq, Hkv=Hkv, D=D, S=S, seed=sum(kv), scale=0.06)
    for kernel in KERNELS:
        say(f"fp8 case q={qs} past={past} heads={Hq}/{Hkv} S={S} D={D} kernel={kernel}")
        _check(b, kernel=kernel, label=f"fp8 q={qs} kernel {kernel}")


def test_fp8_odd_scales_attention():
    say("fp8 attention with odd scales")
    b = _batch([1, 20, 1], [300, 80, 45], Hq=8, Hkv=2, seed=77)
    b.k_scale, b.v_scale = 0.2113, 0.2671   # not powers of two
    _check(b, label="fp8 odd scales")


@pytest.mark.parametrize("kernel", KERNELS)
def test_fp8_nan_codes_in_unowned_slots_do_not_leak(kernel):
    say(f"fp8 nan poison kernel={kernel}")
    b = _batch([1, 5, 40, 1], [33, 21, 75, 250], seed=31, poison_unused=True)
    _check(b, kernel=kernel, label=f"fp8 nan kernel={kernel}")


def test_fp8_head_major_per_head_lengths():
    say("fp8 head-major per-head lengths")
    qs = [1, 33, 2]
    kv = np.array([[50, 20, 90, 7], [40, 64, 33, 100], [2, 9, 130, 61]])
    b = _batch(qs, kv, Hq=8, Hkv=4, seed=9, layout=wl.HEAD_MAJOR)
    for kernel in KERNELS:
        _check(b, kernel=kernel, label=f"fp8 head-major kernel {kernel}")


def _sampled(b, n_rows, label):
    d = Dev(b)
    out = d.attention()
    kc, vc = oracle_after_write(b)
    assert np.array_equal(cache_host(d.k_cache), kc), f"{label}: K cache differs"
    assert np.array_equal(cache_host(d.v_cache), vc), f"{label}: V cache differs"
    rows = sample_rows(b, n_rows)
    ref = oracle_attention(b, kc, vc, rows=rows)
    got = to_host_f32(out)[rows[:, 0], rows[:, 1]]
    return compare(got, ref, label, row_scale=visible_vmax(b, vc, rows))


def test_fp8_llama3_decode_full_size():
    say("fp8 llama3_decode full size")
    _sampled(wl.llama3_decode_fp8(), 512, "fp8 llama3 decode")


def test_fp8_mixed_chunked_full_size():
    say("fp8 mixed_chunked full size")
    _sampled(wl.mixed_chunked_fp8(), 400, "fp8 mixed chunked")


def test_fp8_graph_attention():
    """The graph-capturable call over an FP8 cache, eager and replayed."""
    say("fp8 graph attention")
    b = _batch([1, 40, 1, 3], [60, 700, 120, 33], Hq=16, Hkv=4, seed=13)
    d = Dev(b)
    ga = rpa.GraphAttention(d.q, d.k_cache, d.v_cache, d.tables, d.cu, d.kvl, b.scale,
                            k_new=d.k_new, v_new=d.v_new, max_splits=8, k_scale=b.k_scale,
                            v_scale=b.v_scale)
    k0, v0 = d.k_cache.clone(), d.v_cache.clone()
    out = ga().clone()
    torch.cuda.synchronize()
    assert ga.status() == 0
    kc, vc = oracle_after_write(b)
    assert np.array_equal(cache_host(d.k_cache), kc)
    assert np.array_equal(cache_host(d.v_cache), vc)
    ref = oracle_attention(b, kc, vc)
    compare(to_host_f32(out), ref, "fp8 graph eager", row_scale=visible_vmax(b, vc))
    graph = torch.cuda.CUDAGraph()
    d.k_cache.copy_(k0)
    d.v_cache.copy_(v0)
    with torch.cuda.graph(graph):
        ga()
    torch.cuda.synchronize()
    for i in range(3):
        d.k_cache.copy_(k0)
        d.v_cache.copy_(v0)
        ga.out.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ga.out, out), f"replay {i} differs from the eager call"
