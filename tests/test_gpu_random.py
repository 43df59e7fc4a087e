"""GPU parity over seeded random batches: shapes, group sizes, page sizes, layouts, cache types,
length mixes and forced kernels drawn per case, every output element against the CPU oracle.

Each case draws: head dim 64 or 128; 1-8 KV heads with 1-16 query heads each; page size
16-1024; sequence-major or KV-head-major pages (the latter sometimes with a kv_len per KV
head); bf16 or FP8 E4M3 caches; 1-8 sequences whose q_len is 0, 1, a few, tens or hundreds of
tokens over a past of 0-3000 tokens; the automatic or a forced kernel; the fused or a separate
cache write.  Odd cases also run the graph-capturable call (device-side plan, a random KV
split cap) on fresh copies of the same inputs.  Cache writes bit-exact, attention within
max-abs 2e-2.
"""
import numpy as np
import pytest
import torch

import attention_ragged_paged_amd as rpa
from attention_ragged_paged_amd import workloads as wl
from tests.gpu_util import (Dev, cache_host, compare, oracle_after_write, oracle_attention, say,
                            to_host_f32, visible_vmax)

pytestmark = pytest.mark.gpu

KERNELS = [rpa.KERNEL_AUTO, rpa.KERNEL_DECODE, rpa.KERNEL_PREFILL, rpa.KERNEL_MIXED]


def random_case(seed):
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    Hq = Hkv * int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    S = int(rng.choice([16, 32, 64, 128, 256, 512, 1024]))
    layout = wl.SEQ_MAJOR if rng.random() < 0.6 else wl.HEAD_MAJOR
    kv_dtype = "fp8" if rng.random() < 0.3 else "bf16"
    B = int(rng.integers(1, 9))
    q_lens, kv_lens = [], []
    for _ in range(B):
        r = rng.random()
        q = (0 if r < 0.08 else 1 if r < 0.45 else int(rng.integers(2, 8)) if r < 0.6
             else int(rng.integers(8, 200)) if r < 0.9 else int(rng.integers(200, 700)))
        past = 0 if rng.random() < 0.15 else int(rng.integers(0, 3000))
        q_lens.append(q)
        kv_lens.append(q + past)
    kv = np.asarray(kv_lens)
    if layout == wl.HEAD_MAJOR and rng.random() < 0.5:
        kv = np.stack([np.maximum(np.asarray(q_lens), kv - rng.integers(0, 200, size=B))
                       for _ in range(Hkv)], 1)
    # pages: one set per sequence, or one per (sequence, KV head) in the KV-head-major layout
    per_head = kv if kv.ndim == 2 else np.repeat(kv[:, None], Hkv, 1)
    blocks = per_head if layout == wl.HEAD_MAJOR else kv
    pool = int(((blocks + S - 1) // S).sum())
    scale = float(rng.uniform(0.03, 0.15))
    kernel = int(rng.choice(KERNELS))
    fused = bool(rng.random() < 0.7)
    splits = int(rng.choice([1, 2, 4, 8, 16, 64]))
    b = wl.ragged_batch("rand", q_lens, kv, Hq, Hkv, D, S, pool + 3, seed, layout=layout,
                        scale=scale, kv_dtype=kv_dtype)
    desc = (f"seed {seed}: D={D} heads={Hq}/{Hkv} S={S} layout={layout} kv={kv_dtype} "
            f"q={q_lens} kv_lens={kv.tolist()} kernel={kernel} fused={fused}")
    return b, kernel, fused, splits, desc


@pytest.mark.parametrize("seed", range(10000, 10048))
def test_random_batch(seed):
    b, kernel, fused, splits, desc = random_case(seed)
    say(desc)
    kc, vc = oracle_after_write(b)
    ref = oracle_attention(b, kc, vc)
    d = Dev(b)
    if not fused:
        d.write()
    out = d.attention(fused_write=fused, kernel=kernel)
    assert np.array_equal(cache_host(d.k_cache), kc), f"{desc}: K cache differs"
    assert np.array_equal(cache_host(d.v_cache), vc), f"{desc}: V cache differs"
    scale = visible_vmax(b, vc) if b.kv_fp8 else None
    compare(to_host_f32(out), ref, desc, row_scale=scale)
    if seed % 2 == 0 or b.total_q == 0:
        return
    say(f"  graph call, at most {splits} splits")
    g = Dev(b)
    ga = rpa.GraphAttention(g.q, g.k_cache, g.v_cache, g.tables, g.cu, g.kvl, b.scale,
                            k_new=g.k_new, v_new=g.v_new, max_splits=splits, k_scale=b.k_scale,
                            v_scale=b.v_scale)
    out_g = ga()
    torch.cuda.synchronize()
    assert ga.status() == 0
    assert np.array_equal(cache_host(g.k_cache), kc), f"{desc}: graph K cache differs"
    assert np.array_equal(cache_host(g.v_cache), vc), f"{desc}: graph V cache differs"
    compare(to_host_f32(out_g), ref, desc + " (graph)", row_scale=scale)
