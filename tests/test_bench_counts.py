"""The benchmark's algorithmic work counts (bytes and flops per step) against brute-force
enumeration on small batches: every (query row, visible key) pair and every byte the path
must touch, counted one by one."""
import numpy as np
import pytest

import bench
from attention_ragged_paged_amd import workloads as wl


def _brute_flops(b):
    G = b.num_q_heads // b.num_kv_heads
    kv = b.kv_lens.reshape(b.num_seqs, -1)
    total = 0
    for s in range(b.num_seqs):
        q_len = int(b.cu_q_lens[s + 1] - b.cu_q_lens[s])
        for h in range(b.num_q_heads):
            g = h // G
            kv_len = int(kv[s, g if kv.shape[1] > 1 else 0])
            past = kv_len - q_len
            for t in range(q_len):
                total += (past + t + 1) * 4 * b.head_dim   # q.k and p.v per visible key
    return total


def _brute_bytes(b):
    D, Hq, Hkv, S = b.head_dim, b.num_q_heads, b.num_kv_heads, b.page_size
    eb = b.k_cache.itemsize                             # bytes per cached element
    kv = b.kv_lens.reshape(b.num_seqs, -1)
    total = 0
    for s in range(b.num_seqs):
        for g in range(Hkv):
            L = int(kv[s, g if kv.shape[1] > 1 else 0])
            total += L * D * eb * 2                     # K and V rows of this KV head
            if kv.shape[1] > 1 or g == 0:               # one table per sequence (per head if head-major)
                total += -(-L // S) * 4
    total += b.total_q * Hq * D * 2 * 2                 # Q read, O written
    total += (b.num_seqs + 1) * 4 + kv.size * 4         # cu_q_lens, kv_lens
    total += b.total_q * Hkv * D * 2 * 2                # new K/V read (bf16)
    total += b.total_q * Hkv * D * eb * 2               # and written into the caches
    return total


@pytest.mark.parametrize("make", [
    lambda: wl.tiny_ragged(),
    lambda: wl.ragged_batch("c", [3, 1, 0, 17], [40, 9, 5, 17], 8, 2, 64, 16, 20, 7),
    lambda: wl.ragged_batch("h", [5, 1], np.array([[30, 12], [9, 44]]), 8, 2, 128, 16, 20, 8,
                            layout=wl.HEAD_MAJOR),
    lambda: wl.ragged_batch("f", [3, 1, 0, 17], [40, 9, 5, 17], 8, 2, 64, 16, 20, 7,
                            kv_dtype="fp8"),
])
def test_counts_match_brute_force(make):
    b = make()
    assert bench.causal_flops(b) == _brute_flops(b)
    assert bench.step_bytes(b) == _brute_bytes(b)


def test_traffic_record_is_ignored_when_the_kernel_changed(tmp_path, monkeypatch):
    import json
    import os
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    os.makedirs(tmp_path / "attention_ragged_paged_amd" / "csrc")
    for name in ("attention.hip", "rpa_device.h"):
        (tmp_path / "attention_ragged_paged_amd" / "csrc" / name).write_text("v1")
    sha = bench.kernel_source_sha()
    rec = {"source_sha": sha, "bytes_per_launch": 123}
    (tmp_path / "profiles" / "w_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("w") == 123
    (tmp_path / "attention_ragged_paged_amd" / "csrc" / "attention.hip").write_text("v2")
    assert bench.measured_traffic("w") is None
