"""Helpers shared by the GPU tests: move a seeded batch to the device, run the HIP path
through the C ABI, and compare with the CPU oracle."""
import sys

import numpy as np
import torch

import attention_ragged_paged_amd as rpa
import oracle
from attention_ragged_paged_amd import workloads as wl

ATOL = 2e-2   # max-abs bound for bf16 inputs, fp32 accumulation, bf16 output


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_dev(arr):
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()


def i32_dev(arr):
    return torch.from_numpy(np.ascontiguousarray(arr, np.int32)).cuda()


def to_host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def to_host_f32(t):
    return t.float().cpu().numpy()


def cache_dev(arr):
    """A cache to the device: bf16 bit patterns, or FP8 codes (uint8) as they are."""
    if arr.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(arr)).cuda()
    return bf16_dev(arr)


def cache_host(t):
    """A device cache back as the oracle's array type (uint16 bf16 bits or uint8 codes)."""
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return to_host_bits(t)


class Dev:
    """Device copies of a RaggedBatch."""

    def __init__(self, b: wl.RaggedBatch):
        self.b = b
        self.q = bf16_dev(b.q)
        self.k_new = bf16_dev(b.k_new)
        self.v_new = bf16_dev(b.v_new)
        self.k_cache = cache_dev(b.k_cache)
        self.v_cache = cache_dev(b.v_cache)
        self.tables = i32_dev(b.block_tables)
        self.cu = i32_dev(b.cu_q_lens)
        self.kvl = i32_dev(b.kv_lens)
        self.cu_h = torch.from_numpy(np.ascontiguousarray(b.cu_q_lens, np.int32))
        self.kvl_h = torch.from_numpy(np.ascontiguousarray(b.kv_lens, np.int32))

    def attention(self, fused_write=True, kernel=rpa.KERNEL_AUTO, tables=None, kv_lens=None,
                  kv_lens_host=None):
        out = rpa.attention(self.q, self.k_cache, self.v_cache,
                            self.tables if tables is None else tables, self.cu,
                            self.kvl if kv_lens is None else kv_lens, self.b.scale,
                            k_new=self.k_new if fused_write else None,
                            v_new=self.v_new if fused_write else None,
                            cu_q_lens_host=self.cu_h,
                            kv_lens_host=self.kvl_h if kv_lens_host is None else kv_lens_host,
                            kernel=kernel, k_scale=self.b.k_scale, v_scale=self.b.v_scale)
        torch.cuda.synchronize()
        return out

    def write(self):
        rpa.write_kv(self.k_new, self.v_new, self.k_cache, self.v_cache, self.tables, self.cu,
                     self.kvl, cu_q_lens_host=self.cu_h, kv_lens_host=self.kvl_h,
                     k_scale=self.b.k_scale, v_scale=self.b.v_scale)
        torch.cuda.synchronize()


def oracle_after_write(b: wl.RaggedBatch):
    """Caches after the oracle's scatter of the new tokens."""
    return oracle.write_kv(b.cu_q_lens, b.kv_lens, b.block_tables, b.k_new, b.v_new, b.k_cache,
                           b.v_cache, b.page_size, layout=b.layout, k_scale=b.k_scale,
                           v_scale=b.v_scale)


def oracle_attention(b: wl.RaggedBatch, k_cache, v_cache, **kw):
    """The oracle's attention over the given caches (FP8 caches with the batch's scales)."""
    return oracle.attention(b.q, k_cache, v_cache, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale,
                            b.page_size, b.num_kv_heads, layout=b.layout, k_scale=b.k_scale,
                            v_scale=b.v_scale, **kw)


def sample_rows(b: wl.RaggedBatch, n, seed=0):
    """(token, head) rows spread over every sequence: first/last tokens, tile edges, random."""
    rng = np.random.default_rng(seed)
    rows = set()
    Hq = b.num_q_heads
    for s in range(b.num_seqs):
        q0, q1 = int(b.cu_q_lens[s]), int(b.cu_q_lens[s + 1])
        if q1 == q0:
            continue
        for t in {q0, q1 - 1, (q0 + q1) // 2}:
            rows.add((t, int(rng.integers(Hq))))
            rows.add((t, 0))
            rows.add((t, Hq - 1))
    T = b.total_q
    while len(rows) < n:
        rows.add((int(rng.integers(T)), int(rng.integers(Hq))))
    return np.array(sorted(rows), np.int32)


def compare(got_f32, want_f64, label, row_scale=None, typical=None):
    """max-abs within ATOL, or, with row_scale ([rows] or [T, Hq], one value per output row),
    within ATOL * max(1, row_scale) per row.  typical = (max_abs, mean_abs): bounds on the
    error level itself, far below the contract, that catch regressions the contract would
    let through."""
    err = np.abs(got_f32.astype(np.float64) - want_f64)
    finite = np.isfinite(got_f32).all()
    mx = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    if row_scale is None:
        say(f"  {label}: max-abs {mx:.3e} mean-abs {mean:.3e}")
        assert finite, f"{label}: non-finite output"
        assert mx <= ATOL, f"{label}: max-abs {mx} > {ATOL}"
    else:
        tol = ATOL * np.maximum(1.0, np.asarray(row_scale, np.float64))[..., None]
        rel = float((err / tol).max()) if err.size else 0.0
        say(f"  {label}: max-abs {mx:.3e} mean-abs {mean:.3e}, worst error / row bound {rel:.3f}"
            f" (largest row bound {float(tol.max()):.3g})")
        assert finite, f"{label}: non-finite output"
        assert rel <= 1.0, f"{label}: error {rel:.3f} x the row bound ATOL * max(1, max|V|)"
    if typical is not None:
        assert mx <= typical[0], f"{label}: max-abs {mx:.3e} above its usual level {typical[0]:.1e}"
        assert mean <= typical[1], f"{label}: mean-abs {mean:.3e} above its usual level {typical[1]:.1e}"
    return mx


def visible_vmax(b: wl.RaggedBatch, v_cache, rows=None):
    """Largest |V| value (code value times v_scale for an FP8 cache) over the keys each output
    row sees: [T, Hq], or [n] for sampled rows (token, head).  The bound of an FP8 row scales
    with it: the bf16 rounding of probabilities and output is relative to the values."""
    if v_cache.dtype == np.uint8:
        lut = np.abs(oracle.fp8_decode(np.arange(256, dtype=np.uint8))) * b.v_scale
        lut[np.isnan(lut)] = 0.0
    else:
        lut = None
    S, Hkv, G = b.page_size, b.num_kv_heads, b.num_q_heads // b.num_kv_heads
    out = np.zeros((b.total_q, b.num_q_heads))
    for bi in range(b.num_seqs):
        q0, q1 = int(b.cu_q_lens[bi]), int(b.cu_q_lens[bi + 1])
        if q1 == q0:
            continue
        for g in range(Hkv):
            L = int(b.kv_lens[bi] if b.layout == wl.SEQ_MAJOR else b.kv_lens[bi, g])
            row = b.block_tables[bi] if b.layout == wl.SEQ_MAJOR else b.block_tables[bi, g]
            j = np.arange(L)
            idx = (row[j // S], j % S, np.full(L, g)) if b.layout == wl.SEQ_MAJOR else (row[j // S], j % S)
            v = v_cache[idx]
            m = lut[v].max(axis=1) if lut is not None else np.abs(wl.bf16_to_f32(v)).max(axis=1)
            cm = np.maximum.accumulate(m)
            past = L - (q1 - q0)
            out[q0:q1, g * G:(g + 1) * G] = cm[past + np.arange(q1 - q0)][:, None]
    if rows is not None:
        return out[rows[:, 0], rows[:, 1]]
    return out
