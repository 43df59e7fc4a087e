#!/usr/bin/env python3
"""Benchmark of ragged paged attention on one MI355X; prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one pass of the whole path over one synthetic batch resident in HBM: one
rpa_attention call carrying the new tokens' K/V, i.e. one kernel launch (decode, prefill or
mixed kernel as dispatched) that scatters the new K/V into their pages, attends, and merges
its KV splits; for the block-sparse workload the union-table build comes first.  Each step is timed with HIP
events on the stream the library launches on; the L2 and the 256 MB Infinity Cache are
flushed before every step, outside the events, by reading a 1 GiB buffer (a read leaves
only clean lines behind, so no write-back of flush data lands inside the timed step).

Workloads (all seeded synthetic inputs with Llama-3-8B attention shapes, 32/8 heads, D 128):
  llama3_decode       64 decode sequences, kv_len ~ U[512, 4096], page 16, 20k-page pool (default)
  llama3_prefill      4 x 2048 new tokens, no prior context, page 64
  mixed_chunked       one 512-token chunk at context 8192 + 96 decodes, page 16
  block_union_sparse  4096-query chunk at context 131072, KV-head-major page 64, 10% block mask
  block_union_sparse_colshared
                      the same chunk with a column-shared mask (one draw per head and KV block):
                      attention over about a third of the context's pages per KV head
  tiny_ragged         the 3-sequence parity case (latency only)
  llama3_decode_fp8, mixed_chunked_fp8
                      the same batches over FP8 E4M3 K/V caches (1 byte an element, per-cache
                      scales; new K/V quantized by the call)

`value` is the step's algorithmic throughput: GB/s for the HBM-bound decode and mixed
batches, TFLOP/s for the MFMA-bound prefill and sparse ones.  `roofline` rates the
dominant kernel (the attention launch) against MI355X's published peaks: 8 TB/s HBM3E,
2.5 PFLOP/s dense bf16 MFMA.  `device_reference` gives this GPU's plain copy rate (1 GiB, bytes
read + written) and HBM-bound rooflines add their fraction of it.  `cpu_baseline` times the CPU oracle on the host cores.

The default run measures llama3_decode (the line's `value`) and then, under `workloads`, the
MFMA-bound and mixed halves of the metric: llama3_prefill, mixed_chunked, block_union_sparse
and block_union_sparse_colshared, each with its own throughput, roofline and CPU baseline
(`--only` measures the named workload alone).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "decode HBM GB/s (% peak) + prefill/mixed TFLOP/s (% MFMA peak), tokens/s"
WORKLOAD_BOUND = {"llama3_decode": "hbm", "mixed_chunked": "hbm", "tiny_ragged": "hbm",
                  "llama3_prefill": "mfma", "block_union_sparse": "mfma",
                  "block_union_sparse_colshared": "mfma",
                  "llama3_decode_fp8": "hbm", "mixed_chunked_fp8": "hbm"}
# measured after the headline workload in a default run
EXTRA_WORKLOADS = ("llama3_prefill", "mixed_chunked", "block_union_sparse",
                   "block_union_sparse_colshared")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- algorithmic counts ----

def step_bytes(b, attention_only=False):
    """Algorithmic HBM bytes: every K/V byte of every visible key read once per KV head, Q read,
    O written, block tables and lengths read; plus (whole step) new K/V read and written."""
    D, Hkv, Hq = b.head_dim, b.num_kv_heads, b.num_q_heads
    eb = 1 if b.kv_fp8 else 2   # bytes per cached element
    kv = b.kv_lens.reshape(b.num_seqs, -1)
    if b.layout == 0:
        kv_bytes = int(kv[:, 0].astype(np.int64).sum()) * Hkv * D * eb * 2
        tables = int(((kv[:, 0] + b.page_size - 1) // b.page_size).sum()) * 4
    else:
        kv_bytes = int(kv.astype(np.int64).sum()) * D * eb * 2
        tables = int(((kv + b.page_size - 1) // b.page_size).sum()) * 4
    qo = b.total_q * Hq * D * 2 * 2
    meta = (b.num_seqs + 1) * 4 + kv.size * 4
    total = kv_bytes + qo + tables + meta
    if not attention_only:
        total += b.total_q * Hkv * D * (2 + eb) * 2   # new K/V: bf16 read, cache element written
    return total


def causal_flops(b, kv_lens=None):
    """4 * D flops per visible (query row, key) pair: 2 for q.k, 2 for p.v."""
    kv = (b.kv_lens if kv_lens is None else kv_lens).reshape(b.num_seqs, -1)
    G = b.num_q_heads // b.num_kv_heads
    total = 0
    for s in range(b.num_seqs):
        q_len = int(b.cu_q_lens[s + 1] - b.cu_q_lens[s])
        for col in range(kv.shape[1]):
            past = int(kv[s, col]) - q_len
            pairs = q_len * past + q_len * (q_len + 1) // 2
            heads = b.num_q_heads if kv.shape[1] == 1 else G
            total += pairs * heads
    return 4 * b.head_dim * total


# ----------------------------------------------------------------- traffic counters ------

def kernel_source_sha():
    h = hashlib.sha256()
    for name in ("attention.hip", "rpa_device.h"):
        with open(os.path.join(ROOT, "attention_ragged_paged_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per attention launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
    valid only while the kernel source is unchanged."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != kernel_source_sha():
        return None
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------- CPU baseline ----------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(b, workload, bound, budget_s=12.0):
    """The oracle (unmodified) on the host cores over a bounded sample of the same batch."""
    import oracle
    kc, vc = oracle.write_kv(b.cu_q_lens, b.kv_lens, b.block_tables, b.k_new, b.v_new,
                             b.k_cache, b.v_cache, b.page_size, layout=b.layout,
                             k_scale=b.k_scale, v_scale=b.v_scale)
    threads = oracle.num_threads()
    rows_all = b.total_q * b.num_q_heads
    block_allowed = b.extra.get("allowed")
    # Work of a row = its visible keys; pick a bounded sample of rows (every k-th row).
    est_rate = 6.0e8 * threads   # fp64 multiply-adds per second per thread, to size the sample
    frac = min(1.0, budget_s * est_rate / max(1.0, causal_flops(b) / 2))
    stride = max(1, int(math.ceil(1.0 / frac)))
    idx = np.arange(0, rows_all, stride)
    rows = np.stack([idx // b.num_q_heads, idx % b.num_q_heads], axis=1).astype(np.int32)
    reps = 0
    t0 = time.perf_counter()
    while True:   # repeat a small sample until about budget_s of wall time has been measured
        oracle.attention(b.q, kc, vc, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale,
                         b.page_size, b.num_kv_heads, layout=b.layout,
                         block_allowed=block_allowed, rows=None if stride == 1 else rows,
                         nthreads=threads, k_scale=b.k_scale, v_scale=b.v_scale)
        reps += 1
        if time.perf_counter() - t0 >= 0.8 * budget_s or reps >= 1000:
            break
    dt = (time.perf_counter() - t0) / reps
    share = len(idx) / rows_all
    if bound == "mfma":
        value = causal_flops(b, b.extra.get("compacted_kv_lens")) * share / dt / 1e12
        unit = "TFLOP/s"
    else:
        value = step_bytes(b) * share / dt / 1e9
        unit = "GB/s"
    sample = (f"{len(idx)} of {rows_all} (token, head) rows (every {stride}th row) of the same "
              f"batch after the oracle's KV scatter, {reps} repetition(s), {dt:.2f} s each")
    return {"value": round(value, 4), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": sample, "tokens_per_s": round(b.total_q * share / dt, 2),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


# ----------------------------------------------------------------- device reference ----------

def device_reference(dev):
    """This GPU's plain streaming rate as a second denominator beside the published peak: a
    1 GiB device-to-device copy (bytes read + written), the mean of 5 back-to-back launches
    after a warmup (buffers 4x the Infinity Cache)."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    copy_ms = e0.elapsed_time(e1) / 5
    nbytes = n * 4
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_gbps": round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1), "bytes": nbytes,
            "what": "torch copy_ over 1 GiB fp32, bytes read + written"}


# ----------------------------------------------------------------- main --------------------

def measure(name, args, dev, with_cpu, cpu_budget):
    """Time one workload: inputs in HBM, warmup steps, then args.steps timed steps (each with
    the caches flushed first).  Returns the workload's record (throughput, roofline, CPU
    baseline, configuration)."""
    import torch
    import attention_ragged_paged_amd as rpa
    from attention_ragged_paged_amd import workloads as wl

    bound = WORKLOAD_BOUND[name]
    log(f"[bench] building {name} inputs")
    b = wl.WORKLOADS[name]()

    def to_dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def to_dev_i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

    def to_dev_cache(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev) if a.dtype == np.uint8 \
            else to_dev_bf16(a)

    q, kn, vn = to_dev_bf16(b.q), to_dev_bf16(b.k_new), to_dev_bf16(b.v_new)
    kc, vc = to_dev_cache(b.k_cache), to_dev_cache(b.v_cache)
    base_tables = to_dev_i32(b.block_tables)
    cu, kvl = to_dev_i32(b.cu_q_lens), to_dev_i32(b.kv_lens)
    cu_h = torch.from_numpy(np.ascontiguousarray(b.cu_q_lens, np.int32))
    kvl_h = torch.from_numpy(np.ascontiguousarray(b.kv_lens, np.int32))

    sparse = "mask" in b.extra
    prep_steps = []
    if sparse:
        mask = torch.from_numpy(b.extra["mask"]).to(dev)
        past, ctx = b.extra["past"], b.extra["context"]
        u_tables, u_counts, u_kvl = rpa.build_union_tables(mask, base_tables[0], past, ctx,
                                                           b.page_size)
        torch.cuda.synchronize()
        att_tables = u_tables[None]
        att_kvl = u_kvl[None]
        att_kvl_h = u_kvl[None].cpu()
        b.extra["compacted_kv_lens"] = att_kvl_h.numpy()
        if with_cpu:
            import oracle as _o  # (only for the CPU baseline below)
            _, _, _, sel = _o.union_tables(b.extra["mask"], b.block_tables[0], past, ctx,
                                           b.page_size)
            b.extra["allowed"] = sel[None]
        b.extra["union_density"] = (u_counts.cpu().numpy() / (ctx // b.page_size)).round(4).tolist()

        def build_tables():
            rpa.build_union_tables(mask, base_tables[0], past, ctx, b.page_size,
                                   out_tables=u_tables, out_counts=u_counts, out_kv_lens=u_kvl)
        prep_steps.append(build_tables)
    else:
        att_tables, att_kvl, att_kvl_h = base_tables, kvl, kvl_h

    # The new K/V are written through the attention's tables: for the sparse workload these are
    # the compacted union tables, whose last blocks are the chunk's own pages (same page and
    # slot for every new key as the base tables give).
    attn = rpa.PreparedAttention(q, kc, vc, att_tables, cu, att_kvl, b.scale, k_new=kn, v_new=vn,
                                 cu_q_lens_host=cu_h, kv_lens_host=att_kvl_h, k_scale=b.k_scale,
                                 v_scale=b.v_scale)
    if args.path == "graph":
        ga = rpa.GraphAttention(q, kc, vc, att_tables, cu, att_kvl, b.scale, k_new=kn, v_new=vn,
                                max_splits=16, k_scale=b.k_scale, v_scale=b.v_scale)
        ga()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            ga()
        torch.cuda.synchronize()
        attn = graph.replay
    kind = rpa.select_kernel(q, kc, att_tables, cu_h, att_kvl_h, k_scale=b.k_scale,
                             v_scale=b.v_scale)
    flush_buf = None if args.flush == "none" else torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def flush():
        if flush_buf is None:
            return
        if args.flush == "read":
            flush_buf.sum()
        else:
            flush_buf.fill_(1)

    def one_step(ev=None):
        if ev:
            ev[0].record()
        for p in prep_steps:
            p()
        if ev:
            ev[1].record()
        attn()
        if ev:
            ev[2].record()

    log(f"[bench] {name}: kernel kind {kind}; warmup {args.warmup}")
    for _ in range(args.warmup):
        flush()
        one_step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"[bench] {name}: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        one_step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([e[0].elapsed_time(e[2]) for e in events])
    attn_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    prep_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    ms = float(step_ms.mean())
    attn_avg_ms = float(attn_ms.mean())

    flops = causal_flops(b, b.extra.get("compacted_kv_lens"))
    if bound == "hbm":
        work = step_bytes(b)
        value = work / (ms * 1e-3) / 1e9
        unit = "GB/s"
        ach = step_bytes(b) / (attn_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        work = flops
        value = work / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
        ach = work / (attn_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = measured_traffic(name) if args.path == "host" else None
    roof["kernel"] = {1: "decode_kernel", 2: "prefill_kernel", 3: "mixed_kernel"}[kind] + \
        " (one launch: KV write, attention, split merge)"
    if args.path == "graph":
        roof["kernel"] = "graph replay: graph_kernel (device-planned, persistent)"
    roof["avg_launch_ms"] = round(attn_avg_ms, 5)
    # the metric's MFMA half for every workload: flops of the attention launch
    mfma = {"tflops": round(flops / (attn_avg_ms * 1e-3) / 1e12, 2),
            "frac_of_mfma_peak": round(flops / (attn_avg_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_step": flops}

    cpu = None
    if with_cpu:
        log(f"[bench] {name}: timing the CPU oracle")
        cpu = cpu_baseline(b, name, bound, budget_s=cpu_budget)

    cfg = {"workload": name, "num_seqs": b.num_seqs, "total_q": b.total_q,
           "q_heads": b.num_q_heads, "kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
           "page_size": b.page_size, "pool_pages": b.num_pages, "layout":
           "seq_major" if b.layout == 0 else "kv_head_major", "seed": b.seed,
           "sum_kv_len": int(b.kv_lens.reshape(b.num_seqs, -1)[:, 0].sum()),
           "cache_flush": args.flush, "parallelism": "none (one GPU)", "path": args.path}
    rec = {
        "value": round(value, 3), "unit": unit, "ms_per_step": round(ms, 5),
        "dtype": "bf16 (q, out, new K/V), fp8-e4m3 K/V cache" if b.kv_fp8 else "bf16",
        "config": cfg,
        "tokens_per_s": round(b.total_q / (ms * 1e-3), 1),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, p)), 5) for p in (10, 50, 90)],
        "work_per_step": work, "wall_s_timed_loop": round(wall, 4),
        "roofline": roof, "mfma": mfma, "cpu_baseline": cpu,
    }
    if sparse:
        cfg["union_density"] = b.extra["union_density"]
        cfg["compacted_kv_lens"] = [int(x) for x in b.extra["compacted_kv_lens"].reshape(-1)]
        cfg["mask"] = "column_shared" if name.endswith("colshared") else "per (head, Q-block)"
        rec["union_build_ms"] = round(float(prep_ms.mean()), 5)
    del attn, q, kn, vn, kc, vc
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_decode", choices=sorted(WORKLOAD_BOUND))
    ap.add_argument("--only", action="store_true",
                    help="measure the named workload alone (no extra workloads)")
    ap.add_argument("--flush", choices=("read", "write", "none"), default="read",
                    help="how the caches are flushed before each step (none: warm caches)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device copy 3 times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=("host", "graph"), default="host",
                    help="host: rpa_attention planned from host mirrors (the default); graph: "
                         "rpa_graph_attention (device-side plan + persistent kernel) captured "
                         "once in a HIP graph and replayed every step")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X and has no "
              "multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_ragged_paged_amd as rpa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel(), "launches": 3}))
        return
    rpa.load_library()
    with_cpu = not args.no_cpu_baseline
    ref = device_reference(dev)
    head = measure(args.workload, args, dev, with_cpu, 12.0)
    extras = {}
    if not args.only and args.workload == "llama3_decode":
        for name in EXTRA_WORKLOADS:
            extras[name] = measure(name, args, dev, with_cpu, 8.0)
    for rec in [head, *extras.values()]:
        roof = rec["roofline"]
        if roof["bound"] == "hbm":
            roof["frac_of_device_copy"] = round(roof["achieved"] / ref["copy_gbps"], 4)

    line = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"],
        "data": ("synthetic (seeded N(0,1) bf16 values, FP8 cache codes drawn per field, "
                 "Llama-3-8B attention shapes)" if "fp8" in head["dtype"] else
                 "synthetic (seeded N(0,1) bf16 values, Llama-3-8B attention shapes)"),
    }
    line.update({k: v for k, v in head.items() if k not in ("value", "unit", "ms_per_step", "dtype")})
    line["device_reference"] = ref
    if extras:
        line["workloads"] = extras
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
