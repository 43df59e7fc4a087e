"""GPU parity of the graph-capturable call (device-side planning, persistent attention kernel):
several batches of different composition run through the same fixed buffers, eagerly and as
replays of one captured HIP graph, against the CPU oracle.  Cache writes bit-exact,
attention within max-abs 2e-2."""
import numpy as np
import pytest
import torch

import attention_ragged_paged_amd as rpa
import oracle
from attention_ragged_paged_amd import workloads as wl
from tests.gpu_util import bf16_dev, compare, oracle_after_write, say, to_host_bits, to_host_f32

pytestmark = pytest.mark.gpu

B_MAX, T_MAX, HQ, HKV, D, S, POOL, MAX_PAGES = 8, 96, 16, 4, 128, 16, 160, 48


def _batch(q_lens, kv_lens, seed, layout=wl.SEQ_MAJOR):
    return wl.ragged_batch("g", q_lens, kv_lens, HQ, HKV, D, S, POOL, seed, layout=layout,
                           max_pages=MAX_PAGES)


class Buffers:
    """Fixed device buffers sized by the bounds; each batch is copied into them."""

    def __init__(self, b0):
        dev = torch.device("cuda")
        self.q = torch.zeros(T_MAX, HQ, D, dtype=torch.bfloat16, device=dev)
        self.k_new = torch.zeros(T_MAX, HKV, D, dtype=torch.bfloat16, device=dev)
        self.v_new = torch.zeros(T_MAX, HKV, D, dtype=torch.bfloat16, device=dev)
        self.k_cache = bf16_dev(b0.k_cache)
        self.v_cache = bf16_dev(b0.v_cache)
        tshape = (B_MAX,) + b0.block_tables.shape[1:]
        self.tables = torch.full(tshape, -1, dtype=torch.int32, device=dev)
        self.cu = torch.zeros(B_MAX + 1, dtype=torch.int32, device=dev)
        self.kvl = torch.zeros((B_MAX,) + b0.kv_lens.shape[1:], dtype=torch.int32, device=dev)
        self.out = torch.zeros(T_MAX, HQ, D, dtype=torch.bfloat16, device=dev)

    def load(self, b):
        """Copy batch b in (eager work between graph replays); pad to the bounds."""
        B, T = b.num_seqs, b.total_q
        assert B <= B_MAX and T <= T_MAX
        self.q.zero_()
        self.q[:T].copy_(bf16_dev(b.q))
        self.k_new[:T].copy_(bf16_dev(b.k_new))
        self.v_new[:T].copy_(bf16_dev(b.v_new))
        self.k_cache.copy_(bf16_dev(b.k_cache))
        self.v_cache.copy_(bf16_dev(b.v_cache))
        self.tables.fill_(-1)
        self.tables[:B].copy_(torch.from_numpy(b.block_tables))
        cu = np.full(B_MAX + 1, b.cu_q_lens[-1], dtype=np.int32)
        cu[:B + 1] = b.cu_q_lens
        self.cu.copy_(torch.from_numpy(cu))
        self.kvl.zero_()
        self.kvl[:B].copy_(torch.from_numpy(b.kv_lens))
        self.out.fill_(7.0)


def _check(buf, b, label):
    torch.cuda.synchronize()
    kc, vc = oracle_after_write(b)
    assert np.array_equal(to_host_bits(buf.k_cache), kc), f"{label}: K cache differs"
    assert np.array_equal(to_host_bits(buf.v_cache), vc), f"{label}: V cache differs"
    ref = oracle.attention(b.q, kc, vc, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale,
                           b.page_size, b.num_kv_heads, layout=b.layout)
    got = to_host_f32(buf.out)
    compare(got[:b.total_q], ref, label)
    assert np.all(got[b.total_q:] == 7.0), f"{label}: rows past the batch were written"


BATCHES = [
    ([1, 1, 1, 1, 1], [40, 300, 17, 500, 64]),          # decode only
    ([60, 1, 3, 1], [60, 700, 120, 33]),                 # mixed, one prefill chunk
    ([90], [610]),                                       # one chunked prefill
    ([0, 5, 0, 1, 7, 1, 2, 1], [0, 5, 9, 80, 400, 700, 15, 1]),  # empty sequences inside
]


def test_graph_attention_eager_matches_oracle():
    b0 = _batch(*BATCHES[0], seed=200)
    buf = Buffers(b0)
    ga = rpa.GraphAttention(buf.q, buf.k_cache, buf.v_cache, buf.tables, buf.cu, buf.kvl,
                            b0.scale, k_new=buf.k_new, v_new=buf.v_new, out=buf.out, max_splits=8)
    for i, (qs, kv) in enumerate(BATCHES):
        b = _batch(qs, kv, seed=200 + i)
        say(f"graph eager batch {i}: q={qs} kv={kv}")
        buf.load(b)
        ga()
        _check(buf, b, f"eager batch {i}")
        assert ga.status() == 0


def test_graph_head_major():
    qs, kv = [1, 33, 2], np.array([[50, 20, 90, 7], [40, 64, 33, 100], [2, 9, 130, 61]])
    b = _batch(qs, kv, seed=210, layout=wl.HEAD_MAJOR)
    buf = Buffers(b)
    ga = rpa.GraphAttention(buf.q, buf.k_cache, buf.v_cache, buf.tables, buf.cu, buf.kvl,
                            b.scale, k_new=buf.k_new, v_new=buf.v_new, out=buf.out, max_splits=4)
    say("graph head-major")
    buf.load(b)
    ga()
    _check(buf, b, "head-major")


def test_graph_capture_and_replay():
    """Capture one call, then replay it for batches of different composition, with eager
    copies and synchronisations between replays; every replay against the oracle and
    against an eager call on the same data."""
    b0 = _batch(*BATCHES[1], seed=220)
    buf = Buffers(b0)
    ga = rpa.GraphAttention(buf.q, buf.k_cache, buf.v_cache, buf.tables, buf.cu, buf.kvl,
                            b0.scale, k_new=buf.k_new, v_new=buf.v_new, out=buf.out, max_splits=8)
    buf.load(b0)
    ga()                      # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ga()
    torch.cuda.synchronize()
    for i, (qs, kv) in enumerate(BATCHES + BATCHES[::-1]):
        b = _batch(qs, kv, seed=230 + i)
        say(f"graph replay {i}: q={qs} kv={kv}")
        buf.load(b)
        torch.cuda.synchronize()
        graph.replay()
        _check(buf, b, f"replay {i}")
        replayed = buf.out.clone()
        buf.load(b)
        ga()                  # eager call on the same data
        torch.cuda.synchronize()
        assert torch.equal(buf.out, replayed), f"replay {i} differs from the eager call"


def test_graph_invalid_batch_is_skipped_and_flagged():
    b = _batch(*BATCHES[0], seed=240)
    buf = Buffers(b)
    ga = rpa.GraphAttention(buf.q, buf.k_cache, buf.v_cache, buf.tables, buf.cu, buf.kvl,
                            b.scale, k_new=buf.k_new, v_new=buf.v_new, out=buf.out, max_splits=8)
    buf.load(b)
    buf.kvl[2] = 0            # kv_len 0 < q_len 1: broken precondition
    say("graph invalid batch")
    ga()
    torch.cuda.synchronize()
    assert ga.status() != 0
    assert torch.all(buf.out == 7.0)
    buf.load(b)               # a valid batch afterwards runs normally
    ga()
    _check(buf, b, "after invalid")
    assert ga.status() == 0


def test_host_planned_call_refuses_capture():
    """rpa_attention fixes its plan and split-merge tag on the host; under graph capture it
    returns RPA_ERR_UNSUPPORTED and enqueues nothing, and it still runs eagerly afterwards."""
    say("rpa_attention under capture is refused")
    b = wl.ragged_batch("cap", [1, 1, 3], [900, 40, 300], HQ, HKV, D, S, POOL, 61)
    d_q, d_kc, d_vc = bf16_dev(b.q), bf16_dev(b.k_cache), bf16_dev(b.v_cache)
    d_kn, d_vn = bf16_dev(b.k_new), bf16_dev(b.v_new)
    tb = torch.from_numpy(b.block_tables).cuda()
    cu, kvl = torch.from_numpy(b.cu_q_lens).cuda(), torch.from_numpy(b.kv_lens).cuda()
    side = torch.cuda.Stream()   # the call enqueues on the stream current at construction
    with torch.cuda.stream(side):
        attn = rpa.PreparedAttention(d_q, d_kc, d_vc, tb, cu, kvl, b.scale, k_new=d_kn,
                                     v_new=d_vn, cu_q_lens_host=torch.from_numpy(b.cu_q_lens),
                                     kv_lens_host=torch.from_numpy(b.kv_lens))
    attn.out.fill_(3.0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    raised = None
    with torch.cuda.graph(graph, stream=side):
        try:
            attn()
        except rpa.RpaError as e:
            raised = e
    torch.cuda.synchronize()
    assert raised is not None and raised.status == 2, raised
    assert "rpa_graph_attention" in str(raised)
    assert bool((attn.out.float() == 3.0).all()), "a refused call must enqueue nothing"
    out = attn()
    torch.cuda.synchronize()
    kc, vc = oracle_after_write(b)
    ref = oracle.attention(b.q, kc, vc, b.block_tables, b.cu_q_lens, b.kv_lens, b.scale, S, HKV)
    compare(to_host_f32(out), ref, "eager call after a refused capture")
