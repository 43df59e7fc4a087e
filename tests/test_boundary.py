"""The C-ABI boundary without a GPU: the library loads, exports every entry point the header
declares, validates arguments with specific errors, and classifies batches (host logic only;
no compute call reaches a device here)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import attention_ragged_paged_amd as rpa
from attention_ragged_paged_amd import _rpa
from attention_ragged_paged_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rpa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_rpa.library_path()):
        from attention_ragged_paged_amd import build
        build.build()
    return _rpa.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rpa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(_rpa.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # exported with C linkage (no mangling), visible to dlsym
    for name in _declared_functions():
        ctypes.cast(getattr(lib, name), ctypes.c_void_p)


def test_library_has_no_oracle_dependency(lib):
    # the product path must never reach the CPU oracle
    import subprocess
    deps = subprocess.run(["ldd", _rpa.library_path()], capture_output=True, text=True).stdout
    assert "oracle" not in deps
    syms = subprocess.run(["nm", "-D", _rpa.library_path()], capture_output=True, text=True).stdout
    assert "oracle_" not in syms


def _shape(cu, kv, Hq=4, Hkv=2, D=64, S=16, P=16, max_pages=4, layout=0, kernel=0, kv_dtype=0,
           k_scale=1.0, v_scale=1.0):
    cu = np.ascontiguousarray(cu, np.int32)
    kv = np.ascontiguousarray(kv, np.int32)
    s = _rpa.RpaShape(len(cu) - 1, int(cu[-1]), Hq, Hkv, D, S, P, max_pages, layout, kernel,
                      cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                      kv.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), kv_dtype, k_scale, v_scale)
    s._keep = (cu, kv)
    return s


def _attn(lib, s, scale=0.125, k_new=None, ws=None, ws_bytes=0, ptr=16):
    p = ctypes.c_void_p(ptr)
    return lib.rpa_attention(ctypes.byref(s), p, p, p, p, p, p, scale, k_new, k_new, p, ws,
                             ws_bytes, None)


@pytest.mark.parametrize("kw,frag", [
    (dict(cu=[1, 2], kv=[4]), "cu_q_lens[0]"),
    (dict(cu=[0, 3, 2], kv=[4, 4]), "decreases"),
    (dict(cu=[0, 5], kv=[4]), "kv_len 4 < q_len 5"),
    (dict(cu=[0, 1], kv=[65], max_pages=4), "needs 5 pages"),
    (dict(cu=[0, 1], kv=[4], Hq=3, Hkv=2), "not a multiple"),
    (dict(cu=[0, 1], kv=[4], S=24), "power of two"),
    (dict(cu=[0, 1], kv=[4], S=8), "power of two"),
    (dict(cu=[0, 1], kv=[4], S=2048), "[16, 1024]"),
    (dict(cu=[0, 1], kv=[4], layout=5), "layout"),
    (dict(cu=[0, 1], kv=[4], kernel=9), "kernel"),
    (dict(cu=[0, 1], kv=[4], kv_dtype=3), "kv_dtype"),
    (dict(cu=[0, 1], kv=[4], kv_dtype=1, k_scale=-1.0), "scale"),
    (dict(cu=[0, 1], kv=[4], kv_dtype=1, v_scale=float("nan")), "scale"),
])
def test_invalid_arguments(lib, kw, frag):
    s = _shape(**kw)
    assert _attn(lib, s) == 1
    assert frag in lib.rpa_last_error().decode()
    assert lib.rpa_select_kernel(ctypes.byref(s)) == -1
    assert lib.rpa_attention_workspace_size(ctypes.byref(s)) == ctypes.c_size_t(-1).value


def test_unsupported_head_dim_and_group(lib):
    assert _attn(lib, _shape([0, 1], [4], D=96)) == 2
    assert "head_dim 96" in lib.rpa_last_error().decode()
    assert _attn(lib, _shape([0, 1], [4], Hq=256, Hkv=1)) == 2


def test_bad_scale_and_pointer_checks(lib):
    s = _shape([0, 1], [4])
    assert _attn(lib, s, scale=0.0) == 1 and "scale" in lib.rpa_last_error().decode()
    assert _attn(lib, s, scale=float("nan")) == 1
    assert _attn(lib, s, ptr=0) == 1 and "NULL" in lib.rpa_last_error().decode()
    p = ctypes.c_void_p(16)
    assert lib.rpa_attention(ctypes.byref(s), p, p, p, p, p, p, 0.125, p, None, p, None, 0,
                             None) == 1
    assert "both" in lib.rpa_last_error().decode()


def test_bf16_cache_ignores_scales(lib):
    """The scales are read only for FP8 caches."""
    s = _shape([0, 0, 0], [5, 9], k_scale=0.0, v_scale=float("nan"))
    assert _attn(lib, s, ptr=0) == 0


def test_empty_batch_is_ok_without_device(lib):
    s = _shape([0, 0, 0], [5, 9])
    assert _attn(lib, s, ptr=0) == 0
    assert lib.rpa_last_error().decode() == ""
    p = ctypes.c_void_p(0)
    assert lib.rpa_write_kv(ctypes.byref(s), p, p, p, p, p, p, p, None) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
def test_no_gpu_is_an_error_not_a_fallback(lib):
    s = _shape([0, 1], [4])
    ws = lib.rpa_attention_workspace_size(ctypes.byref(s))
    st = _attn(lib, s, ws=ctypes.c_void_p(16), ws_bytes=ws)
    assert st in (2, 4), st
    assert lib.rpa_last_error().decode() != ""


def _select(lib, b):
    s = _shape(b.cu_q_lens, b.kv_lens.reshape(-1), Hq=b.num_q_heads, Hkv=b.num_kv_heads,
               D=b.head_dim, S=b.page_size, P=b.num_pages, max_pages=b.max_pages, layout=b.layout)
    return lib.rpa_select_kernel(ctypes.byref(s)), lib.rpa_attention_workspace_size(ctypes.byref(s))


def test_dispatch_is_a_function_of_batch_composition(lib):
    # tiny ragged (q_lens 1,1,7 with G=2: at most 14 rows per sequence) -> decode-only
    assert _select(lib, wl.tiny_ragged())[0] == rpa.KERNEL_DECODE
    # 4 x 2048-token prefill -> prefill-only, no split, no workspace
    k, ws = _select(lib, wl.llama3_prefill(num_seqs=1, seq_len=256))
    assert k == rpa.KERNEL_PREFILL
    # chunk + decodes -> mixed
    b = wl.ragged_batch("m", [300, 1, 1], [900, 50, 70], 32, 8, 128, 16, 200, 1)
    assert _select(lib, b)[0] == rpa.KERNEL_MIXED
    # forcing a kernel is honoured
    s = _shape([0, 1, 2], [17, 40], kernel=rpa.KERNEL_PREFILL)
    assert lib.rpa_select_kernel(ctypes.byref(s)) == rpa.KERNEL_PREFILL


def test_decode_workspace_covers_split_partials(lib):
    # one long decode sequence must be split across workgroups -> partials need workspace
    s = _shape([0, 1], [65536], Hq=32, Hkv=8, D=128, S=16, P=5000, max_pages=4096)
    ws = lib.rpa_attention_workspace_size(ctypes.byref(s))
    assert ws > 0 and ws % 4 == 0
    assert _attn(lib, s, ws=ctypes.c_void_p(16), ws_bytes=ws - 4) == 3
    assert "workspace" in lib.rpa_last_error().decode()


def test_union_builder_validation(lib):
    p = ctypes.c_void_p(16)
    assert lib.rpa_build_union_tables(p, 32, 8, 64, 2048, p, 126976, 131072, 64, p, p, p, None) in (2, 4) \
        or not torch.cuda.is_available()
    assert lib.rpa_build_union_tables(p, 32, 6, 64, 2048, p, 0, 10, 64, p, p, p, None) == 1
    assert lib.rpa_build_union_tables(p, 32, 8, 64, 2048, p, 10, 10, 64, p, p, p, None) == 1
    assert lib.rpa_build_union_tables(p, 32, 8, 64, 16, p, 0, 2000, 64, p, p, p, None) == 1
    assert lib.rpa_build_union_tables(p, 32, 8, 64, 40000, p, 0, 2000, 64, p, p, p, None) == 2


def _gshape(**kw):
    f = dict(max_seqs=4, max_tokens=32, max_splits=8, num_q_heads=8, num_kv_heads=2, head_dim=128,
             page_size=16, num_pages=64, max_pages_per_seq=16, layout=0, kv_dtype=0, k_scale=1.0,
             v_scale=1.0)
    f.update(kw)
    return _rpa.RpaGraphShape(*[f[n] for n, _ in _rpa.RpaGraphShape._fields_])


@pytest.mark.parametrize("kw,frag", [
    (dict(max_seqs=0), "max_seqs"),
    (dict(max_tokens=0), "max_tokens"),
    (dict(max_splits=0), "max_splits"),
    (dict(max_splits=65), "max_splits"),
    (dict(num_q_heads=6, num_kv_heads=4), "multiple"),
    (dict(page_size=24), "page_size"),
    (dict(page_size=2048), "page_size"),
    (dict(layout=3), "layout"),
    (dict(kv_dtype=2), "kv_dtype"),
    (dict(kv_dtype=1, k_scale=0.0), "scale"),
    (dict(kv_dtype=1, v_scale=float("inf")), "scale"),
    (dict(kv_dtype=1, k_scale=1e-39), "scale"),
])
def test_graph_shape_validation(lib, kw, frag):
    s = _gshape(**kw)
    assert lib.rpa_graph_workspace_size(ctypes.byref(s)) == ctypes.c_size_t(-1).value
    p = ctypes.c_void_p(16)
    st = lib.rpa_graph_attention(ctypes.byref(s), p, p, p, p, p, p, 0.1, None, None, p, p, 1 << 30,
                                 None)
    assert st == 1 and frag in lib.rpa_last_error().decode()


def test_graph_workspace_and_argument_checks(lib):
    s = _gshape()
    ws = lib.rpa_graph_workspace_size(ctypes.byref(s))
    # plan + arguments + 8 splits of fp32 partials for 32 tokens x 8 heads x 128 dims + counters
    assert ws >= 8 * 32 * 8 * 128 * 4 and ws % 256 == 0
    s1 = _gshape(max_splits=1)   # no splits: no partials, no counters
    assert lib.rpa_graph_workspace_size(ctypes.byref(s1)) < 4096
    p = ctypes.c_void_p(16)
    assert lib.rpa_graph_attention(ctypes.byref(s), p, p, p, p, p, p, float("inf"), None, None, p,
                                   p, ws, None) == 1
    assert lib.rpa_graph_attention(ctypes.byref(s), p, p, p, p, p, p, 0.1, p, None, p, p, ws,
                                   None) == 1
    assert "both" in lib.rpa_last_error().decode()
    assert lib.rpa_graph_attention(ctypes.byref(s), p, p, p, p, p, p, 0.1, None, None, p, None, ws,
                                   None) == 1
    assert lib.rpa_graph_attention(ctypes.byref(s), p, p, p, p, p, p, 0.1, None, None, p, p, ws - 1,
                                   None) == 3


def _rot(lib, s, rd=64, max_pos=64, qs=None, ks=None, tables=16, q=32, q_out=4096):
    p = ctypes.c_void_p(16)
    r = _rpa.RpaRotary(tables, tables, max_pos, rd, 0)
    Hq, Hkv, D = s.num_q_heads, s.num_kv_heads, s.head_dim
    return lib.rpa_rotary_write_kv(ctypes.byref(s), ctypes.c_void_p(q), p, p,
                                   Hq * D if qs is None else qs, Hkv * D if ks is None else ks,
                                   ctypes.byref(r), ctypes.c_void_p(q_out), p, p, p, p, p, None)


@pytest.mark.parametrize("kw,frag", [
    (dict(rd=24), "rotary_dim"),
    (dict(rd=80), "rotary_dim"),
    (dict(qs=100), "row strides"),
    (dict(ks=64), "row strides"),
    (dict(tables=0), "tables"),
    (dict(max_pos=20), "max_position"),
    (dict(q=32, q_out=48), "overlaps"),
    (dict(q=40), "aligned"),
])
def test_rotary_argument_checks(lib, kw, frag):
    s = _shape([0, 1, 3], [4, 30], D=64)
    assert _rot(lib, s, **kw) == 1
    assert frag in lib.rpa_last_error().decode()


def test_rotary_head_major_needs_one_position_per_token(lib):
    s = _shape([0, 1], [[4, 5]], layout=1)
    assert _rot(lib, s) == 1 and "different kv_lens" in lib.rpa_last_error().decode()
