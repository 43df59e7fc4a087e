"""ctypes binding of librpa.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module turns PyTorch
tensors into the raw pointers, sizes and host mirrors the C ABI (include/rpa.h) takes,
passes torch's current HIP stream, and raises on a non-OK status.
"""
from __future__ import annotations

import ctypes
import os

import torch

LAYOUT_SEQ_MAJOR = 0
LAYOUT_HEAD_MAJOR = 1
KERNEL_AUTO = 0
KERNEL_DECODE = 1
KERNEL_PREFILL = 2
KERNEL_MIXED = 3
KV_BF16 = 0
KV_FP8_E4M3 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librpa.so")

_STATUS = {0: "RPA_OK", 1: "RPA_ERR_INVALID_ARGUMENT", 2: "RPA_ERR_UNSUPPORTED",
           3: "RPA_ERR_WORKSPACE_TOO_SMALL", 4: "RPA_ERR_HIP"}

EXPORTED = ("rpa_write_kv", "rpa_attention_workspace_size", "rpa_select_kernel", "rpa_attention",
            "rpa_attention_noalloc",
            "rpa_graph_workspace_size", "rpa_graph_attention", "rpa_build_union_tables",
            "rpa_rotary_write_kv", "rpa_last_error")


class RpaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class RpaShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
        ("h_cu_q_lens", ctypes.POINTER(ctypes.c_int32)),
        ("h_kv_lens", ctypes.POINTER(ctypes.c_int32)),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class RpaGraphShape(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "max_seqs", "max_tokens", "max_splits", "num_q_heads", "num_kv_heads", "head_dim",
        "page_size", "num_pages", "max_pages_per_seq", "layout", "kv_dtype")] + [
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load librpa.so (built in-tree by attention_ragged_paged_amd.build); no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m attention_ragged_paged_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    shp = ctypes.POINTER(RpaShape)
    lib.rpa_write_kv.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.rpa_write_kv.restype = ctypes.c_int
    lib.rpa_rotary_write_kv.argtypes = [shp, vp, vp, vp, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.POINTER(RpaRotary), vp, vp, vp, vp, vp, vp, vp]
    lib.rpa_rotary_write_kv.restype = ctypes.c_int
    lib.rpa_attention_workspace_size.argtypes = [shp]
    lib.rpa_attention_workspace_size.restype = sz
    lib.rpa_select_kernel.argtypes = [shp]
    lib.rpa_select_kernel.restype = i32
    lib.rpa_attention.argtypes = [shp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    lib.rpa_attention.restype = ctypes.c_int
    lib.rpa_attention_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                          vp, vp]
    lib.rpa_attention_noalloc.restype = ctypes.c_int
    gshp = ctypes.POINTER(RpaGraphShape)
    lib.rpa_graph_workspace_size.argtypes = [gshp]
    lib.rpa_graph_workspace_size.restype = sz
    lib.rpa_graph_attention.argtypes = [gshp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                        vp, sz, vp]
    lib.rpa_graph_attention.restype = ctypes.c_int
    lib.rpa_build_union_tables.argtypes = [vp, i32, i32, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.rpa_build_union_tables.restype = ctypes.c_int
    lib.rpa_last_error.argtypes = []
    lib.rpa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise RpaError(status, load_library().rpa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _host_i32(t):
    h = t.detach().to("cpu", torch.int32).contiguous()
    return h, h.data_ptr()


def _need_contig(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def kv_dtype_of(k_cache, v_cache=None):
    """KV_BF16 for bfloat16 caches, KV_FP8_E4M3 for caches of E4M3 codes (uint8 or
    torch.float8_e4m3fn storage)."""
    def one(t):
        if t.dtype == torch.bfloat16:
            return KV_BF16
        if t.dtype in (torch.uint8, torch.float8_e4m3fn):
            return KV_FP8_E4M3
        raise ValueError(f"cache dtype {t.dtype}: expected bfloat16, uint8 or float8_e4m3fn")
    d = one(k_cache)
    if v_cache is not None and one(v_cache) != d:
        raise ValueError("k_cache and v_cache must have the same element type")
    return d


class RpaRotary(ctypes.Structure):
    _fields_ = [("cos_cache", ctypes.c_void_p), ("sin_cache", ctypes.c_void_p),
                ("max_position", ctypes.c_int32), ("rotary_dim", ctypes.c_int32),
                ("interleaved", ctypes.c_int32)]


class _Shape:
    """An RpaShape plus the host tensors it points into (kept alive with it)."""

    def __init__(self, *, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                 max_pages, layout, cu_q_lens_host, kv_lens_host, kernel=KERNEL_AUTO,
                 kv_dtype=KV_BF16, k_scale=1.0, v_scale=1.0):
        self.cu, cu_p = _host_i32(cu_q_lens_host)
        self.kv, kv_p = _host_i32(kv_lens_host)
        B = self.cu.numel() - 1
        self.c = RpaShape(B, int(self.cu[-1]) if B >= 0 else 0, num_q_heads, num_kv_heads, head_dim,
                          page_size, num_pages, max_pages, layout, kernel,
                          ctypes.cast(cu_p, ctypes.POINTER(ctypes.c_int32)),
                          ctypes.cast(kv_p, ctypes.POINTER(ctypes.c_int32)),
                          kv_dtype, float(k_scale), float(v_scale))

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _cache_geometry(k_cache, block_tables):
    if k_cache.dim() == 4:   # [P, S, Hkv, D]
        return LAYOUT_SEQ_MAJOR, k_cache.shape[2], k_cache.shape[1], k_cache.shape[3]
    if k_cache.dim() == 3:   # [P, S, D], tables [B, Hkv, max_pages]
        return LAYOUT_HEAD_MAJOR, block_tables.shape[1], k_cache.shape[1], k_cache.shape[2]
    raise ValueError("k_cache must be [P, S, Hkv, D] (sequence-major) or [P, S, D] (KV-head-major)")


def _shape_for(q_heads, k_cache, block_tables, cu_q_lens, kv_lens, cu_q_lens_host, kv_lens_host,
               kernel, k_scale=1.0, v_scale=1.0, v_cache=None):
    layout, Hkv, S, D = _cache_geometry(k_cache, block_tables)
    return _Shape(num_q_heads=q_heads, num_kv_heads=Hkv, head_dim=D, page_size=S,
                  num_pages=k_cache.shape[0], max_pages=block_tables.shape[-1], layout=layout,
                  cu_q_lens_host=cu_q_lens if cu_q_lens_host is None else cu_q_lens_host,
                  kv_lens_host=kv_lens if kv_lens_host is None else kv_lens_host, kernel=kernel,
                  kv_dtype=kv_dtype_of(k_cache, v_cache), k_scale=k_scale, v_scale=v_scale)


def write_kv(k_new, v_new, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, *,
             cu_q_lens_host=None, kv_lens_host=None, k_scale=1.0, v_scale=1.0):
    """Scatter k_new / v_new ([T, Hkv, D] bf16) into the paged caches in place (rpa_write_kv).
    FP8 caches (uint8 / float8_e4m3fn) store codes with the given scales."""
    lib = load_library()
    _need_contig(k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                 block_tables=block_tables, cu_q_lens=cu_q_lens, kv_lens=kv_lens)
    shape = _shape_for(k_new.shape[1] if k_new.dim() == 3 else 1, k_cache, block_tables, cu_q_lens,
                       kv_lens, cu_q_lens_host, kv_lens_host, KERNEL_AUTO, k_scale, v_scale,
                       v_cache)
    _check(lib.rpa_write_kv(shape.ref, _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                            _ptr(block_tables), _ptr(cu_q_lens), _ptr(kv_lens),
                            _stream(k_cache.device)))


def _row_view(t, heads, name):
    """(pointer, row stride in elements) of a [T, heads, D] view whose rows may be strided
    (a slice of packed QKV); dims and heads must be dense within a row."""
    if t.dim() != 3 or t.shape[1] != heads or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [T, {heads}, D] with dense heads and dims")
    return ctypes.c_void_p(t.data_ptr()), t.stride(0)


def split_packed_qkv(qkv, num_q_heads, num_kv_heads):
    """Views q [T, Hq, D], k and v [T, Hkv, D] of packed QKV [T, (Hq + 2 Hkv) * D] (no copy)."""
    T = qkv.shape[0]
    x = qkv.reshape(T, num_q_heads + 2 * num_kv_heads, -1)
    return (x[:, :num_q_heads], x[:, num_q_heads:num_q_heads + num_kv_heads],
            x[:, num_q_heads + num_kv_heads:])


def rotary_write_kv(q, k, v, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, *,
                    cos_cache=None, sin_cache=None, rotary_dim=0, interleaved=False, q_out=None,
                    cu_q_lens_host=None, kv_lens_host=None, k_scale=1.0, v_scale=1.0):
    """Rotate the new rows of Q and K, write the rotated Q to q_out and scatter K and V into
    the caches (rpa_rotary_write_kv).  q [T, Hq, D], k and v [T, Hkv, D] bf16, which may be
    strided row views of packed QKV (see split_packed_qkv); cos_cache, sin_cache fp32
    [max_position, rotary_dim / 2].  Returns q_out."""
    lib = load_library()
    Hq, Hkv = q.shape[1], k.shape[1]
    qp, qs = _row_view(q, Hq, "q")
    kp, ks = _row_view(k, Hkv, "k")
    vp_, vs = _row_view(v, Hkv, "v")
    if ks != vs:
        raise ValueError("k and v must share one row stride")
    _need_contig(k_cache=k_cache, v_cache=v_cache, block_tables=block_tables, cu_q_lens=cu_q_lens,
                 kv_lens=kv_lens, q_out=q_out, cos_cache=cos_cache, sin_cache=sin_cache)
    shape = _shape_for(Hq, k_cache, block_tables, cu_q_lens, kv_lens, cu_q_lens_host, kv_lens_host,
                       KERNEL_AUTO, k_scale, v_scale, v_cache)
    if q_out is None:
        q_out = torch.empty((q.shape[0], Hq, q.shape[2]), dtype=q.dtype, device=q.device)
    rot = None
    if rotary_dim:
        rot = RpaRotary(cos_cache.data_ptr(), sin_cache.data_ptr(), cos_cache.shape[0],
                        int(rotary_dim), int(bool(interleaved)))
    _check(lib.rpa_rotary_write_kv(shape.ref, qp, kp, vp_, qs, ks,
                                   None if rot is None else ctypes.byref(rot), _ptr(q_out),
                                   _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                   _ptr(cu_q_lens), _ptr(kv_lens), _stream(q.device)))
    return q_out


def workspace_size(q, k_cache, block_tables, cu_q_lens_host, kv_lens_host, kernel=KERNEL_AUTO,
                   k_scale=1.0, v_scale=1.0):
    lib = load_library()
    shape = _shape_for(q.shape[1], k_cache, block_tables, None, None, cu_q_lens_host, kv_lens_host,
                       kernel, k_scale, v_scale)
    n = lib.rpa_attention_workspace_size(shape.ref)
    if n == ctypes.c_size_t(-1).value:
        _check(1)
    return int(n)


def select_kernel(q, k_cache, block_tables, cu_q_lens_host, kv_lens_host, kernel=KERNEL_AUTO,
                  k_scale=1.0, v_scale=1.0):
    lib = load_library()
    shape = _shape_for(q.shape[1], k_cache, block_tables, None, None, cu_q_lens_host, kv_lens_host,
                       kernel, k_scale, v_scale)
    k = lib.rpa_select_kernel(shape.ref)
    if k < 0:
        _check(1)
    return int(k)


def attention(q, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, scale, *, k_new=None,
              v_new=None, out=None, workspace=None, cu_q_lens_host=None, kv_lens_host=None,
              kernel=KERNEL_AUTO, k_scale=1.0, v_scale=1.0):
    """Ragged paged causal GQA attention (rpa_attention); returns out [T, Hq, D] bf16.

    cu_q_lens_host / kv_lens_host: CPU int32 mirrors of the device metadata; when omitted
    they are copied from the device (a synchronising copy).  FP8 caches (uint8 or
    float8_e4m3fn storage of E4M3 codes) take their scales k_scale, v_scale.
    """
    lib = load_library()
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 cu_q_lens=cu_q_lens, kv_lens=kv_lens, k_new=k_new, v_new=v_new, out=out)
    shape = _shape_for(q.shape[1], k_cache, block_tables, cu_q_lens, kv_lens, cu_q_lens_host,
                       kv_lens_host, kernel, k_scale, v_scale, v_cache)
    if out is None:
        out = torch.empty_like(q)
    need = lib.rpa_attention_workspace_size(shape.ref)
    if need == ctypes.c_size_t(-1).value:
        _check(1)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.rpa_attention(shape.ref, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                             _ptr(cu_q_lens), _ptr(kv_lens), float(scale), _ptr(k_new),
                             _ptr(v_new), _ptr(out), _ptr(workspace), ws_bytes,
                             _stream(q.device)))
    return out


# Bytes of the library's static scratch (RPA_NOALLOC_SCRATCH_BYTES in include/rpa.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def attention_noalloc(q, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, scale, *, out,
                      k_new=None, v_new=None, cu_q_lens_host=None, kv_lens_host=None,
                      kernel=KERNEL_AUTO, k_scale=1.0, v_scale=1.0):
    """rpa_attention_noalloc: attention whose split partials live in the library's static
    device scratch (no workspace); writes into the caller's ``out`` and returns it.  Calls
    that overlap in time on one GPU race on that scratch."""
    lib = load_library()
    _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                 cu_q_lens=cu_q_lens, kv_lens=kv_lens, k_new=k_new, v_new=v_new, out=out)
    shape = _shape_for(q.shape[1], k_cache, block_tables, cu_q_lens, kv_lens, cu_q_lens_host,
                       kv_lens_host, kernel, k_scale, v_scale, v_cache)
    _check(lib.rpa_attention_noalloc(shape.ref, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(block_tables), _ptr(cu_q_lens), _ptr(kv_lens),
                                     float(scale), _ptr(k_new), _ptr(v_new), _ptr(out),
                                     _stream(q.device)))
    return out


def build_union_tables(mask, base_tables, past, kv_len, page_size, *, out_tables=None,
                       out_counts=None, out_kv_lens=None):
    """Per-KV-head block tables of one chunk (rpa_build_union_tables).

    mask: uint8 [Hq, nQB, nKB] (device); base_tables: int32 [Hkv, nKB] (device).
    Returns (tables [Hkv, nKB], counts [Hkv], kv_lens [Hkv]), all int32 on the device.
    """
    lib = load_library()
    _need_contig(mask=mask, base_tables=base_tables)
    Hq, nQB, nKB = mask.shape
    Hkv = base_tables.shape[0]
    dev = mask.device
    if out_tables is None:
        out_tables = torch.empty((Hkv, nKB), dtype=torch.int32, device=dev)
    if out_counts is None:
        out_counts = torch.empty(Hkv, dtype=torch.int32, device=dev)
    if out_kv_lens is None:
        out_kv_lens = torch.empty(Hkv, dtype=torch.int32, device=dev)
    _check(lib.rpa_build_union_tables(_ptr(mask), Hq, Hkv, nQB, nKB, _ptr(base_tables), int(past),
                                      int(kv_len), int(page_size), _ptr(out_tables),
                                      _ptr(out_counts), _ptr(out_kv_lens), _stream(dev)))
    return out_tables, out_counts, out_kv_lens


class PreparedAttention:
    """rpa_attention with every argument marshalled once; calling it only enqueues the work.

    For tight loops (benchmarks, serving steps) where the batch metadata does not change.
    The tensors passed here must stay alive and keep their shapes while the object is used.
    Not for HIP graph capture: a call on a capturing stream raises RpaError
    (RPA_ERR_UNSUPPORTED) and enqueues nothing; GraphAttention is the capturable form.
    """

    def __init__(self, q, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, scale, *,
                 k_new=None, v_new=None, out=None, cu_q_lens_host=None, kv_lens_host=None,
                 kernel=KERNEL_AUTO, workspace=None, k_scale=1.0, v_scale=1.0):
        self.lib = load_library()
        _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                     cu_q_lens=cu_q_lens, kv_lens=kv_lens, k_new=k_new, v_new=v_new, out=out)
        self.shape = _shape_for(q.shape[1], k_cache, block_tables, cu_q_lens, kv_lens,
                                cu_q_lens_host, kv_lens_host, kernel, k_scale, v_scale, v_cache)
        self.out = torch.empty_like(q) if out is None else out
        need = self.lib.rpa_attention_workspace_size(self.shape.ref)
        if need == ctypes.c_size_t(-1).value:
            _check(1)
        if workspace is None and need > 0:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
        self.workspace = workspace
        self.keep = (q, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, k_new, v_new)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self.args = (self.shape.ref, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                     _ptr(cu_q_lens), _ptr(kv_lens), ctypes.c_float(scale), _ptr(k_new),
                     _ptr(v_new), _ptr(self.out), _ptr(workspace), ctypes.c_size_t(ws_bytes),
                     _stream(q.device))

    def __call__(self):
        _check(self.lib.rpa_attention(*self.args))
        return self.out


class PreparedWriteKV:
    """rpa_write_kv with its arguments marshalled once (see PreparedAttention)."""

    def __init__(self, k_new, v_new, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, *,
                 cu_q_lens_host=None, kv_lens_host=None, k_scale=1.0, v_scale=1.0):
        self.lib = load_library()
        self.shape = _shape_for(k_new.shape[1], k_cache, block_tables, cu_q_lens, kv_lens,
                                cu_q_lens_host, kv_lens_host, KERNEL_AUTO, k_scale, v_scale,
                                v_cache)
        self.keep = (k_new, v_new, k_cache, v_cache, block_tables, cu_q_lens, kv_lens)
        self.args = (self.shape.ref, _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                     _ptr(block_tables), _ptr(cu_q_lens), _ptr(kv_lens), _stream(k_cache.device))

    def __call__(self):
        _check(self.lib.rpa_write_kv(*self.args))


class GraphAttention:
    """rpa_graph_attention over fixed buffers: a call reads no host data, so it can be captured
    in a HIP graph (torch.cuda.graph) and replayed after the buffers' device contents change.

    The buffers fix the bounds: q and out have max_tokens rows, cu_q_lens has max_seqs + 1
    entries (sequences past the live batch repeat the last offset and have kv_len 0), kv_lens
    and block_tables max_seqs rows.  The workspace (state that persists from call to call) is
    allocated zeroed here.  Every call enqueues on the current stream at call time.
    """

    def __init__(self, q, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, scale, *,
                 k_new=None, v_new=None, out=None, max_splits=16, k_scale=1.0, v_scale=1.0):
        self.lib = load_library()
        _need_contig(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                     cu_q_lens=cu_q_lens, kv_lens=kv_lens, k_new=k_new, v_new=v_new, out=out)
        layout, Hkv, S, D = _cache_geometry(k_cache, block_tables)
        self.shape = RpaGraphShape(cu_q_lens.numel() - 1, q.shape[0], max_splits, q.shape[1], Hkv,
                                   D, S, k_cache.shape[0], block_tables.shape[-1], layout,
                                   kv_dtype_of(k_cache, v_cache), float(k_scale), float(v_scale))
        need = self.lib.rpa_graph_workspace_size(ctypes.byref(self.shape))
        if need == ctypes.c_size_t(-1).value:
            _check(1)
        self.workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
        self.out = torch.empty_like(q) if out is None else out
        self.device = q.device
        self.keep = (q, k_cache, v_cache, block_tables, cu_q_lens, kv_lens, k_new, v_new)
        self.args = (ctypes.byref(self.shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                     _ptr(block_tables), _ptr(cu_q_lens), _ptr(kv_lens), ctypes.c_float(scale),
                     _ptr(k_new), _ptr(v_new), _ptr(self.out), _ptr(self.workspace),
                     ctypes.c_size_t(need))

    def __call__(self):
        _check(self.lib.rpa_graph_attention(*self.args, _stream(self.device)))
        return self.out

    def status(self) -> int:
        """The planning kernel's status word of the last call (0: the batch was valid)."""
        return int(self.workspace[:4].view(torch.int32).item())
