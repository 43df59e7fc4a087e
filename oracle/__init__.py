"""CPU oracle for ragged paged attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library and its Python binding
never import it; the two share no code.

The arithmetic lives in ``rpa_oracle.c`` (plain C, scalar loops, fp64); this
module only builds it with gcc and marshals numpy arrays through ctypes.
Values are bfloat16 bit patterns carried as ``numpy.uint16``.

Functions (each cites the passage it follows in ``rpa_oracle.c``):
  write_kv        scatter of new K/V rows into their page slots
  attention       page gather + softmax attention, fp64, all rows or sampled rows
  union_tables    Q-block union -> intra-group union -> ascending compaction
  rotary_qkv      rotary embedding of new Q/K (packed or separate Q, K, V), then the scatter
  fp8_encode, fp8_decode
                  FP8 E4M3 (OCP) codes of a quantized cache; write_kv and attention
                  take uint8 caches with per-tensor k_scale / v_scale as FP8 caches
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rpa_oracle.c")
_LIB = os.path.join(_HERE, "librpa_oracle.so")

SEQ_MAJOR = 0
HEAD_MAJOR = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP over query rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_write_kv.argtypes = [i, p, p, i, i, i, i, i, i, p, p, p, p, p]
        lib.oracle_write_kv.restype = i
        lib.oracle_attention.argtypes = [i, p, p, i, i, i, i, i, i, i, p, p, p, p,
                                         ctypes.c_double, p, ctypes.c_int64, p, p, i]
        lib.oracle_attention.restype = i
        lib.oracle_union_tables.argtypes = [p, i, i, i, i, p, i, i, i, p, p, p, p]
        lib.oracle_union_tables.restype = i
        lib.oracle_write_kv_fp8.argtypes = [i, p, p, i, i, i, i, i, i, p, p, p, p, p,
                                            ctypes.c_float, ctypes.c_float]
        lib.oracle_write_kv_fp8.restype = i
        lib.oracle_attention_fp8.argtypes = [i, p, p, i, i, i, i, i, i, i, p, p, p, p,
                                             ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                             p, ctypes.c_int64, p, p, i]
        lib.oracle_attention_fp8.restype = i
        lib.oracle_fp8_encode.argtypes = [p, p, ctypes.c_int64]
        lib.oracle_fp8_encode.restype = i
        lib.oracle_fp8_decode.argtypes = [p, p, ctypes.c_int64]
        lib.oracle_fp8_decode.restype = i
        lib.oracle_rotary_qkv.argtypes = [i, p, p, i, i, i, i, i, i, i, p, p, p, p,
                                          ctypes.c_int64, ctypes.c_int64, p, p, i, i, i, p, p, p,
                                          i, ctypes.c_float, ctypes.c_float]
        lib.oracle_rotary_qkv.restype = i
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return _load().oracle_num_threads()


def fp8_encode(y):
    """FP8 E4M3 codes (uint8) of float32 values: clamp to +-448, round to nearest even."""
    lib = _load()
    yy = _c(y, np.float32)
    out = np.zeros(yy.shape, dtype=np.uint8)
    lib.oracle_fp8_encode(_ptr(yy), _ptr(out), yy.size)
    return out


def fp8_decode(codes):
    """Values (float64) of FP8 E4M3 codes; the two NaN codes give NaN."""
    lib = _load()
    cc = _c(codes, np.uint8)
    out = np.zeros(cc.shape, dtype=np.float64)
    lib.oracle_fp8_decode(_ptr(cc), _ptr(out), cc.size)
    return out


def write_kv(cu_q_lens, kv_lens, tables, k_new, v_new, k_cache, v_cache, page_size,
             layout=SEQ_MAJOR, k_scale=1.0, v_scale=1.0):
    """Return (k_cache', v_cache'): copies of the caches with the new rows scattered in.

    uint8 caches are FP8 caches with scales k_scale, v_scale: each new value x is stored
    as fp8_encode(float32(x) * float32(1 / scale))."""
    lib = _load()
    cu = _c(cu_q_lens, np.int32)
    kl = _c(kv_lens, np.int32)
    tb = _c(tables, np.int32)
    kn = _c(k_new, np.uint16)
    vn = _c(v_new, np.uint16)
    kv8 = np.asarray(k_cache).dtype == np.uint8
    cdt = np.uint8 if kv8 else np.uint16
    kc = np.array(k_cache, dtype=cdt, copy=True, order="C")
    vc = np.array(v_cache, dtype=cdt, copy=True, order="C")
    B = cu.shape[0] - 1
    Hkv, D = kn.shape[1], kn.shape[2]
    args = (B, _ptr(cu), _ptr(kl), Hkv, D, int(page_size), layout, tb.shape[-1], kc.shape[0],
            _ptr(tb), _ptr(kn), _ptr(vn), _ptr(kc), _ptr(vc))
    if kv8:
        rc = lib.oracle_write_kv_fp8(*args, float(k_scale), float(v_scale))
    else:
        rc = lib.oracle_write_kv(*args)
    if rc != 0:
        raise ValueError(f"oracle_write_kv failed with code {rc}")
    return kc, vc


def rotary_qkv(cu_q_lens, kv_lens, tables, q, k, v, k_cache, v_cache, page_size, cos_cache,
               sin_cache, rotary_dim, interleaved, layout=SEQ_MAJOR, k_scale=1.0, v_scale=1.0):
    """Rotary embedding of the new rows, then their scatter.

    q [T, Hq, D], k and v [T, Hkv, D] (uint16 bf16 bits; a packed [T, Hq + 2 Hkv, D] array is
    split by slicing); cos_cache, sin_cache float32 [max_position, rotary_dim / 2].
    Returns (q_out [T, Hq, D], k_cache', v_cache') with the caches copied, not modified.
    uint8 caches are FP8 caches with scales k_scale, v_scale."""
    lib = _load()
    cu = _c(cu_q_lens, np.int32)
    kl = _c(kv_lens, np.int32)
    tb = _c(tables, np.int32)
    qq, kk, vv = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    T, Hq, D = qq.shape
    Hkv = kk.shape[1]
    kv8 = np.asarray(k_cache).dtype == np.uint8
    cdt = np.uint8 if kv8 else np.uint16
    kc = np.array(k_cache, dtype=cdt, copy=True, order="C")
    vc = np.array(v_cache, dtype=cdt, copy=True, order="C")
    cs = _c(cos_cache, np.float32)
    sn = _c(sin_cache, np.float32)
    q_out = np.zeros((T, Hq, D), dtype=np.uint16)
    B = cu.shape[0] - 1
    rc = lib.oracle_rotary_qkv(B, _ptr(cu), _ptr(kl), Hq, Hkv, D, int(page_size), layout,
                               tb.shape[-1], kc.shape[0], _ptr(tb), _ptr(qq), _ptr(kk), _ptr(vv),
                               Hq * D, Hkv * D, _ptr(cs), _ptr(sn), cs.shape[0] if cs.ndim else 0,
                               int(rotary_dim), int(bool(interleaved)), _ptr(q_out), _ptr(kc),
                               _ptr(vc), int(kv8), float(k_scale), float(v_scale))
    if rc != 0:
        raise ValueError(f"oracle_rotary_qkv failed with code {rc}")
    return q_out, kc, vc


def attention(q, k_cache, v_cache, tables, cu_q_lens, kv_lens, scale, page_size,
              num_kv_heads, layout=SEQ_MAJOR, block_allowed=None, rows=None, nthreads=0,
              k_scale=1.0, v_scale=1.0):
    """fp64 attention of every row ([T, Hq, D]) or of sampled rows ([n, D]).

    rows: optional int array [n, 2] of (token, query head).
    block_allowed: optional uint8 [B, Hkv, max_pages] restricting visible key blocks.
    uint8 caches are FP8 caches: a cached K value is fp8_decode(code) * k_scale, V likewise.
    """
    lib = _load()
    qq = _c(q, np.uint16)
    kv8 = np.asarray(k_cache).dtype == np.uint8
    kc = _c(k_cache, np.uint8 if kv8 else np.uint16)
    vc = _c(v_cache, np.uint8 if kv8 else np.uint16)
    cu = _c(cu_q_lens, np.int32)
    kl = _c(kv_lens, np.int32)
    tb = _c(tables, np.int32)
    T, Hq, D = qq.shape
    B = cu.shape[0] - 1
    ba = None if block_allowed is None else _c(block_allowed, np.uint8)
    if rows is None:
        out = np.zeros((T, Hq, D), dtype=np.float64)
        rr, n = None, 0
    else:
        rr = _c(rows, np.int32).reshape(-1, 2)
        n = rr.shape[0]
        out = np.zeros((n, D), dtype=np.float64)
    head = (B, _ptr(cu), _ptr(kl), Hq, int(num_kv_heads), D, int(page_size), layout,
            tb.shape[-1], kc.shape[0], _ptr(tb), _ptr(qq), _ptr(kc), _ptr(vc))
    tail = (_ptr(ba), n, _ptr(rr), _ptr(out), int(nthreads))
    if kv8:
        rc = lib.oracle_attention_fp8(*head, float(k_scale), float(v_scale), float(scale), *tail)
    else:
        rc = lib.oracle_attention(*head, float(scale), *tail)
    if rc != 0:
        raise ValueError(f"oracle_attention failed with code {rc}")
    return out


def union_tables(mask, base_tables, past, kv_len, page_size):
    """Return (tables [Hkv, nKB], counts [Hkv], kv_lens [Hkv], selected [Hkv, nKB])."""
    lib = _load()
    m = _c(mask, np.uint8)
    bt = _c(base_tables, np.int32)
    Hq, nQB, nKB = m.shape
    Hkv = bt.shape[0]
    tables = np.zeros((Hkv, nKB), dtype=np.int32)
    counts = np.zeros(Hkv, dtype=np.int32)
    kvl = np.zeros(Hkv, dtype=np.int32)
    sel = np.zeros((Hkv, nKB), dtype=np.uint8)
    rc = lib.oracle_union_tables(_ptr(m), Hq, Hkv, nQB, nKB, _ptr(bt), int(past), int(kv_len),
                                 int(page_size), _ptr(tables), _ptr(counts), _ptr(kvl), _ptr(sel))
    if rc != 0:
        raise ValueError(f"oracle_union_tables failed with code {rc}")
    return tables, counts, kvl, sel
