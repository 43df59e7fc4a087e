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


def write_kv(cu_q_lens, kv_lens, tables, k_new, v_new, k_cache, v_cache, page_size,
             layout=SEQ_MAJOR):
    """Return (k_cache', v_cache'): copies of the caches with the new rows scattered in."""
    lib = _load()
    cu = _c(cu_q_lens, np.int32)
    kl = _c(kv_lens, np.int32)
    tb = _c(tables, np.int32)
    kn = _c(k_new, np.uint16)
    vn = _c(v_new, np.uint16)
    kc = np.array(k_cache, dtype=np.uint16, copy=True, order="C")
    vc = np.array(v_cache, dtype=np.uint16, copy=True, order="C")
    B = cu.shape[0] - 1
    Hkv, D = kn.shape[1], kn.shape[2]
    rc = lib.oracle_write_kv(B, _ptr(cu), _ptr(kl), Hkv, D, int(page_size), layout,
                             tb.shape[-1], kc.shape[0], _ptr(tb), _ptr(kn), _ptr(vn),
                             _ptr(kc), _ptr(vc))
    if rc != 0:
        raise ValueError(f"oracle_write_kv failed with code {rc}")
    return kc, vc


def attention(q, k_cache, v_cache, tables, cu_q_lens, kv_lens, scale, page_size,
              num_kv_heads, layout=SEQ_MAJOR, block_allowed=None, rows=None, nthreads=0):
    """fp64 attention of every row ([T, Hq, D]) or of sampled rows ([n, D]).

    rows: optional int array [n, 2] of (token, query head).
    block_allowed: optional uint8 [B, Hkv, max_pages] restricting visible key blocks.
    """
    lib = _load()
    qq = _c(q, np.uint16)
    kc = _c(k_cache, np.uint16)
    vc = _c(v_cache, np.uint16)
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
    rc = lib.oracle_attention(B, _ptr(cu), _ptr(kl), Hq, int(num_kv_heads), D, int(page_size),
                              layout, tb.shape[-1], kc.shape[0], _ptr(tb), _ptr(qq), _ptr(kc),
                              _ptr(vc), float(scale), _ptr(ba), n, _ptr(rr), _ptr(out),
                              int(nthreads))
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
