"""fp64 CPU oracle for one context-parallel rank's exact attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY. Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package. It shares no code with the HIP path
(``context_ring_attention_amd``) and neither imports the other.

The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only builds and loads it and
converts numpy arrays. Page citations are in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _declare(lib):
    """Argument and result types of the library's entry points."""
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_shard_tokens.argtypes = [ctypes.c_int, i32p, i64p, i64p, ctypes.c_int, ctypes.c_int,
                                     i32p, i64p, i64p, ctypes.c_int64, i64p]
    lib.orc_shard_tokens.restype = ctypes.c_int
    lib.orc_attention.argtypes = [f32p, f32p, f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, i32p, i64p, i32p, i64p, ctypes.c_int,
                                  ctypes.c_double, i64p, ctypes.c_int64, f64p, f64p]
    lib.orc_attention.restype = ctypes.c_int
    lib.orc_merge.argtypes = [ctypes.c_int, ctypes.POINTER(f64p), ctypes.POINTER(f64p),
                              ctypes.c_int64, ctypes.c_int, f64p, f64p]
    lib.orc_merge.restype = None
    lib.orc_split_bounds.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, i64p, i64p]
    lib.orc_split_bounds.restype = None
    lib.orc_attention_backward.argtypes = [f32p, f32p, f32p, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p, i64p, i32p,
                                           i64p, ctypes.c_int, ctypes.c_double, f64p, f64p, f32p,
                                           f64p, f64p, f64p]
    lib.orc_attention_backward.restype = ctypes.c_int
    for name in ("orc_pass_kv_shard", "orc_pass_q_query", "orc_pass_q_slot"):
        getattr(lib, name).argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def use_library(path):
    """Routes every oracle call through the library at ``path`` (None: back to liboracle.so).
    Used by the test that plants mistakes in a copy of oracle.c to check the pins catch them."""
    global _lib
    _lib = None if path is None else _declare(ctypes.CDLL(path))


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def num_threads() -> int:
    return _load().orc_num_threads()


def shard_tokens(ranges, cp_world: int, rank: int):
    """Tokens owned by ``rank``. ``ranges``: list of (seq_id, begin, end).

    Returns (seq int32[n], pos int64[n], global_index int64[n]) in the rank's local order.
    """
    lib = _load()
    seq = np.ascontiguousarray([r[0] for r in ranges], dtype=np.int32)
    beg = np.ascontiguousarray([r[1] for r in ranges], dtype=np.int64)
    end = np.ascontiguousarray([r[2] for r in ranges], dtype=np.int64)
    n = ctypes.c_int64(0)
    rc = lib.orc_shard_tokens(len(ranges), _ptr(seq, ctypes.c_int32), _ptr(beg, ctypes.c_int64),
                              _ptr(end, ctypes.c_int64), cp_world, rank, None, None, None, 0,
                              ctypes.byref(n))
    if rc < 0:
        raise ValueError("orc_shard_tokens: bad arguments")
    cap = n.value
    ts = np.zeros(max(cap, 1), np.int32)
    tp = np.zeros(max(cap, 1), np.int64)
    tg = np.zeros(max(cap, 1), np.int64)
    rc = lib.orc_shard_tokens(len(ranges), _ptr(seq, ctypes.c_int32), _ptr(beg, ctypes.c_int64),
                              _ptr(end, ctypes.c_int64), cp_world, rank, _ptr(ts, ctypes.c_int32),
                              _ptr(tp, ctypes.c_int64), _ptr(tg, ctypes.c_int64), cap,
                              ctypes.byref(n))
    if rc != 0:
        raise RuntimeError("orc_shard_tokens failed")
    return ts[:cap], tp[:cap], tg[:cap]


def attention(q, k, v, n_h: int, n_kv: int, q_seq, q_pos, k_seq, k_pos, causal: bool,
              scale: float, rows=None):
    """fp64 attention of query tokens over keys. q: [tq, n_h, d], k/v: [tk, n_kv, d] (fp32).

    Returns (o float64 [n, n_h, d], lse float64 [n, n_h]) with n = tq or len(rows).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    tq = q.shape[0]
    tk = k.shape[0]
    d = q.shape[-1]
    assert q.shape == (tq, n_h, d) and k.shape == (tk, n_kv, d) and v.shape == (tk, n_kv, d)
    q_seq = np.ascontiguousarray(q_seq, dtype=np.int32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    k_seq = np.ascontiguousarray(k_seq, dtype=np.int32)
    k_pos = np.ascontiguousarray(k_pos, dtype=np.int64)
    assert q_seq.shape == (tq,) and q_pos.shape == (tq,)
    assert k_seq.shape == (tk,) and k_pos.shape == (tk,)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_out = rows.shape[0]
        rows_p = _ptr(rows, ctypes.c_int64)
    else:
        n_out = tq
        rows_p = None
    o = np.zeros((n_out, n_h, d), np.float64)
    lse = np.zeros((n_out, n_h), np.float64)
    # zero-size arrays still need a valid pointer
    kk = k if tk else np.zeros((1, n_kv, d), np.float32)
    vv = v if tk else np.zeros((1, n_kv, d), np.float32)
    ks = k_seq if tk else np.zeros(1, np.int32)
    kp = k_pos if tk else np.zeros(1, np.int64)
    rc = lib.orc_attention(_ptr(q, ctypes.c_float), _ptr(kk, ctypes.c_float),
                           _ptr(vv, ctypes.c_float), tq, tk, n_h, n_kv, d,
                           _ptr(q_seq, ctypes.c_int32), _ptr(q_pos, ctypes.c_int64),
                           _ptr(ks, ctypes.c_int32), _ptr(kp, ctypes.c_int64), int(causal),
                           float(scale), rows_p, n_out, _ptr(o, ctypes.c_double),
                           _ptr(lse, ctypes.c_double))
    if rc != 0:
        raise ValueError("orc_attention: bad arguments")
    return o, lse


def attention_backward(q, k, v, n_h: int, n_kv: int, q_seq, q_pos, k_seq, k_pos, causal: bool,
                       scale: float, o, lse, d_o):
    """fp64 gradients of the partial attention of the query tokens over the given keys, from the
    final forward (o [tq, n_h, d], lse [tq, n_h]) and the output gradient d_o [tq, n_h, d].

    Returns (dq float64 [tq, n_h, d], dk float64 [tk, n_kv, d], dv float64 [tk, n_kv, d]).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    d_o = np.ascontiguousarray(d_o, dtype=np.float32)
    o = np.ascontiguousarray(o, dtype=np.float64)
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    tq, tk, d = q.shape[0], k.shape[0], q.shape[-1]
    assert q.shape == (tq, n_h, d) and k.shape == (tk, n_kv, d) and v.shape == (tk, n_kv, d)
    assert o.shape == (tq, n_h, d) and d_o.shape == (tq, n_h, d) and lse.shape == (tq, n_h)
    q_seq = np.ascontiguousarray(q_seq, dtype=np.int32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    k_seq = np.ascontiguousarray(k_seq, dtype=np.int32)
    k_pos = np.ascontiguousarray(k_pos, dtype=np.int64)
    dq = np.zeros((tq, n_h, d), np.float64)
    dk = np.zeros((max(tk, 1), n_kv, d), np.float64)
    dv = np.zeros((max(tk, 1), n_kv, d), np.float64)
    kk = k if tk else np.zeros((1, n_kv, d), np.float32)
    vv = v if tk else np.zeros((1, n_kv, d), np.float32)
    ks = k_seq if tk else np.zeros(1, np.int32)
    kp = k_pos if tk else np.zeros(1, np.int64)
    rc = lib.orc_attention_backward(_ptr(q, ctypes.c_float), _ptr(kk, ctypes.c_float),
                                    _ptr(vv, ctypes.c_float), tq, tk, n_h, n_kv, d,
                                    _ptr(q_seq, ctypes.c_int32), _ptr(q_pos, ctypes.c_int64),
                                    _ptr(ks, ctypes.c_int32), _ptr(kp, ctypes.c_int64), int(causal),
                                    float(scale), _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
                                    _ptr(d_o, ctypes.c_float), _ptr(dq, ctypes.c_double),
                                    _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double))
    if rc != 0:
        raise ValueError("orc_attention_backward: bad arguments")
    return dq, dk[:tk], dv[:tk]


def merge(o_parts, lse_parts):
    """LSE-weighted merge. o_parts[i]: [rows, d] fp64, lse_parts[i]: [rows] fp64."""
    lib = _load()
    n = len(o_parts)
    assert n == len(lse_parts) and n >= 1
    o_parts = [np.ascontiguousarray(x, dtype=np.float64) for x in o_parts]
    lse_parts = [np.ascontiguousarray(x, dtype=np.float64) for x in lse_parts]
    rows, d = o_parts[0].shape
    f64p = ctypes.POINTER(ctypes.c_double)
    op = (f64p * n)(*[_ptr(x, ctypes.c_double) for x in o_parts])
    lp = (f64p * n)(*[_ptr(x, ctypes.c_double) for x in lse_parts])
    o = np.zeros((rows, d), np.float64)
    lse = np.zeros(rows, np.float64)
    lib.orc_merge(n, op, lp, rows, d, _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    return o, lse


def split_bounds(length: int, n_splits: int):
    """[(lo, hi)] key ranges of the n_splits decode splits of a request with ``length`` keys."""
    lib = _load()
    out = []
    lo = ctypes.c_int64(0)
    hi = ctypes.c_int64(0)
    for c in range(n_splits):
        lib.orc_split_bounds(length, n_splits, c, ctypes.byref(lo), ctypes.byref(hi))
        out.append((lo.value, hi.value))
    return out


def _ring(name, *args) -> int:
    v = getattr(_load(), name)(*[int(a) for a in args])
    if v < 0:
        raise ValueError(f"{name}{args}: bad arguments")
    return v


def pass_kv_shard(cp_world: int, rank: int, step: int) -> int:
    """KV shard held by ``rank`` at ring Pass-KV step ``step``."""
    return _ring("orc_pass_kv_shard", cp_world, rank, step)


def pass_q_query(cp_world: int, kv_shard: int, step: int) -> int:
    """Q shard hosted by the owner of ``kv_shard`` at ring Pass-Q step ``step``."""
    return _ring("orc_pass_q_query", cp_world, kv_shard, step)


def pass_q_slot(cp_world: int, q_shard: int, kv_shard: int) -> int:
    """Storage slot of the Pass-Q partial of ``q_shard`` against ``kv_shard``."""
    return _ring("orc_pass_q_slot", cp_world, q_shard, kv_shard)
