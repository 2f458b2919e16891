"""Thin ctypes binding of libcpattn.so (the C ABI of include/cpattn.h).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory (``tensor.data_ptr()``) and streams
(``torch.cuda.current_stream().cuda_stream``). There is no CPU fallback: if the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcpattn.so")

CP_OK, CP_E_ARG, CP_E_SHAPE, CP_E_UNSUPPORTED, CP_E_CAPACITY, CP_E_HIP = 0, -1, -2, -3, -4, -5
CP_F32, CP_BF16 = 0, 1
CP_MAX_SEGMENTS = 64
CP_MAX_MERGE_PARTS = 64
CP_DECODE_NOALLOC_MAX_BYTES = 72 * 1024 * 1024

CP_PASS_KV, CP_PASS_Q = 0, 1

EXPORTED = ("cp_shard_map", "cp_partial_attn", "cp_merge_lse", "cp_decode_splitkv",
            "cp_decode_workspace_bytes", "cp_decode_splitkv_ex", "cp_decode_workspace_bytes_ex",
            "cp_decode_splitkv_noalloc", "cp_attn_bwd_delta", "cp_attn_bwd_workspace_bytes",
            "cp_partial_attn_bwd", "cp_ring_pass_kv_bwd",
            "cp_ring_pass_kv", "cp_ring_workspace_bytes", "cp_ring_pass_q", "cp_select_ring_variant",
            "cp_status_string", "cp_last_error")


class CpSegment(ctypes.Structure):
    """cp_segment: shard rows [local_start, local_start+len) hold positions
    [pos_start, pos_start+len) of sequence seq_id."""
    _fields_ = [("seq_id", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("pos_start", ctypes.c_int64), ("len", ctypes.c_int64),
                ("local_start", ctypes.c_int64)]

    def as_tuple(self):
        return (self.seq_id, self.pos_start, self.len, self.local_start)


class CpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


_lib = None


def _status_name(status: int) -> str:
    names = {0: "CP_OK", -1: "CP_E_ARG", -2: "CP_E_SHAPE", -3: "CP_E_UNSUPPORTED",
             -4: "CP_E_CAPACITY", -5: "CP_E_HIP"}
    return names.get(status, f"status {status}")


def load():
    """Load libcpattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m "
                           "context_ring_attention_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    i32, i64 = ctypes.c_int, ctypes.c_int64
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    segp = ctypes.POINTER(CpSegment)
    f = ctypes.c_float
    lib.cp_shard_map.argtypes = [i32, i32p, i64p, i64p, i32, i32, segp, i32,
                                 ctypes.POINTER(ctypes.c_int), i64p, i64, i64p]
    lib.cp_partial_attn.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, i32, segp, i32, segp, i32,
                                    i32, f, vp, vp, i32, vp]
    lib.cp_merge_lse.argtypes = [i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i64, i32, vp, i32, vp, vp]
    lib.cp_decode_splitkv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f, vp, vp, vp,
                                      i32, vp, vp]
    lib.cp_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.cp_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.cp_decode_splitkv_ex.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f, i32, vp,
                                         vp, vp, i32, vp, vp]
    lib.cp_decode_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f, i32,
                                              vp, i32, vp, vp]
    lib.cp_decode_workspace_bytes_ex.argtypes = [i32, i32, i32, i32, i32]
    lib.cp_decode_workspace_bytes_ex.restype = ctypes.c_size_t
    lib.cp_ring_pass_kv.argtypes = [vp, i64, segp, i32, i32, i32, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                    i64p, ctypes.POINTER(segp), ctypes.POINTER(ctypes.c_int), i32, i32,
                                    i32, i32, i32, f, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp,
                                    vp, i32, vp, vp, ctypes.c_size_t, vp]
    lib.cp_ring_workspace_bytes.argtypes = [i64, i32, i32]
    lib.cp_ring_workspace_bytes.restype = ctypes.c_size_t
    lib.cp_ring_pass_q.argtypes = [i32, ctypes.POINTER(vp), i64p, ctypes.POINTER(segp),
                                   ctypes.POINTER(ctypes.c_int), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                   i64p, ctypes.POINTER(segp), ctypes.POINTER(ctypes.c_int), i32, i32,
                                   i32, i32, i32, f, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                   ctypes.POINTER(vp), i32, ctypes.POINTER(vp), vp]
    lib.cp_attn_bwd_delta.argtypes = [vp, vp, i32, i64, i32, vp, vp]
    lib.cp_attn_bwd_workspace_bytes.argtypes = [i32]
    lib.cp_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.cp_partial_attn_bwd.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, i32, segp, i32, segp, i32,
                                        i32, f, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.cp_ring_pass_kv_bwd.argtypes = [vp, i64, segp, i32, i32, i32, ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), i64p, ctypes.POINTER(segp),
                                        ctypes.POINTER(ctypes.c_int), i32, i32, i32, i32, i32, f, vp,
                                        vp, vp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp,
                                        ctypes.c_size_t, vp]
    lib.cp_select_ring_variant.argtypes = [i64, i64, i32, i32, i32, i32, i32, ctypes.c_double,
                                           ctypes.c_double, ctypes.POINTER(ctypes.c_int),
                                           ctypes.POINTER(ctypes.c_int)]
    for name in ("cp_shard_map", "cp_partial_attn", "cp_merge_lse", "cp_decode_splitkv",
                 "cp_decode_splitkv_ex", "cp_decode_splitkv_noalloc", "cp_ring_pass_kv", "cp_ring_pass_q",
                 "cp_attn_bwd_delta", "cp_partial_attn_bwd", "cp_ring_pass_kv_bwd",
                 "cp_select_ring_variant"):
        getattr(lib, name).restype = ctypes.c_int
    lib.cp_status_string.argtypes = [ctypes.c_int]
    lib.cp_status_string.restype = ctypes.c_char_p
    lib.cp_last_error.argtypes = []
    lib.cp_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != CP_OK:
        raise CpError(status, load().cp_last_error().decode())


def last_error() -> str:
    return load().cp_last_error().decode()


# ----------------------------------------------------------------------------------- helpers
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _req(t, name: str, dtypes=None, shape=None, numel=None):
    """Checks what the C ABI cannot see behind a raw pointer: a tensor argument must be a
    contiguous device tensor of the expected dtype and shape. (A host tensor's address handed to a
    kernel would fault the GPU; a strided view would be read with the wrong layout.) Plain integer
    addresses are passed through unchecked. Kept to a few attribute reads: it runs on every call."""
    if t is None or type(t) is int:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


_DT = {}


def _types(key):
    """dtype tuples used by the checks (built once; torch is imported lazily)."""
    if not _DT:
        import torch
        _DT.update(f32=(torch.float32,), bf16=(torch.bfloat16,), i64=(torch.int64,),
                   inp=(torch.float32, torch.bfloat16))
    return _DT[key]


def _float_types():
    return _types("f32")


def _in_types():
    return _types("inp")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return CP_BF16
    if t.dtype == torch.float32:
        return CP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def segments(rows: Sequence[Sequence[int]]):
    """ctypes array of CpSegment from (seq_id, pos_start, len, local_start) tuples."""
    arr = (CpSegment * max(1, len(rows)))()
    for i, (s, p, n, loc) in enumerate(rows):
        arr[i] = CpSegment(int(s), 0, int(p), int(n), int(loc))
    return arr, len(rows)


def _segarg(segs):
    if isinstance(segs, tuple) and len(segs) == 2 and isinstance(segs[1], int):
        return segs
    return segments(segs)


# ----------------------------------------------------------------------------------- entry points
def shard_map(ranges, cp_world: int, rank: int, with_tokens: bool = True):
    """cp_shard_map. ranges: list of (seq_id, begin, end).

    Returns (list of (seq_id, pos_start, len, local_start), int64 global token indices or None).
    """
    lib = load()
    n = len(ranges)
    seq = np.ascontiguousarray([r[0] for r in ranges], dtype=np.int32)
    beg = np.ascontiguousarray([r[1] for r in ranges], dtype=np.int64)
    end = np.ascontiguousarray([r[2] for r in ranges], dtype=np.int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    n_segs = ctypes.c_int(0)
    n_tok = ctypes.c_int64(0)
    st = lib.cp_shard_map(n, seq.ctypes.data_as(i32p), beg.ctypes.data_as(i64p),
                          end.ctypes.data_as(i64p), cp_world, rank, None, 0, ctypes.byref(n_segs),
                          None, 0, ctypes.byref(n_tok))
    if st not in (CP_OK, CP_E_CAPACITY):
        _check(st)
    segs = (CpSegment * max(1, n_segs.value))()
    toks = np.zeros(max(1, n_tok.value), np.int64) if with_tokens else None
    st = lib.cp_shard_map(n, seq.ctypes.data_as(i32p), beg.ctypes.data_as(i64p),
                          end.ctypes.data_as(i64p), cp_world, rank, segs, n_segs.value,
                          ctypes.byref(n_segs), toks.ctypes.data_as(i64p) if with_tokens else None,
                          n_tok.value, ctypes.byref(n_tok))
    _check(st)
    rows = [segs[i].as_tuple() for i in range(n_segs.value)]
    return rows, (toks[: n_tok.value] if with_tokens else None)


def partial_attn(q, k, v, q_segs, kv_segs, causal: bool, softmax_scale: float, o, lse,
                 accumulate: bool = False, stream=None, check: bool = True):
    """cp_partial_attn. q: [tq, n_h, d], k/v: [tk, n_kv, d] (same dtype), o fp32, lse fp32."""
    lib = load()
    qa, nq = _segarg(q_segs)
    ka, nk = _segarg(kv_segs)
    tq, n_h, d = q.shape
    tk, n_kv = k.shape[0], k.shape[1]
    if check:
        _req(q, "q", _in_types())
        _req(k, "k", (q.dtype,), (tk, n_kv, d))
        _req(v, "v", (q.dtype,), (tk, n_kv, d))
        _req(o, "o", _float_types(), (tq, n_h, d))
        _req(lse, "lse", _float_types(), numel=tq * n_h)
    _check(lib.cp_partial_attn(_ptr(q), _ptr(k), _ptr(v), tq, tk, n_h, n_kv, d, _dtype_code(q),
                               qa, nq, ka, nk, int(causal), float(softmax_scale), _ptr(o), _ptr(lse),
                               int(accumulate), _stream(stream)))


def merge_lse(o_parts, lse_parts, o_out, lse_out=None, stream=None, check: bool = True):
    """cp_merge_lse over fp32 parts [rows, d] (any shape whose last dim is d)."""
    lib = load()
    n = len(o_parts)
    d = o_parts[0].shape[-1]
    rows = o_parts[0].numel() // d
    if len(lse_parts) != n:
        raise ValueError(f"{n} O parts but {len(lse_parts)} LSE parts")
    if check:
        for i in range(n):
            _req(o_parts[i], f"o_parts[{i}]", _float_types(), numel=rows * d)
            _req(lse_parts[i], f"lse_parts[{i}]", _float_types(), numel=rows)
        _req(o_out, "o_out", _in_types(), numel=rows * d)
        _req(lse_out, "lse_out", _float_types(), numel=rows)
    op = (ctypes.c_void_p * n)(*[_ptr(t) for t in o_parts])
    lp = (ctypes.c_void_p * n)(*[_ptr(t) for t in lse_parts])
    _check(lib.cp_merge_lse(n, op, lp, rows, d, _ptr(o_out), _dtype_code(o_out), _ptr(lse_out),
                            _stream(stream)))


def _ws_code(ws_dtype) -> int:
    if ws_dtype in ("f32", CP_F32):
        return CP_F32
    if ws_dtype in ("bf16", CP_BF16):
        return CP_BF16
    raise ValueError(f"ws_dtype must be 'f32' or 'bf16', got {ws_dtype!r}")


def decode_workspace_bytes(batch: int, n_h: int, d_h: int, n_splits: int, ws_dtype="f32") -> int:
    """cp_decode_workspace_bytes_ex: bytes of one split workspace (partial O in ws_dtype, then
    fp32 LSEs)."""
    return load().cp_decode_workspace_bytes_ex(batch, n_h, d_h, n_splits, _ws_code(ws_dtype))


def decode_workspace(batch: int, n_h: int, d_h: int, n_splits: int, device="cuda", ws_dtype="f32"):
    """One caller-owned workspace of cp_decode_workspace_bytes_ex bytes, returned as its two views:
    ws_o [batch, n_splits, n_h, d_h] (fp32 by default, bf16 for the half-size workspace) and
    ws_lse fp32 [batch, n_splits, n_h]."""
    import torch
    code = _ws_code(ws_dtype)
    nbytes = decode_workspace_bytes(batch, n_h, d_h, n_splits, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    elt, tdt = (2, torch.bfloat16) if code == CP_BF16 else (4, torch.float32)
    o_bytes = batch * n_splits * n_h * d_h * elt
    ws_o = ws[:o_bytes].view(tdt).view(batch, n_splits, n_h, d_h)
    ws_lse = ws[o_bytes:].view(torch.float32).view(batch, n_splits, n_h)
    return ws_o, ws_lse


def decode_splitkv(q, k_cache, v_cache, kv_offset, kv_len, n_splits: int, softmax_scale: float,
                   ws_o, ws_lse, o_out, lse_out=None, stream=None, check: bool = True):
    """cp_decode_splitkv (fp32 ws_o) or cp_decode_splitkv_ex (bf16 ws_o: the half-size workspace).
    q [B, n_h, d] bf16; caches [sum L, n_kv, d]; offsets/lens int64 device.

    check=False skips the tensor checks (about 3 us of host time per call): for loops whose
    tensors were validated on an earlier call."""
    import torch
    lib = load()
    B, n_h, d = q.shape
    n_kv = k_cache.shape[1]
    ws_bf16 = getattr(ws_o, "dtype", None) == torch.bfloat16
    if check:
        bf16, i64, f32 = _types("bf16"), _types("i64"), _types("f32")
        _req(q, "q", bf16)
        _req(k_cache, "k_cache", bf16)
        _req(v_cache, "v_cache", bf16, k_cache.shape)
        if k_cache.dim() != 3 or k_cache.shape[2] != d:
            raise ValueError(f"k_cache has shape {tuple(k_cache.shape)}, expected [tokens, n_kv, {d}]")
        _req(kv_offset, "kv_offset", i64, (B,))
        _req(kv_len, "kv_len", i64, (B,))
        _req(ws_o, "ws_o", _types("inp"), numel=B * n_splits * n_h * d)
        _req(ws_lse, "ws_lse", f32, numel=B * n_splits * n_h)
        _req(o_out, "o_out", _types("inp"), (B, n_h, d))
        _req(lse_out, "lse_out", f32, numel=B * n_h)
    if ws_bf16:
        _check(lib.cp_decode_splitkv_ex(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_offset),
                                        _ptr(kv_len), B, n_h, n_kv, d, _dtype_code(q), n_splits,
                                        float(softmax_scale), CP_BF16, _ptr(ws_o), _ptr(ws_lse),
                                        _ptr(o_out), _dtype_code(o_out), _ptr(lse_out),
                                        _stream(stream)))
    else:
        _check(lib.cp_decode_splitkv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_offset),
                                     _ptr(kv_len), B, n_h, n_kv, d, _dtype_code(q), n_splits,
                                     float(softmax_scale), _ptr(ws_o), _ptr(ws_lse), _ptr(o_out),
                                     _dtype_code(o_out), _ptr(lse_out), _stream(stream)))


def decode_splitkv_noalloc(q, k_cache, v_cache, kv_offset, kv_len, n_splits: int,
                           softmax_scale: float, o_out, lse_out=None, ws_dtype="f32", stream=None,
                           check: bool = True):
    """cp_decode_splitkv_noalloc: decode with the split workspace in the library's own device
    array (no workspace argument, nothing allocated). Arguments as decode_splitkv."""
    lib = load()
    B, n_h, d = q.shape
    n_kv = k_cache.shape[1]
    if check:
        bf16, i64, f32 = _types("bf16"), _types("i64"), _types("f32")
        _req(q, "q", bf16)
        _req(k_cache, "k_cache", bf16)
        _req(v_cache, "v_cache", bf16, k_cache.shape)
        if k_cache.dim() != 3 or k_cache.shape[2] != d:
            raise ValueError(f"k_cache has shape {tuple(k_cache.shape)}, expected [tokens, n_kv, {d}]")
        _req(kv_offset, "kv_offset", i64, (B,))
        _req(kv_len, "kv_len", i64, (B,))
        _req(o_out, "o_out", _types("inp"), (B, n_h, d))
        _req(lse_out, "lse_out", f32, numel=B * n_h)
    _check(lib.cp_decode_splitkv_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_offset),
                                         _ptr(kv_len), B, n_h, n_kv, d, _dtype_code(q), n_splits,
                                         float(softmax_scale), _ws_code(ws_dtype), _ptr(o_out),
                                         _dtype_code(o_out), _ptr(lse_out), _stream(stream)))


def ring_workspace_bytes(tq: int, n_h: int, d_h: int) -> int:
    """cp_ring_workspace_bytes: one partial of the optional running-mode workspace of ring_pass_kv."""
    return int(load().cp_ring_workspace_bytes(int(tq), int(n_h), int(d_h)))


def ring_workspace(tq: int, n_h: int, d_h: int, partials: int = 1, device="cuda"):
    """A device workspace of `partials` partials (uint8): a step may split into partials + 1 parts."""
    import torch
    return torch.empty(partials * ring_workspace_bytes(tq, n_h, d_h), dtype=torch.uint8, device=device)


def ring_pass_kv(q, q_segs, rank: int, k_shards, v_shards, kv_segs, causal: bool,
                 softmax_scale: float, o_out, lse_out=None, o_parts=None, lse_parts=None,
                 o_acc=None, lse_acc=None, workspace=None, stream=None, check: bool = True):
    """cp_ring_pass_kv for one rank. k_shards/v_shards/kv_segs: per shard id. workspace: optional
    device tensor (see ring_workspace) that lets a running-mode step of a small Q shard split over
    its keys."""
    lib = load()
    N = len(k_shards)
    qa, nq = _segarg(q_segs)
    tq, n_h, d = q.shape
    n_kv = k_shards[0].shape[1]
    if len(v_shards) != N or len(kv_segs) != N:
        raise ValueError("k_shards, v_shards and kv_segs must have one entry per shard")
    if check:
        _req(q, "q", _in_types())
        for i in range(N):
            _req(k_shards[i], f"k_shards[{i}]", (q.dtype,))
            _req(v_shards[i], f"v_shards[{i}]", (q.dtype,), tuple(k_shards[i].shape))
            if k_shards[i].dim() != 3 or tuple(k_shards[i].shape[1:]) != (n_kv, d):
                raise ValueError(f"k_shards[{i}] has shape {tuple(k_shards[i].shape)}, expected [tokens, {n_kv}, {d}]")
        for name, parts, shp in (("o_parts", o_parts, (tq, n_h, d)), ("lse_parts", lse_parts, None)):
            if parts is not None:
                if len(parts) != N:
                    raise ValueError(f"{name} must have {N} entries")
                for i, t in enumerate(parts):
                    _req(t, f"{name}[{i}]", _float_types(), shp, None if shp else tq * n_h)
        _req(o_acc, "o_acc", _float_types(), (tq, n_h, d))
        _req(lse_acc, "lse_acc", _float_types(), numel=tq * n_h)
        _req(o_out, "o_out", _in_types(), (tq, n_h, d))
        _req(lse_out, "lse_out", _float_types(), numel=tq * n_h)
    vp = ctypes.c_void_p
    segp = ctypes.POINTER(CpSegment)
    ks = (vp * N)(*[_ptr(t) for t in k_shards])
    vs = (vp * N)(*[_ptr(t) for t in v_shards])
    tk = (ctypes.c_int64 * N)(*[t.shape[0] for t in k_shards])
    seg_objs = [_segarg(s) for s in kv_segs]
    kvs = (segp * N)(*[ctypes.cast(a, segp) for a, _ in seg_objs])
    nkv = (ctypes.c_int * N)(*[n for _, n in seg_objs])
    op = (vp * N)(*[_ptr(t) for t in o_parts]) if o_parts is not None else None
    lp = (vp * N)(*[_ptr(t) for t in lse_parts]) if lse_parts is not None else None
    wp, wb = _ws(workspace)
    _check(lib.cp_ring_pass_kv(_ptr(q), tq, qa, nq, N, rank, ks, vs, tk, kvs, nkv, n_h, n_kv, d,
                               _dtype_code(q), int(causal), float(softmax_scale), op, lp,
                               _ptr(o_acc), _ptr(lse_acc), _ptr(o_out), _dtype_code(o_out),
                               _ptr(lse_out), wp, wb, _stream(stream)))


def select_ring_variant(new_tokens: int, cached_tokens: int, cp_world: int, n_h: int, n_kv: int,
                        d_h: int, elem_bytes: int, link_bytes_per_s: float,
                        attn_flops_per_s: float):
    """cp_select_ring_variant. Returns ("pass_kv" | "pass_q", reason)."""
    lib = load()
    v = ctypes.c_int(-1)
    r = ctypes.c_int(-1)
    _check(lib.cp_select_ring_variant(new_tokens, cached_tokens, cp_world, n_h, n_kv, d_h,
                                      elem_bytes, float(link_bytes_per_s),
                                      float(attn_flops_per_s), ctypes.byref(v), ctypes.byref(r)))
    return ("pass_kv" if v.value == CP_PASS_KV else "pass_q"), r.value


def ring_pass_q(q_shards, q_segs, k_shards, v_shards, kv_segs, causal: bool, softmax_scale: float,
                o_parts, lse_parts, o_out, lse_out=None, stream=None, check: bool = True):
    """cp_ring_pass_q over all ranks. o_parts/lse_parts: N*N buffers, slot q*N + s."""
    lib = load()
    N = len(q_shards)
    vp = ctypes.c_void_p
    segp = ctypes.POINTER(CpSegment)
    n_h, d = q_shards[0].shape[1], q_shards[0].shape[2]
    n_kv = k_shards[0].shape[1]
    if not (len(q_segs) == len(k_shards) == len(v_shards) == len(kv_segs) == len(o_out) == N):
        raise ValueError("q_shards, q_segs, k_shards, v_shards, kv_segs and o_out need one entry per rank")
    if len(o_parts) != N * N or len(lse_parts) != N * N:
        raise ValueError(f"o_parts and lse_parts need {N * N} entries (slot q*N + s)")
    if check:
        dt = q_shards[0].dtype
        for i in range(N):
            _req(q_shards[i], f"q_shards[{i}]", (dt,))
            if q_shards[i].dim() != 3 or tuple(q_shards[i].shape[1:]) != (n_h, d):
                raise ValueError(f"q_shards[{i}] has shape {tuple(q_shards[i].shape)}, expected [tokens, {n_h}, {d}]")
            _req(k_shards[i], f"k_shards[{i}]", (dt,))
            _req(v_shards[i], f"v_shards[{i}]", (dt,), tuple(k_shards[i].shape))
            if k_shards[i].dim() != 3 or tuple(k_shards[i].shape[1:]) != (n_kv, d):
                raise ValueError(f"k_shards[{i}] has shape {tuple(k_shards[i].shape)}, expected [tokens, {n_kv}, {d}]")
            tqi = q_shards[i].shape[0]
            _req(o_out[i], f"o_out[{i}]", _in_types(), (tqi, n_h, d))
            if lse_out is not None:
                _req(lse_out[i], f"lse_out[{i}]", _float_types(), numel=tqi * n_h)
            for s_ in range(N):
                _req(o_parts[i * N + s_], f"o_parts[{i * N + s_}]", _float_types(), (tqi, n_h, d))
                _req(lse_parts[i * N + s_], f"lse_parts[{i * N + s_}]", _float_types(), numel=tqi * n_h)
    qs = (vp * N)(*[_ptr(t) for t in q_shards])
    tq = (ctypes.c_int64 * N)(*[t.shape[0] for t in q_shards])
    qseg_objs = [_segarg(s) for s in q_segs]
    qsg = (segp * N)(*[ctypes.cast(a, segp) for a, _ in qseg_objs])
    nqs = (ctypes.c_int * N)(*[n for _, n in qseg_objs])
    ks = (vp * N)(*[_ptr(t) for t in k_shards])
    vs = (vp * N)(*[_ptr(t) for t in v_shards])
    tk = (ctypes.c_int64 * N)(*[t.shape[0] for t in k_shards])
    kseg_objs = [_segarg(s) for s in kv_segs]
    ksg = (segp * N)(*[ctypes.cast(a, segp) for a, _ in kseg_objs])
    nks = (ctypes.c_int * N)(*[n for _, n in kseg_objs])
    op = (vp * (N * N))(*[_ptr(t) for t in o_parts])
    lp = (vp * (N * N))(*[_ptr(t) for t in lse_parts])
    oo = (vp * N)(*[_ptr(t) for t in o_out])
    lo = (vp * N)(*[_ptr(t) for t in lse_out]) if lse_out is not None else None
    _check(lib.cp_ring_pass_q(N, qs, tq, qsg, nqs, ks, vs, tk, ksg, nks, n_h, n_kv, d,
                              _dtype_code(q_shards[0]), int(causal), float(softmax_scale), op, lp,
                              oo, _dtype_code(o_out[0]), lo, _stream(stream)))


# ----------------------------------------------------------------------------------- backward
def attn_bwd_delta(o, d_o, delta, stream=None, check: bool = True):
    """cp_attn_bwd_delta: delta = rowsum(dO * O). o fp32 [..., d], d_o [..., d], delta fp32 [...]."""
    lib = load()
    d = o.shape[-1]
    rows = o.numel() // d
    if check:
        _req(o, "o", _float_types(), numel=rows * d)
        _req(d_o, "d_o", _in_types(), numel=rows * d)
        _req(delta, "delta", _float_types(), numel=rows)
    _check(lib.cp_attn_bwd_delta(_ptr(o), _ptr(d_o), _dtype_code(d_o), rows, d, _ptr(delta),
                                 _stream(stream)))


def attn_bwd_workspace_bytes(d_h: int) -> int:
    """cp_attn_bwd_workspace_bytes: size of the optional backward workspace for head dim d_h."""
    return int(load().cp_attn_bwd_workspace_bytes(int(d_h)))


def attn_bwd_workspace(d_h: int, device="cuda"):
    """A device workspace of cp_attn_bwd_workspace_bytes(d_h) bytes (uint8, 256-byte aligned)."""
    import torch
    return torch.empty(attn_bwd_workspace_bytes(d_h), dtype=torch.uint8, device=device)


def _ws(workspace):
    return (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())


def partial_attn_bwd(q, k, v, q_segs, kv_segs, causal: bool, softmax_scale: float, lse, delta, d_o,
                     dq, dk, dv, workspace=None, stream=None, check: bool = True):
    """cp_partial_attn_bwd: adds one ring step's gradient contributions into dq, dk, dv (fp32).
    workspace: optional device tensor (see attn_bwd_workspace) that lets the dK/dV work split."""
    lib = load()
    qa, nq = _segarg(q_segs)
    ka, nk = _segarg(kv_segs)
    tq, n_h, d = q.shape
    tk, n_kv = k.shape[0], k.shape[1]
    if check:
        _req(q, "q", _in_types())
        _req(k, "k", (q.dtype,), (tk, n_kv, d))
        _req(v, "v", (q.dtype,), (tk, n_kv, d))
        _req(lse, "lse", _float_types(), numel=tq * n_h)
        _req(delta, "delta", _float_types(), numel=tq * n_h)
        _req(d_o, "d_o", (q.dtype,), (tq, n_h, d))
        _req(dq, "dq", _float_types(), (tq, n_h, d))
        _req(dk, "dk", _float_types(), (tk, n_kv, d))
        _req(dv, "dv", _float_types(), (tk, n_kv, d))
        _req(workspace, "workspace")
    _check(lib.cp_partial_attn_bwd(_ptr(q), _ptr(k), _ptr(v), tq, tk, n_h, n_kv, d, _dtype_code(q),
                                   qa, nq, ka, nk, int(causal), float(softmax_scale), _ptr(lse),
                                   _ptr(delta), _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv),
                                   *_ws(workspace), _stream(stream)))


def ring_pass_kv_bwd(q, q_segs, rank: int, k_shards, v_shards, kv_segs, causal: bool,
                     softmax_scale: float, o, lse, d_o, delta, dq, dk_shards, dv_shards,
                     workspace=None, stream=None, check: bool = True):
    """cp_ring_pass_kv_bwd for one rank: adds its gradient contributions into dq and into every
    KV shard's dk_shards[s] / dv_shards[s]."""
    lib = load()
    N = len(k_shards)
    qa, nq = _segarg(q_segs)
    tq, n_h, d = q.shape
    n_kv = k_shards[0].shape[1]
    if not (len(v_shards) == len(kv_segs) == len(dk_shards) == len(dv_shards) == N):
        raise ValueError("k_shards, v_shards, kv_segs, dk_shards and dv_shards need one entry per shard")
    if check:
        _req(q, "q", _in_types())
        _req(o, "o", _float_types(), (tq, n_h, d))
        _req(lse, "lse", _float_types(), numel=tq * n_h)
        _req(d_o, "d_o", (q.dtype,), (tq, n_h, d))
        _req(delta, "delta", _float_types(), numel=tq * n_h)
        _req(dq, "dq", _float_types(), (tq, n_h, d))
        for i in range(N):
            shp = tuple(k_shards[i].shape)
            _req(k_shards[i], f"k_shards[{i}]", (q.dtype,))
            _req(v_shards[i], f"v_shards[{i}]", (q.dtype,), shp)
            _req(dk_shards[i], f"dk_shards[{i}]", _float_types(), shp)
            _req(dv_shards[i], f"dv_shards[{i}]", _float_types(), shp)
        _req(workspace, "workspace")
    vp = ctypes.c_void_p
    segp = ctypes.POINTER(CpSegment)
    ks = (vp * N)(*[_ptr(t) for t in k_shards])
    vs = (vp * N)(*[_ptr(t) for t in v_shards])
    tk = (ctypes.c_int64 * N)(*[t.shape[0] for t in k_shards])
    seg_objs = [_segarg(s_) for s_ in kv_segs]
    kvs = (segp * N)(*[ctypes.cast(a, segp) for a, _ in seg_objs])
    nkv = (ctypes.c_int * N)(*[n for _, n in seg_objs])
    dks = (vp * N)(*[_ptr(t) for t in dk_shards])
    dvs = (vp * N)(*[_ptr(t) for t in dv_shards])
    _check(lib.cp_ring_pass_kv_bwd(_ptr(q), tq, qa, nq, N, rank, ks, vs, tk, kvs, nkv, n_h, n_kv, d,
                                   _dtype_code(q), int(causal), float(softmax_scale), _ptr(o),
                                   _ptr(lse), _ptr(d_o), _ptr(delta), _ptr(dq), dks, dvs,
                                   *_ws(workspace), _stream(stream)))
