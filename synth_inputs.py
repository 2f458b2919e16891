"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention arithmetic: it only draws random numbers and describes workload
shapes. Both the tests/bench (HIP path) and the oracle consume what it returns.

Recipe (per token, so that any shard can be regenerated without materialising a whole
1M-token tensor): tensor ``tensor_id`` of seed ``seed`` is drawn in blocks of 4096 tokens;
block ``j`` comes from ``torch.Generator().manual_seed(seed*1000003 + tensor_id*65537 + j)``
and ``torch.randn([4096, *per_token_shape])``, times ``std``.  bf16 workloads round those fp32
values to bf16 (round to nearest even, torch's conversion); the oracle consumes the rounded
values widened back to fp32 (exact).
"""
from __future__ import annotations

import math

import numpy as np
import torch

BLOCK = 4096
TID_Q, TID_K, TID_V, TID_LEN, TID_PO, TID_PL, TID_MISC, TID_DO = 1, 2, 3, 4, 5, 6, 7, 8
# saved forward activations drawn directly (backward tests at sizes the oracle forward cannot redo)
TID_SAVED_O, TID_SAVED_LSE = 9, 10

K1 = 1024

# Workloads: one attention layer's per-GPU head share (16 query heads, 1 KV head under TP8 for
# the 128-query-head / 8-KV-head model), D_H = 128, except the tiny fp32 ring.
CONFIGS = {
    "tiny_ring_fp32": dict(
        kind="pass_kv", seqs=[256], cp=4, n_h=4, n_kv=1, d_h=64, dtype="f32",
        std=1.0 / math.sqrt(64)),
    "prefill_128k_cp4": dict(
        kind="pass_kv", seqs=[128 * K1], cp=4, n_h=16, n_kv=1, d_h=128, dtype="bf16", std=1.0),
    "persistent_kv_8k_on_120k": dict(
        kind="pass_q", new=8 * K1, cached=120 * K1, cp=4, n_h=16, n_kv=1, d_h=128,
        dtype="bf16", std=1.0),
    "decode_b32_32k_128k": dict(
        kind="decode", batch=32, len_lo=32 * K1, len_hi=128 * K1, n_splits=256, n_h=16, n_kv=1,
        d_h=128, dtype="bf16", std=1.0),
    "prefill_1m_varlen_cp8": dict(
        kind="pass_kv", seqs=[64 * K1, 192 * K1, 256 * K1, 512 * K1], cp=8, n_h=16, n_kv=1,
        d_h=128, dtype="bf16", std=1.0),
}


def _block_seed(seed: int, tensor_id: int, block: int) -> int:
    return (seed * 1000003 + tensor_id * 65537 + block) & 0x7FFFFFFFFFFFFFFF


def normal_tokens(seed: int, tensor_id: int, token_index, per_token_shape, std: float = 1.0):
    """fp32 torch tensor [len(token_index), *per_token_shape] of seeded N(0, std^2) values.

    ``token_index`` holds global token indices (any order, repeats allowed).
    """
    idx = np.asarray(token_index, dtype=np.int64).reshape(-1)
    per = int(np.prod(per_token_shape)) if len(per_token_shape) else 1
    out = torch.empty((idx.shape[0], per), dtype=torch.float32)
    if idx.shape[0] == 0:
        return out.reshape((0, *per_token_shape))
    blocks = idx // BLOCK
    order = np.argsort(blocks, kind="stable")
    sb = blocks[order]
    starts = np.flatnonzero(np.r_[True, sb[1:] != sb[:-1]])
    ends = np.r_[starts[1:], len(sb)]
    g = torch.Generator()
    for s, e in zip(starts, ends):
        b = int(sb[s])
        g.manual_seed(_block_seed(seed, tensor_id, b))
        blk = torch.randn((BLOCK, per), generator=g, dtype=torch.float32)
        sel = order[s:e]
        out[torch.from_numpy(sel)] = blk[torch.from_numpy(idx[sel] - b * BLOCK)]
    if std != 1.0:
        out.mul_(std)
    return out.reshape((idx.shape[0], *per_token_shape))


def to_dtype(x: torch.Tensor, dtype: str):
    """Round fp32 values to the workload dtype. Returns (values_as_dtype, exact_fp32_view)."""
    if dtype == "bf16":
        xb = x.to(torch.bfloat16)
        return xb, xb.to(torch.float32)
    if dtype == "f32":
        return x, x
    raise ValueError(dtype)


def decode_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Cached KV lengths, integer uniform on [lo, hi] inclusive."""
    g = torch.Generator()
    g.manual_seed(_block_seed(seed, TID_LEN, 0))
    return torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64).numpy()


def random_partials(seed: int, n_parts: int, rows: int, d_h: int, p_empty: float = 0.1):
    """Synthetic partial results for merge tests: O ~ N(0,1), LSE ~ N(0, 3^2), and with
    probability ``p_empty`` a part of a row is empty (O = 0, LSE = -inf). Some rows are empty in
    every part. fp32 torch tensors: o [n, rows, d], lse [n, rows]."""
    g = torch.Generator()
    g.manual_seed(_block_seed(seed, TID_PO, 0))
    o = torch.randn((n_parts, rows, d_h), generator=g, dtype=torch.float32)
    lse = 3.0 * torch.randn((n_parts, rows), generator=g, dtype=torch.float32)
    empty = torch.rand((n_parts, rows), generator=g) < p_empty
    if rows >= 4:
        empty[:, 1] = True          # a row that no part saw
        empty[1:, 2] = True if n_parts > 1 else empty[1:, 2]  # a row seen by one part only
    lse[empty] = -math.inf
    o[empty] = 0.0
    return o, lse


def uniform_ints(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    g = torch.Generator()
    g.manual_seed(_block_seed(seed, TID_MISC, 0))
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64).numpy()
