"""Builders of ring workloads for the parity tests and the bench.

The HIP side takes its shard layout from the library's cp_shard_map and the oracle side from the
oracle's own shard map (the two are checked bit-exact elsewhere); both draw Q/K/V from the seeded
generators in synth_inputs, per global token index.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import synth_inputs as si


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


class Shard:
    """One rank's tokens: product segments (for the library) and device tensors."""

    def __init__(self, segs, tokens):
        self.segs = segs          # list of (seq_id, pos_start, len, local_start)
        self.tokens = tokens      # global packed token index per local row
        self.q = self.k = self.v = None


def product_shards(ranges, N, ranks=None):
    from context_ring_attention_amd import binding as cp
    ranks = range(N) if ranks is None else ranks
    return {r: Shard(*cp.shard_map(ranges, N, r)) for r in ranks}


def device_tensor(seed, tid, tokens, shape, std, dtype, device="cuda", gen=None):
    x = (gen or si.normal_tokens)(seed, tid, tokens, shape, std)
    xd, _ = si.to_dtype(x, dtype)
    return xd.contiguous().to(device)


def oracle_view(seed, tid, tokens, shape, std, dtype, gen=None):
    """The exact fp32 values the device holds for these tokens (bf16-rounded when bf16)."""
    x = (gen or si.normal_tokens)(seed, tid, tokens, shape, std)
    _, xf = si.to_dtype(x, dtype)
    return xf.numpy()


class Planted:
    """Seeded inputs with planted structure, for driving the online softmax's rarely taken paths
    (a row max that jumps late, scores spread over tens of nats). Input construction only: it
    draws the same seeded N(0, std^2) tokens as synth_inputs.normal_tokens and then, per global
    token index g,
      - Q and K may take their own std (q_std, k_std: wide score ranges); V keeps `std`;
      - Q: adds q_bias * u to every query head (u = the all-ones direction / sqrt(D));
      - K: adds ramp * (g / total) * u (keys score higher the later they sit), and overwrites the
        keys at `spikes` {g: a} with a * u, so a query scores them about scale * a * (q.u + q_bias).
    V is plain. The device and the oracle both take their values from here, so they see identical
    (bf16-rounded) inputs."""

    def __init__(self, q_bias=0.0, ramp=0.0, spikes=None, total=1, q_std=None, k_std=None):
        self.q_bias, self.ramp, self.spikes, self.total = q_bias, ramp, dict(spikes or {}), max(1, total)
        self.q_std, self.k_std = q_std, k_std

    def __call__(self, seed, tid, tokens, shape, std):
        tokens = np.asarray(tokens, np.int64)
        if tid == si.TID_Q and self.q_std is not None:
            std = self.q_std
        if tid == si.TID_K and self.k_std is not None:
            std = self.k_std
        x = si.normal_tokens(seed, tid, tokens, shape, std)
        d = shape[-1]
        u = torch.full((d,), 1.0 / math.sqrt(d))
        if tid == si.TID_Q and self.q_bias:
            x += self.q_bias * u
        if tid == si.TID_K:
            if self.ramp:
                x += (self.ramp * torch.from_numpy(tokens / self.total).float()).view(-1, *([1] * len(shape))) * u
            for g, a in self.spikes.items():
                hit = np.flatnonzero(tokens == g)
                if hit.size:
                    x[torch.from_numpy(hit)] = (a * u).expand(shape)
        return x


def seq_pos_of(ranges, tokens):
    """(seq, pos) of packed global token indices under the same base rule as the shard map."""
    lens = {}
    for s, b, e in ranges:
        lens[s] = max(lens.get(s, 0), e)
    ids = sorted(lens)
    bases = np.cumsum([0] + [lens[i] for i in ids[:-1]])
    tokens = np.asarray(tokens, np.int64)
    idx = np.searchsorted(bases, tokens, side="right") - 1
    seq = np.asarray(ids, np.int64)[idx]
    pos = tokens - bases[idx]
    return seq.astype(np.int32), pos


def sample_rows(segs, n_random, seed):
    """Local rows to check at full size: first and last row of every segment plus random rows."""
    rows = set()
    for _, _, n, loc in segs:
        rows.add(loc)
        rows.add(loc + n - 1)
        rows.add(loc + n // 2)
    total = sum(n for _, _, n, _ in segs)
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.integers(0, total, n_random))
    return np.array(sorted(rows), np.int64)


def scale_of(d_h: int) -> float:
    return 1.0 / math.sqrt(d_h)
