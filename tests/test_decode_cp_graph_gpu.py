"""Decode across CP ranks and decode under HIP graph capture, against the oracle.

Decode context parallelism ("Context Parallelism for Scalable Million-Token Inference", section
"核心创新", decode row): every rank holds a load-balanced shard of each request's KV cache, runs
split-KV decode over it, and the per-rank partials are merged with the same LSE-weighted rule.
The result must equal single-device attention over the whole cache. The software-stack section
of the same page names CUDA Graphs for the decode step; here the step (split kernel + split
merge) is captured into a HIP graph through torch and replayed.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from ring_cases import device_tensor, log, oracle_view, scale_of

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3  # bf16 inputs


def _oracle_decode(seed, lengths, offs, n_h, n_kv, d, scale, q_seed=None):
    """Oracle attention of each request's query over its whole cache (K/V drawn with `seed`, the
    query with `q_seed`, default the same)."""
    B = len(lengths)
    qf = oracle_view(seed if q_seed is None else q_seed, si.TID_Q, np.arange(B), (n_h, d), 1.0, "bf16")
    outs, lses = [], []
    for b in range(B):
        lo, L = int(offs[b]), int(lengths[b])
        kf = oracle_view(seed, si.TID_K, np.arange(lo, lo + L), (n_kv, d), 1.0, "bf16")
        vf = oracle_view(seed, si.TID_V, np.arange(lo, lo + L), (n_kv, d), 1.0, "bf16")
        o, l = oracle.attention(qf[b:b + 1], kf, vf, n_h, n_kv, np.zeros(1, np.int32),
                                np.array([L], np.int64), np.zeros(L, np.int32), np.arange(L), False, scale)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)


def _check(o_dev, l_dev, o_ref, l_ref, what):
    o = o_dev.float().cpu().numpy().reshape(o_ref.shape)
    lse = l_dev.float().cpu().numpy().reshape(l_ref.shape)
    err_o = float(np.max(np.abs(o - o_ref)))
    err_l = float(np.max(np.abs(lse - l_ref)))
    log(f"{what}: max|dO| {err_o:.2e}, max|dLSE| {err_l:.2e}")
    assert err_o <= TOL_O and err_l <= TOL_LSE, what


def test_decode_across_cp_ranks_merged():
    from context_ring_attention_amd import binding as cp
    seed, N, n_h, n_kv, d, S = 0, 4, 16, 1, 128, 16
    lengths = np.array([3000, 517, 1290, 64], np.int64)
    B = len(lengths)
    offs = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    scale = scale_of(d)
    q = device_tensor(seed, si.TID_Q, np.arange(B), (n_h, d), 1.0, "bf16")
    ranges = [(b, 0, int(lengths[b])) for b in range(B)]
    o_parts, l_parts = [], []
    for r in range(N):
        segs, toks = cp.shard_map(ranges, N, r)
        # rank r's packed cache: its tokens of every request, request by request (two chunks each)
        lens_r = np.zeros(B, np.int64)
        offs_r = np.zeros(B, np.int64)
        first = {}
        for seq, pos, ln, loc in segs:
            first.setdefault(seq, loc)
            lens_r[seq] += ln
        for b in range(B):
            offs_r[b] = first.get(b, 0)
        kc = device_tensor(seed, si.TID_K, toks, (n_kv, d), 1.0, "bf16")
        vc = device_tensor(seed, si.TID_V, toks, (n_kv, d), 1.0, "bf16")
        ws_o, ws_l = cp.decode_workspace(B, n_h, d, S)
        o_r = torch.empty(B, n_h, d, device="cuda")
        l_r = torch.empty(B, n_h, device="cuda")
        cp.decode_splitkv(q, kc, vc, torch.from_numpy(offs_r).cuda(), torch.from_numpy(lens_r).cuda(), S,
                          scale, ws_o, ws_l, o_r, l_r)
        o_parts.append(o_r.view(B * n_h, d))
        l_parts.append(l_r.view(B * n_h))
    o_out = torch.empty(B * n_h, d, device="cuda")
    l_out = torch.empty(B * n_h, device="cuda")
    cp.merge_lse(o_parts, l_parts, o_out, l_out)
    torch.cuda.synchronize()
    o_ref, l_ref = _oracle_decode(seed, lengths, offs, n_h, n_kv, d, scale)
    _check(o_out, l_out, o_ref, l_ref, f"decode over {N} ranks, merged")


def test_decode_step_graph_replays_match_eager():
    from context_ring_attention_amd import binding as cp
    n_h, n_kv, d, S = 16, 1, 128, 256
    lengths = np.array([4097, 300, 1000], np.int64)
    B = len(lengths)
    offs = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    total = int(lengths.sum())
    scale = scale_of(d)
    kc = device_tensor(0, si.TID_K, np.arange(total), (n_kv, d), 1.0, "bf16")
    vc = device_tensor(0, si.TID_V, np.arange(total), (n_kv, d), 1.0, "bf16")
    offs_d = torch.from_numpy(offs).cuda()
    lens_d = torch.from_numpy(lengths).cuda()
    ws_o, ws_l = cp.decode_workspace(B, n_h, d, S)
    q = torch.empty(B, n_h, d, dtype=torch.bfloat16, device="cuda")
    o_g = torch.empty(B, n_h, d, device="cuda")
    l_g = torch.empty(B, n_h, device="cuda")
    step = lambda o, l: cp.decode_splitkv(q, kc, vc, offs_d, lens_d, S, scale, ws_o, ws_l, o, l)

    q.copy_(device_tensor(11, si.TID_Q, np.arange(B), (n_h, d), 1.0, "bf16"))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        step(o_g, l_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(o_g, l_g)
    torch.cuda.synchronize()

    o_e = torch.empty_like(o_g)
    l_e = torch.empty_like(l_g)
    for rep, qseed in enumerate([11, 12, 13]):
        # the program's own eager work between replays: new query, an eager step, a sync
        q.copy_(device_tensor(qseed, si.TID_Q, np.arange(B), (n_h, d), 1.0, "bf16"))
        step(o_e, l_e)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), f"replay {rep} differs from eager"
        log(f"replay {rep}: identical to the eager step")
    # and the graph's result against the oracle (last query)
    o_ref, l_ref = _oracle_decode(0, lengths, offs, n_h, n_kv, d, scale, q_seed=13)
    _check(o_g, l_g, o_ref, l_ref, "graph replay vs oracle")
