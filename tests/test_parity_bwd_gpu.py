"""GPU parity of the backward (cp_ring_pass_kv_bwd, cp_partial_attn_bwd) against the fp64 oracle,
element by element.

In context parallelism each rank sends the K/V gradient contributions of its Q shard back to the
owners of the KV shards, a reduce-scatter ("Context Parallelism과 Expert Parallelism", §6). On one
device every rank's ring backward adds into per-shard dK/dV accumulators, so after all ranks ran
they must equal the oracle's gradient of the whole attention restricted to each shard's keys,
and every rank's dQ the gradient of its rows. Both sides take the same saved forward results: the
oracle's forward output and LSE rounded to fp32.

Bound (derived in the design notes): for bf16 inputs the products run on bf16 MFMA with fp32
accumulation, and the probabilities P and score gradients dS are rounded to bf16 (at most 2^-8
relative each) as MFMA operands, so each gradient element may differ from the exact value by a small
fraction of the largest element of its tensor: max|err| <= 1e-2 * max|ref| + 1e-3. fp32 inputs run
in fp32 throughout: max|err| <= 1e-5 * max(1, max|ref|).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from ring_cases import Planted, device_tensor, log, oracle_view, product_shards, scale_of

pytestmark = pytest.mark.gpu

BOUND = {"bf16": (1e-2, 1e-3), "f32": (1e-5, 1e-5)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(gpu, ref, what, dtype="bf16"):
    rel, tol_abs = BOUND[dtype]
    g = gpu.float().cpu().numpy().astype(np.float64).reshape(ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    err = float(np.max(np.abs(g - ref))) if ref.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    log(f"  {what}: max|err|={err:.3e} max|ref|={scale:.3e} rel={err / max(scale, 1e-30):.2e}")
    bound = rel * scale + tol_abs if dtype == "bf16" else rel * max(1.0, scale)
    assert err <= bound, what


_WS = {}


def workspace(d, nbytes=None):
    """The backward workspace (one per head dimension, shared by the tests), or its first nbytes."""
    from context_ring_attention_amd import binding as cp
    if d not in _WS:
        _WS[d] = cp.attn_bwd_workspace(d)
    return _WS[d] if nbytes is None else _WS[d][:nbytes]


def run_bwd(seqs, N, n_h, n_kv, d, seed=0, causal=True, gen=None, step_check=None, dtype="bf16",
            ws=True, ws_bytes=None):
    """ws: give the calls the backward workspace (so the dK/dV work of small launches is split
    over several workgroups per key tile), ws_bytes: only that much of it (fewer parts)."""
    from context_ring_attention_amd import binding as cp
    wsp = workspace(d, ws_bytes) if ws else None
    ranges = [(i, 0, L) for i, L in enumerate(seqs)]
    scale = scale_of(d)
    std = 1.0 / np.sqrt(d) if dtype == "f32" else 1.0
    log(f"bwd seqs={seqs[:8]}{'...' if len(seqs) > 8 else ''} N={N} n_h={n_h} n_kv={n_kv} d={d} "
        f"causal={causal} {dtype} workspace={'none' if wsp is None else wsp.numel()}")
    sh = product_shards(ranges, N)
    # oracle side: the whole batch in global token order
    T = int(sum(seqs))
    g_all = np.arange(T)
    seq_all = np.concatenate([np.full(L, i, np.int32) for i, L in enumerate(seqs)])
    pos_all = np.concatenate([np.arange(L, dtype=np.int64) for L in seqs])
    qf = oracle_view(seed, si.TID_Q, g_all, (n_h, d), std, dtype, gen)
    kf = oracle_view(seed, si.TID_K, g_all, (n_kv, d), std, dtype, gen)
    vf = oracle_view(seed, si.TID_V, g_all, (n_kv, d), std, dtype, gen)
    gf = oracle_view(seed, si.TID_DO, g_all, (n_h, d), 1.0, dtype)
    o_ref, l_ref = oracle.attention(qf, kf, vf, n_h, n_kv, seq_all, pos_all, seq_all, pos_all, causal, scale)
    o32, l32 = o_ref.astype(np.float32), l_ref.astype(np.float32)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(qf, kf, vf, n_h, n_kv, seq_all, pos_all, seq_all,
                                                       pos_all, causal, scale, o32, l32, gf)
    # device side: every rank's ring backward, dK/dV summed per shard
    ks = [device_tensor(seed, si.TID_K, sh[s].tokens, (n_kv, d), std, dtype, gen=gen) for s in range(N)]
    vs = [device_tensor(seed, si.TID_V, sh[s].tokens, (n_kv, d), std, dtype, gen=gen) for s in range(N)]
    dks = [torch.zeros(k.shape, device="cuda") for k in ks]
    dvs = [torch.zeros(k.shape, device="cuda") for k in ks]
    kv_segs = [sh[s].segs for s in range(N)]
    dqs = {}
    for r in range(N):
        toks = sh[r].tokens
        q = device_tensor(seed, si.TID_Q, toks, (n_h, d), std, dtype, gen=gen)
        d_o = device_tensor(seed, si.TID_DO, toks, (n_h, d), 1.0, dtype)
        o = torch.from_numpy(o32[toks]).cuda()
        lse = torch.from_numpy(l32[toks]).cuda()
        delta = torch.empty(len(toks), n_h, device="cuda")
        dq = torch.zeros(len(toks), n_h, d, device="cuda")
        cp.ring_pass_kv_bwd(q, sh[r].segs, r, ks, vs, kv_segs, causal, scale, o, lse, d_o, delta, dq, dks, dvs,
                            workspace=wsp)
        dqs[r] = dq
        if step_check is not None and r == step_check[0]:
            # one ring step alone against the oracle's partial backward over that shard's keys
            t = step_check[1]
            s = oracle.pass_kv_shard(N, r, t)
            dq1 = torch.zeros_like(dq)
            dk1 = torch.zeros_like(dks[s])
            dv1 = torch.zeros_like(dvs[s])
            cp.partial_attn_bwd(q, ks[s], vs[s], sh[r].segs, sh[s].segs, causal, scale, lse, delta, d_o,
                                dq1, dk1, dv1, workspace=wsp)
            torch.cuda.synchronize()
            kt = sh[s].tokens
            p_dq, p_dk, p_dv = oracle.attention_backward(
                qf[toks], kf[kt], vf[kt], n_h, n_kv, seq_all[toks], pos_all[toks], seq_all[kt],
                pos_all[kt], causal, scale, o32[toks], l32[toks], gf[toks])
            _check(dq1, p_dq, f"rank {r} step {t} dQ", dtype)
            _check(dk1, p_dk, f"rank {r} step {t} dK (shard {s})", dtype)
            _check(dv1, p_dv, f"rank {r} step {t} dV (shard {s})", dtype)
    torch.cuda.synchronize()
    for r in range(N):
        _check(dqs[r], dq_ref[sh[r].tokens], f"rank {r} dQ", dtype)
    for s in range(N):
        _check(dks[s], dk_ref[sh[s].tokens], f"shard {s} dK (all ranks)", dtype)
        _check(dvs[s], dv_ref[sh[s].tokens], f"shard {s} dV (all ranks)", dtype)


def test_bwd_ring_cp4_two_sequences():
    run_bwd([700, 1300], 4, 16, 1, 128, seed=51, step_check=(1, 2))


def test_bwd_without_workspace_and_with_a_small_one():
    """No workspace: one workgroup per key tile. A workspace of 3 slots per tile: 3 parts."""
    run_bwd([700, 1300], 4, 16, 1, 128, seed=51, step_check=(1, 2), ws=False)
    slot = 128 * 128 * 4 * 2
    run_bwd([1500], 2, 16, 1, 128, seed=64, step_check=(0, 1), ws_bytes=3 * 6 * slot)
    run_bwd([333, 64], 2, 8, 2, 64, seed=65, ws=False)


def test_bwd_split_is_deterministic():
    """Two calls with the same workspace add bit-identical contributions."""
    from context_ring_attention_amd import binding as cp
    seqs, N, n_h, n_kv, d = [1200], 2, 16, 1, 128
    sh = product_shards([(0, 0, seqs[0])], N)
    std, scale = 1.0, scale_of(d)
    r, s = 0, 1
    q = device_tensor(70, si.TID_Q, sh[r].tokens, (n_h, d), std, "bf16")
    d_o = device_tensor(70, si.TID_DO, sh[r].tokens, (n_h, d), 1.0, "bf16")
    k = device_tensor(70, si.TID_K, sh[s].tokens, (n_kv, d), std, "bf16")
    v = device_tensor(70, si.TID_V, sh[s].tokens, (n_kv, d), std, "bf16")
    lse = torch.full((len(sh[r].tokens), n_h), 3.0, device="cuda")
    delta = torch.full((len(sh[r].tokens), n_h), 0.25, device="cuda")
    outs = []
    for _ in range(2):
        dq = torch.zeros(len(sh[r].tokens), n_h, d, device="cuda")
        dk = torch.zeros(k.shape, device="cuda")
        dv = torch.zeros(k.shape, device="cuda")
        cp.partial_attn_bwd(q, k, v, sh[r].segs, sh[s].segs, True, scale, lse, delta, d_o, dq, dk, dv,
                            workspace=workspace(d))
        outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_bwd_gqa_d64():
    run_bwd([500, 333], 2, 8, 2, 64, seed=52, step_check=(0, 1))


def test_bwd_without_causal_mask():
    run_bwd([600, 90], 2, 16, 1, 128, seed=53, causal=False, step_check=(1, 0))


def test_bwd_degenerate_shapes():
    run_bwd([1], 1, 16, 1, 128, seed=54)              # one token: dS = 0, dV = dO
    run_bwd([3, 9, 1], 2, 4, 4, 64, seed=55)          # MHA, empty chunks
    run_bwd([129, 257], 3, 16, 1, 128, seed=56)       # ragged tiles of 128 keys / 256 rows


def test_bwd_group_sizes_that_straddle_tiles():
    run_bwd([700, 333], 2, 21, 7, 128, seed=57)
    run_bwd([900], 3, 10, 2, 64, seed=58)


def test_bwd_wide_scores():
    run_bwd([800, 500], 2, 16, 1, 128, seed=59, gen=Planted(q_std=3.0, k_std=3.0))


def test_bwd_many_sequences_split_over_launches():
    lens = [int(x) for x in np.random.default_rng(60).integers(1, 60, size=70)]
    run_bwd(lens, 2, 16, 1, 128, seed=60)


def test_bwd_tiny_ring_fp32():
    """The tiny fp32 ring's backward: T=256, 4 query heads, 1 KV head, D=64, CP=4."""
    run_bwd([256], 4, 4, 1, 64, seed=61, step_check=(2, 1), dtype="f32")


def test_bwd_fp32_ragged_gqa_d128():
    run_bwd([77, 300, 5], 3, 8, 2, 128, seed=62, dtype="f32")
    run_bwd([200], 2, 4, 4, 64, seed=63, causal=False, dtype="f32")
