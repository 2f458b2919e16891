"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Each output row checked is compared with the oracle's exact result over the row's full visible
key set; rows are sampled (first, middle and last token of every chunk plus random tokens, all
query heads of each: at least 32 tokens, 512 (token, head) rows, per rank), since the oracle
cannot redo 10-200 TFLOP of attention.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from ring_cases import device_tensor, log, oracle_view, product_shards, sample_rows, scale_of
from test_parity_gpu import assert_close, run_pass_kv, run_pass_q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_full_prefill_128k_cp4_all_ranks_running():
    cfg = si.CONFIGS["prefill_128k_cp4"]
    run_pass_kv(cfg["seqs"], cfg["cp"], cfg["n_h"], cfg["n_kv"], cfg["d_h"], "bf16", seed=0,
                mode="running", n_sample=28)


def test_full_prefill_128k_cp4_partials_seed1():
    cfg = si.CONFIGS["prefill_128k_cp4"]
    run_pass_kv(cfg["seqs"], cfg["cp"], cfg["n_h"], cfg["n_kv"], cfg["d_h"], "bf16", seed=1,
                mode="partials", ranks=[1], n_sample=28, check_partials=True)


def test_full_persistent_kv_pass_q():
    cfg = si.CONFIGS["persistent_kv_8k_on_120k"]
    run_pass_q(cfg["cached"], cfg["new"], cfg["cp"], cfg["n_h"], cfg["n_kv"], cfg["d_h"],
               n_sample=28, check_partials=True)


def test_full_prefill_1m_varlen_cp8():
    cfg = si.CONFIGS["prefill_1m_varlen_cp8"]
    run_pass_kv(cfg["seqs"], cfg["cp"], cfg["n_h"], cfg["n_kv"], cfg["d_h"], "bf16", seed=0,
                mode="running", ranks=[0, 7], n_sample=10)


@pytest.fixture(scope="module")
def decode_b32():
    """The B=32, 256-split decode workload on the device (cache, queries, offsets, lengths), and a
    second V cache with values 8 times larger."""
    cfg = si.CONFIGS["decode_b32_32k_128k"]
    B, n_h, n_kv, d = cfg["batch"], cfg["n_h"], cfg["n_kv"], cfg["d_h"]
    lens = si.decode_lengths(0, B, cfg["len_lo"], cfg["len_hi"])
    assert lens.min() >= cfg["len_lo"] and lens.max() <= cfg["len_hi"]
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    total = int(lens.sum())
    log(f"decode full: B={B} total keys {total}")
    toks = np.arange(total)
    dev = dict(kc=device_tensor(0, si.TID_K, toks, (n_kv, d), 1.0, "bf16"),
               vc=device_tensor(0, si.TID_V, toks, (n_kv, d), 1.0, "bf16"),
               vc8=device_tensor(0, si.TID_V, toks, (n_kv, d), 8.0, "bf16"),
               q=device_tensor(0, si.TID_Q, np.arange(B), (n_h, d), 1.0, "bf16"),
               offs=torch.from_numpy(offs).cuda(), lens=torch.from_numpy(lens).cuda())
    return cfg, lens, offs, dev


@pytest.mark.parametrize("ws,v_std", [("f32", 1.0), ("bf16", 1.0), ("f32", 8.0), ("bf16", 8.0)])
def test_full_decode_b32_256_splits(decode_b32, ws, v_std):
    """Every request's merged output and chosen split partials, in the launch configuration the
    bench times, for both workspace precisions; V = 8 N(0,1) checks the bound relative to |V|."""
    from context_ring_attention_amd import binding as cp
    cfg, lens, offs, dev = decode_b32
    B, n_h, n_kv, d, S = cfg["batch"], cfg["n_h"], cfg["n_kv"], cfg["d_h"], cfg["n_splits"]
    ws_o, ws_l = cp.decode_workspace(B, n_h, d, S, ws_dtype=ws)
    o = torch.empty(B, n_h, d, device="cuda")
    l = torch.empty(B, n_h, device="cuda")
    scale = scale_of(d)
    vc = dev["vc8"] if v_std != 1.0 else dev["vc"]
    log(f"decode full ws={ws} v_std={v_std}")
    cp.decode_splitkv(dev["q"], dev["kc"], vc, dev["offs"], dev["lens"], S, scale, ws_o, ws_l, o, l)
    torch.cuda.synchronize()
    tol = (2e-2 * v_std, 1e-3)
    qf = oracle_view(0, si.TID_Q, np.arange(B), (n_h, d), 1.0, "bf16")
    rng = np.random.default_rng(0)
    worst = 0.0
    for b in range(B):
        lo, L = int(offs[b]), int(lens[b])
        kf = oracle_view(0, si.TID_K, np.arange(lo, lo + L), (n_kv, d), 1.0, "bf16")
        vf = oracle_view(0, si.TID_V, np.arange(lo, lo + L), (n_kv, d), v_std, "bf16")
        zs = np.zeros(1, np.int32)
        qp = np.array([L], np.int64)
        kseq = np.zeros(L, np.int32)
        kpos = np.arange(L)
        o_ref, l_ref = oracle.attention(qf[b:b + 1], kf, vf, n_h, n_kv, zs, qp, kseq, kpos, False, scale)
        assert_close(o[b:b + 1], l[b:b + 1], o_ref, l_ref, "bf16", f"request {b} (L={L})", tol)
        worst = max(worst, float(np.max(np.abs(o[b:b + 1].cpu().numpy() - o_ref))))
        if b % 8 == 0:
            bounds = oracle.split_bounds(L, S)
            for c in (0, int(rng.integers(1, S - 1)), S - 1):
                a, e = bounds[c]
                o_p, l_p = oracle.attention(qf[b:b + 1], kf[a:e], vf[a:e], n_h, n_kv, zs, qp,
                                            kseq[a:e], kpos[a:e], False, scale)
                assert_close(ws_o[b, c], ws_l[b, c], o_p, l_p, "bf16", f"request {b} split {c}", tol)
    log(f"decode full ws={ws} v_std={v_std}: worst max|dO| over requests {worst:.3e}")
