"""GPU parity: the HIP path through the C ABI against the fp64 oracle, on the same seeded inputs.

Tolerances (max-abs): fp32 inputs 1e-5 on O and LSE; bf16 inputs 2e-2 on O and 1e-3 on LSE.
Rows that saw no key must be O = 0, LSE = -inf on both sides. Small cases compare every element
(several workgroup tiles, ragged chunk lengths); full-size workloads compare sampled rows, each
against the oracle's exact result over its full visible key set.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from ring_cases import device_tensor, log, oracle_view, product_shards, sample_rows, scale_of

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from context_ring_attention_amd import binding
    binding.load()


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what, tol=None):
    tol_o, tol_l = tol or TOL[dtype]
    o_g = o_gpu.float().cpu().numpy().astype(np.float64).reshape(o_ref.shape)
    l_g = lse_gpu.float().cpu().numpy().astype(np.float64).reshape(lse_ref.shape)
    inf_g, inf_r = np.isneginf(l_g), np.isneginf(lse_ref)
    assert np.array_equal(inf_g, inf_r), f"{what}: empty-row pattern differs"
    assert np.all(np.isfinite(o_g)), f"{what}: non-finite output"
    assert np.all(o_g[inf_r] == 0.0), f"{what}: empty rows must be zero"
    err_o = float(np.max(np.abs(o_g - o_ref))) if o_ref.size else 0.0
    fin = ~inf_r
    err_l = float(np.max(np.abs(l_g[fin] - lse_ref[fin]))) if fin.any() else 0.0
    log(f"  {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} rows={lse_ref.size} empty={int(inf_r.sum())}")
    assert err_o <= tol_o and err_l <= tol_l, what


def _oracle_keys(ranges, N, shard_ids, seed, n_kv, d, std, dtype, gen=None):
    ks, vs, sq, ps = [], [], [], []
    for s in shard_ids:
        seq, pos, glob = oracle.shard_tokens(ranges, N, s)
        ks.append(oracle_view(seed, si.TID_K, glob, (n_kv, d), std, dtype, gen))
        vs.append(oracle_view(seed, si.TID_V, glob, (n_kv, d), std, dtype, gen))
        sq.append(seq)
        ps.append(pos)
    return np.concatenate(ks), np.concatenate(vs), np.concatenate(sq), np.concatenate(ps)


def run_pass_kv(seqs, N, n_h, n_kv, d, dtype, seed=0, causal=True, ranks=None, mode="partials",
                check_partials=True, n_sample=None, std=None, gen=None, ws=False):
    from context_ring_attention_amd import binding as cp
    ranges = [(i, 0, L) for i, L in enumerate(seqs)]
    std = std if std is not None else (1.0 / np.sqrt(d) if dtype == "f32" else 1.0)
    scale = scale_of(d)
    ranks = list(range(N)) if ranks is None else ranks
    sh = product_shards(ranges, N)
    for s in sh.values():
        s.k = device_tensor(seed, si.TID_K, s.tokens, (n_kv, d), std, dtype, gen=gen)
        s.v = device_tensor(seed, si.TID_V, s.tokens, (n_kv, d), std, dtype, gen=gen)
    all_keys = _oracle_keys(ranges, N, range(N), seed, n_kv, d, std, dtype, gen)
    for r in ranks:
        log(f"pass-kv seqs={seqs} N={N} rank={r} n_h={n_h} n_kv={n_kv} d={d} {dtype} mode={mode} causal={causal} ws={ws}")
        q = device_tensor(seed, si.TID_Q, sh[r].tokens, (n_h, d), std, dtype, gen=gen)
        tq = q.shape[0]
        o_out = torch.empty(tq, n_h, d, dtype=torch.float32, device="cuda")
        lse_out = torch.empty(tq, n_h, dtype=torch.float32, device="cuda")
        kw = {}
        if mode == "partials":
            kw["o_parts"] = [torch.full((tq, n_h, d), float("nan"), device="cuda") for _ in range(N)]
            kw["lse_parts"] = [torch.empty(tq, n_h, device="cuda") for _ in range(N)]
        elif mode == "running":          # in place, as bench.py runs it
            kw["o_acc"], kw["lse_acc"] = o_out, lse_out
        else:                            # separate running buffers, final copy through the merge
            kw["o_acc"] = torch.empty(tq, n_h, d, device="cuda")
            kw["lse_acc"] = torch.empty(tq, n_h, device="cuda")
        if ws:                           # lets a small Q shard's steps split over their keys
            kw["workspace"] = cp.ring_workspace(tq, n_h, d, partials=int(ws))
        cp.ring_pass_kv(q, sh[r].segs, r, [sh[s].k for s in range(N)], [sh[s].v for s in range(N)],
                        [sh[s].segs for s in range(N)], causal, scale, o_out, lse_out, **kw)
        torch.cuda.synchronize()

        q_seq, q_pos, q_glob = oracle.shard_tokens(ranges, N, r)
        qf = oracle_view(seed, si.TID_Q, q_glob, (n_h, d), std, dtype, gen)
        rows = sample_rows(sh[r].segs, n_sample, seed + r) if n_sample else None
        kf, vf, kseq, kpos = all_keys
        o_ref, l_ref = oracle.attention(qf, kf, vf, n_h, n_kv, q_seq, q_pos, kseq, kpos, causal,
                                        scale, rows=rows)
        sel = slice(None) if rows is None else torch.from_numpy(rows).cuda()
        assert_close(o_out[sel], lse_out[sel], o_ref, l_ref, dtype, f"rank {r} merged")
        if mode == "partials" and check_partials:
            for t in range(N):
                s = oracle.pass_kv_shard(N, r, t)
                kf, vf, kseq, kpos = _oracle_keys(ranges, N, [s], seed, n_kv, d, std, dtype, gen)
                o_p, l_p = oracle.attention(qf, kf, vf, n_h, n_kv, q_seq, q_pos, kseq, kpos, causal,
                                            scale, rows=rows)
                assert_close(kw["o_parts"][t][sel], kw["lse_parts"][t][sel], o_p, l_p, dtype,
                             f"rank {r} step {t} (kv shard {s})")


# --------------------------------------------------------------------------- small, every element
def test_tiny_ring_fp32_all_ranks():
    """The tiny ring: T=256, 4 query heads, 1 KV head, D=64, fp32, CP=4, all partials + merge."""
    run_pass_kv([256], 4, 4, 1, 64, "f32")


def test_tiny_ring_fp32_running_merge():
    run_pass_kv([256], 4, 4, 1, 64, "f32", mode="running")
    run_pass_kv([256], 4, 4, 1, 64, "f32", mode="running_out", ranks=[3])


def test_fp32_ragged_multi_sequence_d128_gqa():
    run_pass_kv([77, 300, 5], 3, 8, 2, 128, "f32", seed=1)


def test_bf16_ring_ragged_two_sequences():
    run_pass_kv([1000, 2333], 4, 16, 1, 128, "bf16", ranks=[0, 3])


def test_bf16_ring_running_merge_bf16_d64_gqa4():
    run_pass_kv([700, 1500], 4, 8, 2, 64, "bf16", seed=2, mode="running", ranks=[1, 2])


def test_bf16_running_mode_steps_split_over_keys():
    """Running-mode steps whose Q tiles cannot fill the CUs split over their keys when a ring
    workspace is given (the second half of every KV run in the workspace, merged in place): ranks
    of an 8192-token-per-rank ring at 4:1 and 2:1 head ratios, causal and not, against the oracle on
    sampled rows; a small ring where no step splits, with the workspace, every element."""
    run_pass_kv([32768], 4, 4, 1, 128, "bf16", mode="running", ranks=[0, 3], ws=True, n_sample=384)
    run_pass_kv([20000, 12768], 4, 2, 1, 64, "bf16", seed=3, mode="running_out", ranks=[1], ws=True,
                n_sample=384)
    run_pass_kv([16384, 16384], 4, 4, 1, 128, "bf16", seed=4, causal=False, mode="running", ranks=[2],
                ws=True, n_sample=384)
    run_pass_kv([700, 1500], 4, 8, 2, 64, "bf16", seed=2, mode="running", ranks=[1], ws=True)
    # 8192 tokens per rank at 1:1 heads (32 Q tiles): up to 4 parts of 2048 keys with 7 partials
    run_pass_kv([32768], 4, 1, 1, 128, "bf16", seed=5, mode="running", ranks=[0, 2], ws=7, n_sample=512)
    run_pass_kv([24000, 8768], 4, 2, 2, 64, "bf16", seed=6, causal=False, mode="running_out", ranks=[3],
                ws=3, n_sample=512)


def test_bf16_degenerate_shapes():
    run_pass_kv([1], 1, 16, 1, 128, "bf16", seed=3)                   # a single token, no ring
    run_pass_kv([3, 9, 1], 2, 4, 4, 64, "bf16", seed=4)               # MHA, empty chunks
    run_pass_kv([500], 2, 2, 1, 128, "bf16", seed=5, causal=False)    # no mask


def test_bf16_d128_several_kv_heads():
    # strided K/V rows (n_kv heads per row) through the per-tile load descriptors
    run_pass_kv([900, 1700], 4, 32, 4, 128, "bf16", seed=6, ranks=[1])   # 8 query heads per KV head
    run_pass_kv([600], 2, 4, 4, 128, "bf16", seed=7, mode="running")    # MHA: 256 tokens per tile


def test_bf16_seed1_second_draw():
    run_pass_kv([2048], 4, 16, 1, 128, "bf16", seed=1, ranks=[2], check_partials=False)


# --------------------------------------------------------------------------- Pass-Q
def run_pass_q(P, T, N, n_h, n_kv, d, dtype="bf16", seed=0, n_sample=None, check_partials=True):
    """Pass-Q over persistent KV: sequence i has P[i] cached and T[i] new tokens (scalars: one
    sequence)."""
    from context_ring_attention_amd import binding as cp
    std = 1.0
    scale = scale_of(d)
    Ps = P if isinstance(P, (list, tuple)) else [P]
    Ts = T if isinstance(T, (list, tuple)) else [T]
    q_ranges = [(i, p, p + t) for i, (p, t) in enumerate(zip(Ps, Ts))]
    kv_ranges = [r for i, (p, t) in enumerate(zip(Ps, Ts)) for r in ((i, 0, p), (i, p, p + t))]
    qsh = product_shards(q_ranges, N)
    ksh = product_shards(kv_ranges, N)
    for s in ksh.values():
        s.k = device_tensor(seed, si.TID_K, s.tokens, (n_kv, d), std, dtype)
        s.v = device_tensor(seed, si.TID_V, s.tokens, (n_kv, d), std, dtype)
    qs = [device_tensor(seed, si.TID_Q, qsh[r].tokens, (n_h, d), std, dtype) for r in range(N)]
    log(f"pass-q P={P} T={T} N={N} n_h={n_h} d={d}")
    o_parts = [torch.full((qs[i // N].shape[0], n_h, d), float("nan"), device="cuda") for i in range(N * N)]
    lse_parts = [torch.empty(qs[i // N].shape[0], n_h, device="cuda") for i in range(N * N)]
    o_out = [torch.empty(x.shape[0], n_h, d, device="cuda") for x in qs]
    lse_out = [torch.empty(x.shape[0], n_h, device="cuda") for x in qs]
    cp.ring_pass_q(qs, [qsh[r].segs for r in range(N)], [ksh[s].k for s in range(N)],
                   [ksh[s].v for s in range(N)], [ksh[s].segs for s in range(N)], True, scale,
                   o_parts, lse_parts, o_out, lse_out)
    torch.cuda.synchronize()
    kf, vf, kseq, kpos = _oracle_keys(kv_ranges, N, range(N), seed, n_kv, d, std, dtype)
    for qi in range(N):
        q_seq, q_pos, q_glob = oracle.shard_tokens(q_ranges, N, qi)
        qf = oracle_view(seed, si.TID_Q, q_glob, (n_h, d), std, dtype)
        rows = sample_rows(qsh[qi].segs, n_sample, seed + qi) if n_sample else None
        sel = slice(None) if rows is None else torch.from_numpy(rows).cuda()
        o_ref, l_ref = oracle.attention(qf, kf, vf, n_h, n_kv, q_seq, q_pos, kseq, kpos, True, scale,
                                        rows=rows)
        assert_close(o_out[qi][sel], lse_out[qi][sel], o_ref, l_ref, dtype, f"q shard {qi} merged")
        if check_partials:
            # every slot: the partial of Q shard qi against KV shard s, wherever the ring put it
            for s in range(N):
                kf1, vf1, ks1, kp1 = _oracle_keys(kv_ranges, N, [s], seed, n_kv, d, std, dtype)
                o_p, l_p = oracle.attention(qf, kf1, vf1, n_h, n_kv, q_seq, q_pos, ks1, kp1, True,
                                            scale, rows=rows)
                slot = oracle.pass_q_slot(N, qi, s)
                assert_close(o_parts[slot][sel], lse_parts[slot][sel], o_p, l_p, dtype,
                             f"slot {slot} = (q shard {qi}, kv shard {s})")


def test_pass_q_persistent_kv_small():
    run_pass_q(P=3000, T=520, N=4, n_h=16, n_kv=1, d=128)


def test_pass_q_varlen_cp8_split_launches():
    # 8 ranks, 5 sequences: each KV shard has 20 runs, so a ring step's 8 partials need several
    # launches (at most 64 pooled runs each)
    run_pass_q(P=[300, 41, 700, 0, 129], T=[64, 200, 17, 90, 1], N=8, n_h=8, n_kv=2, d=64)


# --------------------------------------------------------------------------- merge kernel
@pytest.mark.parametrize("n_parts,rows,d,out", [(1, 37, 64, "f32"), (3, 1000, 128, "f32"),
                                                (17, 513, 128, "bf16"), (64, 129, 64, "bf16")])
def test_merge_lse_against_oracle(n_parts, rows, d, out):
    from context_ring_attention_amd import binding as cp
    log(f"merge n_parts={n_parts} rows={rows} d={d} out={out}")
    o, lse = si.random_partials(7 + n_parts, n_parts, rows, d)
    o_dev = [o[i].contiguous().cuda() for i in range(n_parts)]
    l_dev = [lse[i].contiguous().cuda() for i in range(n_parts)]
    o_out = torch.empty(rows, d, dtype=torch.bfloat16 if out == "bf16" else torch.float32, device="cuda")
    l_out = torch.empty(rows, device="cuda")
    cp.merge_lse(o_dev, l_dev, o_out, l_out)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge([o[i].double().numpy() for i in range(n_parts)],
                                [lse[i].double().numpy() for i in range(n_parts)])
    tol = 2e-2 if out == "bf16" else 1e-5
    o_g = o_out.float().cpu().numpy()
    l_g = l_out.cpu().numpy()
    assert np.array_equal(np.isneginf(l_g), np.isneginf(l_ref))
    fin = np.isfinite(l_ref)
    assert np.max(np.abs(o_g - o_ref)) <= tol
    assert np.max(np.abs(l_g[fin] - l_ref[fin])) <= 1e-5
    assert np.all(o_g[~fin] == 0)


def test_merge_in_place_fp32():
    from context_ring_attention_amd import binding as cp
    o, lse = si.random_partials(3, 4, 300, 128)
    o_dev = [o[i].contiguous().cuda() for i in range(4)]
    l_dev = [lse[i].contiguous().cuda() for i in range(4)]
    cp.merge_lse(o_dev, l_dev, o_dev[0], l_dev[0])   # O and LSE both merged in place
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge([o[i].double().numpy() for i in range(4)], [lse[i].double().numpy() for i in range(4)])
    assert np.max(np.abs(o_dev[0].cpu().numpy() - o_ref)) <= 1e-5
    l_g = l_dev[0].cpu().numpy()
    assert np.array_equal(np.isneginf(l_g), np.isneginf(l_ref))
    fin = np.isfinite(l_ref)
    assert np.max(np.abs(l_g[fin] - l_ref[fin])) <= 1e-5


# --------------------------------------------------------------------------- decode
def run_decode(lengths, n_h, n_kv, d, n_splits, seed=0, out="f32", check_splits=None, ws="f32",
               std=1.0, gen=None, tol_scale=1.0):
    """Split-KV decode through the C ABI against the oracle: every request's merged (O, LSE), and
    the split partials listed in check_splits. ws: workspace precision of the partial O ("f32",
    cp_decode_splitkv; "bf16", cp_decode_splitkv_ex). tol_scale widens the O bound for inputs
    whose values are tol_scale times larger than N(0,1) (the bound is relative to |V|)."""
    from context_ring_attention_amd import binding as cp
    lengths = np.asarray(lengths, np.int64)
    B = len(lengths)
    offs = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    total = int(lengths.sum())
    log(f"decode B={B} n_splits={n_splits} total_keys={total} n_h={n_h} n_kv={n_kv} d={d} ws={ws}")
    scale = scale_of(d)
    toks = np.arange(total)
    kc = device_tensor(seed, si.TID_K, toks, (n_kv, d), std, "bf16", gen=gen)
    vc = device_tensor(seed, si.TID_V, toks, (n_kv, d), std, "bf16", gen=gen)
    q = device_tensor(seed, si.TID_Q, np.arange(B), (n_h, d), std, "bf16", gen=gen)
    ws_o, ws_l = cp.decode_workspace(B, n_h, d, n_splits, ws_dtype=ws)
    o_out = torch.empty(B, n_h, d, dtype=torch.bfloat16 if out == "bf16" else torch.float32, device="cuda")
    l_out = torch.empty(B, n_h, device="cuda")
    cp.decode_splitkv(q, kc, vc, torch.from_numpy(offs).cuda(), torch.from_numpy(lengths).cuda(),
                      n_splits, scale, ws_o, ws_l, o_out, l_out)
    torch.cuda.synchronize()
    qf = oracle_view(seed, si.TID_Q, np.arange(B), (n_h, d), std, "bf16", gen)
    tol = (TOL["bf16"][0] * tol_scale, TOL["bf16"][1])
    for b in range(B):
        lo, L = int(offs[b]), int(lengths[b])
        kf = oracle_view(seed, si.TID_K, np.arange(lo, lo + L), (n_kv, d), std, "bf16", gen)
        vf = oracle_view(seed, si.TID_V, np.arange(lo, lo + L), (n_kv, d), std, "bf16", gen)
        qs_ = np.zeros(1, np.int32)
        qp_ = np.array([L], np.int64)
        o_ref, l_ref = oracle.attention(qf[b:b + 1], kf, vf, n_h, n_kv, qs_, qp_, np.zeros(L, np.int32),
                                        np.arange(L), False, scale)
        assert_close(o_out[b:b + 1], l_out[b:b + 1], o_ref, l_ref, "bf16", f"request {b} (L={L})", tol)
        splits = oracle.split_bounds(L, n_splits)
        for c in (check_splits or []):
            a, e = splits[c]
            o_p, l_p = oracle.attention(qf[b:b + 1], kf[a:e], vf[a:e], n_h, n_kv, qs_, qp_,
                                        np.zeros(e - a, np.int32), np.arange(a, e), False, scale)
            assert_close(ws_o[b, c], ws_l[b, c], o_p, l_p, "bf16", f"request {b} split {c}", tol)


@pytest.mark.parametrize("ws", ["f32", "bf16"])
def test_decode_small_ragged(ws):
    run_decode([3000, 1, 100, 4097, 257], 16, 1, 128, 256, check_splits=[0, 1, 99, 255], ws=ws)


def test_decode_empty_requests_four_waves_per_split():
    # small grid: four waves share each split; requests with no cached key give O = 0, LSE = -inf
    run_decode([0, 37, 0, 2000, 5], 16, 1, 128, 256, seed=4, check_splits=[0, 128, 255])
    run_decode([0, 37, 0, 2000, 5], 16, 1, 128, 256, seed=4, check_splits=[0, 128, 255], ws="bf16")


def test_decode_one_wave_per_split_with_empty_splits():
    # 8 requests x 256 splits = 2048 workgroups: one wave per split; short requests leave most
    # splits empty
    run_decode([0, 1, 255, 256, 257, 1000, 3, 700], 16, 1, 128, 256, seed=5, check_splits=[0, 1, 200, 255])


def test_decode_gqa_d64_bf16_out():
    run_decode([999, 64, 2500], 8, 2, 64, 16, seed=1, out="bf16", check_splits=[0, 15])
    run_decode([999, 64, 2500], 8, 2, 64, 16, seed=1, out="bf16", check_splits=[0, 15], ws="bf16")


def test_decode_more_than_16_heads_per_group():
    run_decode([700, 33], 40, 2, 128, 8, seed=2, check_splits=[3])


def test_decode_batch_over_64():
    # more requests than the kernel ranks by length: units are then taken in request order
    lens = [int(x) for x in np.random.default_rng(7).integers(1, 300, size=70)]
    run_decode(lens, 8, 1, 64, 4, seed=3, check_splits=[0, 3])


def test_decode_large_grids_with_empty_splits():
    """Grids of several rounds of one-wave workgroups: 80 requests (above 64, so taken in request
    order) with 20 heads per KV head (two head blocks), and 40 ranked requests at 256 splits, both
    with empty splits; D_H 128 and 64, fp32 and bf16 workspaces."""
    lens = [int(x) for x in np.random.default_rng(16).integers(0, 400, size=80)]
    run_decode(lens, 40, 2, 128, 32, seed=16, check_splits=[0, 17, 31])
    lens = [int(x) for x in np.random.default_rng(17).integers(0, 3000, size=40)]
    run_decode(lens, 16, 1, 128, 256, seed=17, check_splits=[0, 1, 128, 255])
    run_decode(lens, 16, 1, 64, 256, seed=17, check_splits=[0, 255], ws="bf16")


# --------------------------------------------------------------------------- table and split limits
def test_bf16_full_segment_tables():
    # 32 ragged sequences at CP = 1: each owns 2 chunks, so the Q and KV tables hold 64 runs each,
    # the most one call accepts
    lens = [int(x) for x in np.random.default_rng(12).integers(2, 150, size=32)]
    run_pass_kv(lens, 1, 16, 1, 128, "bf16", seed=6, mode="partials")


def test_decode_most_splits_and_a_single_split():
    # 1024 splits (the limit): most splits of the short requests are empty; then one split, where
    # the merge of a single partial must return it unchanged
    run_decode([5000, 1023, 1, 2048], 16, 1, 128, 1024, seed=8, check_splits=[0, 1, 511, 1023])
    run_decode([3000, 1, 777], 8, 1, 64, 1, seed=9, check_splits=[0])


def test_decode_negative_length_reads_as_empty():
    from context_ring_attention_amd import binding as cp
    n_h, d, S, L = 16, 128, 256, 300
    toks = np.arange(L)
    kc = device_tensor(10, si.TID_K, toks, (1, d), 1.0, "bf16")
    vc = device_tensor(10, si.TID_V, toks, (1, d), 1.0, "bf16")
    q = device_tensor(10, si.TID_Q, np.arange(2), (n_h, d), 1.0, "bf16")
    offs = torch.tensor([0, 0], dtype=torch.int64, device="cuda")
    lens = torch.tensor([-7, L], dtype=torch.int64, device="cuda")
    ws_o, ws_l = cp.decode_workspace(2, n_h, d, S)
    o = torch.full((2, n_h, d), float("nan"), device="cuda")
    lse = torch.empty(2, n_h, device="cuda")
    cp.decode_splitkv(q, kc, vc, offs, lens, S, scale_of(d), ws_o, ws_l, o, lse)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    qf = oracle_view(10, si.TID_Q, np.arange(2), (n_h, d), 1.0, "bf16")
    kf = oracle_view(10, si.TID_K, toks, (1, d), 1.0, "bf16")
    vf = oracle_view(10, si.TID_V, toks, (1, d), 1.0, "bf16")
    o_ref, l_ref = oracle.attention(qf[1:2], kf, vf, n_h, 1, np.zeros(1, np.int32), np.array([L]),
                                    np.zeros(L, np.int32), np.arange(L), False, scale_of(d))
    assert_close(o[1:2], lse[1:2], o_ref, l_ref, "bf16", "request after an empty one")


def test_bf16_group_sizes_that_straddle_tiles():
    # row = token * G + head: with G = 3 or 5 a 256-row workgroup tile starts and ends inside a
    # token's heads; G = 32 puts 8 tokens in a tile
    run_pass_kv([700, 333], 2, 21, 7, 128, "bf16", seed=11, mode="partials")
    run_pass_kv([900], 3, 10, 2, 64, "bf16", seed=12, mode="running", ranks=[1])
    run_pass_kv([513, 64], 2, 64, 2, 128, "bf16", seed=13, mode="partials", ranks=[0])


def test_decode_group_sizes_that_straddle_head_blocks():
    run_decode([1500, 37, 0], 21, 7, 128, 256, seed=14, check_splits=[0, 255])
    run_decode([800, 2049], 10, 2, 64, 32, seed=15, out="bf16", check_splits=[5])


# Shapes whose (request, split, head block) units number 4 to 8 per SIMD of a 256-CU device take
# the persistent split kernel (one wave per SIMD walking several units, partials stored at its end).
@pytest.mark.parametrize("ws", ["f32", "bf16"])
def test_decode_persistent_walkers_ragged(ws):
    # 16 requests x 256 splits: 4 units per wave; empty requests, requests shorter than the split
    # count (empty splits) and lengths that do not divide
    lens = [0, 1, 255, 257, 3000, 40000, 12345, 0, 999, 65536, 31, 5000, 20000, 2, 777, 100000]
    run_decode(lens, 16, 1, 128, 256, seed=21, check_splits=[0, 1, 128, 255], ws=ws)


def test_decode_persistent_walkers_d64_head_blocks_and_kv_heads():
    # D_H 64, 16 requests x 512 splits: 8 units per wave
    lens = [int(x) for x in np.random.default_rng(22).integers(0, 20000, size=16)]
    run_decode(lens, 8, 1, 64, 512, seed=22, check_splits=[0, 511], out="bf16")
    # two head blocks per KV head (20 query heads per KV head): 4 units per wave
    run_decode([3000, 0, 777, 12000, 64, 5000, 1, 9000], 20, 1, 128, 256, seed=23, check_splits=[0, 255])
    # two KV heads of 8 query heads each: 4 units per wave
    run_decode([2500, 1, 0, 7000, 300, 4096, 4097, 60], 16, 2, 128, 256, seed=24, check_splits=[7, 200])
    # 64 requests: two rounds of waves with 8 units each
    lens = [int(x) for x in np.random.default_rng(26).integers(0, 3000, size=64)]
    run_decode(lens, 16, 1, 128, 256, seed=26, check_splits=[0, 255])


@pytest.mark.parametrize("ws", ["f32", "bf16"])
@pytest.mark.parametrize("n_sub", [32, 48, 64])
def test_decode_persistent_walkers_equal_one_wave_splits_bitwise(ws, n_sub):
    """The persistent walkers run each split as the one-wave kernel does, so their partials and
    merged results are bit-identical: n_sub requests x 256 splits (32: one round of waves with 8
    units each; 48 and 64: two rounds with 6 and 8) against the same requests inside a
    65-request call (over 64 requests: one wave per split)."""
    from context_ring_attention_amd import binding as cp
    rng = np.random.default_rng(25)
    lens65 = rng.integers(0, 6000, size=65).astype(np.int64)
    lens65[[3, 17]] = 0
    d, n_h, S = 128, 16, 256
    res = []
    for lens in (lens65[:n_sub], lens65):
        B = len(lens)
        offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        toks = np.arange(int(lens.sum()))
        kc = device_tensor(25, si.TID_K, toks, (1, d), 1.0, "bf16")
        vc = device_tensor(25, si.TID_V, toks, (1, d), 1.0, "bf16")
        q = device_tensor(25, si.TID_Q, np.arange(B), (n_h, d), 1.0, "bf16")
        ws_o, ws_l = cp.decode_workspace(B, n_h, d, S, ws_dtype=ws)
        o = torch.empty(B, n_h, d, device="cuda")
        l = torch.empty(B, n_h, device="cuda")
        log(f"decode B={B} n_splits={S} ws={ws} (bitwise comparison of the two split kernels)")
        cp.decode_splitkv(q, kc, vc, torch.from_numpy(offs).cuda(), torch.from_numpy(lens).cuda(), S,
                          scale_of(d), ws_o, ws_l, o, l)
        torch.cuda.synchronize()
        res.append((ws_o[:n_sub].clone(), ws_l[:n_sub].clone(), o[:n_sub].clone(), l[:n_sub].clone()))
    for a, b, what in zip(res[0], res[1], ("split O", "split LSE", "O", "LSE")):
        assert torch.equal(a, b), f"{what} differs between the persistent and one-wave split kernels"
