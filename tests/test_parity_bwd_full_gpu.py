"""GPU parity of the ring backward at the full 128K-token CP 4 size, in the launch configuration
bench.py times (every rank's cp_ring_pass_kv_bwd with the backward workspace), on sampled
outputs the oracle computes one by one.

The backward of a ring step is a function of Q, K, V, dO and the saved forward results (O, LSE)
("Context Parallelism과 Expert Parallelism", §6: the K/V gradients go back to the owners of the
K/V chunks, a sum per chunk). The oracle cannot redo the 70 TFLOP forward that would give every
row's O and LSE, so both sides take the same seeded saved activations instead: O ~ N(0, 0.3^2)
and LSE = ln(visible keys) + 0.5 + 0.1 N(0, 1), so that the probabilities exp(s - LSE) of a row sum
to about one as in a real backward. Compared:
  - dQ of sampled rows (first and last token of every chunk of rank 0 plus random tokens, all 16
    heads): the oracle's gradient of those rows over their whole visible key set;
  - dK and dV of sampled keys of every KV shard (first and last key of every chunk plus random
    keys), summed over all four ranks' ring steps: the oracle's gradient of those keys over every
    query row of the sequence.
Bound as in test_parity_bwd_gpu: max|err| <= 1e-2 * max|ref| + 1e-3 per tensor.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from ring_cases import device_tensor, log, oracle_view, product_shards, sample_rows, scale_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(gpu, ref, what):
    g = np.asarray(gpu, np.float64).reshape(ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    err = float(np.max(np.abs(g - ref)))
    scale = float(np.max(np.abs(ref)))
    log(f"  {what}: max|err|={err:.3e} max|ref|={scale:.3e} rel={err / max(scale, 1e-30):.2e}")
    assert err <= 1e-2 * scale + 1e-3, what


def test_full_backward_128k_cp4_sampled():
    from context_ring_attention_amd import binding as cp
    cfg = si.CONFIGS["prefill_128k_cp4"]
    N, n_h, n_kv, d = cfg["cp"], cfg["n_h"], cfg["n_kv"], cfg["d_h"]
    T = cfg["seqs"][0]
    seed, scale = 3, scale_of(d)
    sh = product_shards([(0, 0, T)], N)
    g_all = np.arange(T)
    pos_all = np.arange(T, dtype=np.int64)
    seq_all = np.zeros(T, np.int32)

    def saved(tokens):  # the seeded saved activations of these global tokens (positions = tokens)
        o = si.normal_tokens(seed, si.TID_SAVED_O, tokens, (n_h, d), 0.3).numpy()
        noise = si.normal_tokens(seed, si.TID_SAVED_LSE, tokens, (n_h,), 0.1).numpy()
        lse = (np.log(np.asarray(tokens, np.float64) + 1.0)[:, None] + 0.5 + noise).astype(np.float32)
        return o, lse

    # ---- device: every rank's ring backward, as the bench runs it
    log("bwd full 128K CP4: device side")
    ws = cp.attn_bwd_workspace(d)
    ks = [device_tensor(seed, si.TID_K, sh[s].tokens, (n_kv, d), 1.0, "bf16") for s in range(N)]
    vs = [device_tensor(seed, si.TID_V, sh[s].tokens, (n_kv, d), 1.0, "bf16") for s in range(N)]
    dks = [torch.zeros(k.shape, device="cuda") for k in ks]
    dvs = [torch.zeros(k.shape, device="cuda") for k in ks]
    kv_segs = [sh[s].segs for s in range(N)]
    dq0 = None
    for r in range(N):
        toks = sh[r].tokens
        q = device_tensor(seed, si.TID_Q, toks, (n_h, d), 1.0, "bf16")
        d_o = device_tensor(seed, si.TID_DO, toks, (n_h, d), 1.0, "bf16")
        o, lse = saved(toks)
        o, lse = torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda()
        delta = torch.empty(len(toks), n_h, device="cuda")
        dq = torch.zeros(len(toks), n_h, d, device="cuda")
        cp.ring_pass_kv_bwd(q, sh[r].segs, r, ks, vs, kv_segs, True, scale, o, lse, d_o, delta, dq,
                            dks, dvs, workspace=ws)
        if r == 0:
            dq0 = dq
        torch.cuda.synchronize()
    del ws

    # ---- dQ of sampled rows of rank 0 against every key they see
    rows = sample_rows(sh[0].segs, 20, seed)
    toks = sh[0].tokens[rows]
    log(f"  oracle dQ: {len(toks)} tokens x {n_h} heads")
    o, lse = saved(toks)
    kf = oracle_view(seed, si.TID_K, g_all, (n_kv, d), 1.0, "bf16")
    vf = oracle_view(seed, si.TID_V, g_all, (n_kv, d), 1.0, "bf16")
    dq_ref, _, _ = oracle.attention_backward(
        oracle_view(seed, si.TID_Q, toks, (n_h, d), 1.0, "bf16"), kf, vf, n_h, n_kv,
        seq_all[toks], pos_all[toks], seq_all, pos_all, True, scale, o, lse,
        oracle_view(seed, si.TID_DO, toks, (n_h, d), 1.0, "bf16"))
    _check(dq0[torch.from_numpy(rows).cuda()].cpu().numpy(), dq_ref, "rank 0 dQ (sampled rows)")

    # ---- dK, dV of sampled keys of every shard against every query row of the sequence
    qf = oracle_view(seed, si.TID_Q, g_all, (n_h, d), 1.0, "bf16")
    gf = oracle_view(seed, si.TID_DO, g_all, (n_h, d), 1.0, "bf16")
    o_all, lse_all = saved(g_all)
    for s in range(N):
        krows = sample_rows(sh[s].segs, 4, seed + 10 + s)
        kt = sh[s].tokens[krows]
        log(f"  oracle dK/dV: shard {s}, {len(kt)} keys")
        _, dk_ref, dv_ref = oracle.attention_backward(
            qf, kf[kt], vf[kt], n_h, n_kv, seq_all, pos_all, seq_all[kt], pos_all[kt], True, scale,
            o_all, lse_all, gf)
        idx = torch.from_numpy(krows).cuda()
        _check(dks[s][idx].cpu().numpy(), dk_ref, f"shard {s} dK (sampled keys, all ranks)")
        _check(dvs[s][idx].cpu().numpy(), dv_ref, f"shard {s} dV (sampled keys, all ranks)")
