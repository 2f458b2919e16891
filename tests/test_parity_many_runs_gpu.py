"""GPU parity for segment tables longer than one kernel launch takes (CP_MAX_SEGMENTS = 64 runs),
element by element against the oracle.

Load-balanced sharding of a batch of variable-length requests ("Context Parallelism for Scalable
Million-Token Inference", §4, load-balanced sharding) gives every rank two runs per request, so a
batch of more than 32 requests overflows one launch's tables. The library then splits the Q runs
into groups of whole sequences (each with only its own sequences' KV runs), and folds KV runs
beyond one launch into the same rows by further launches. These cases cover both paths.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from ring_cases import device_tensor, log, oracle_view, scale_of, torch_dtype
from test_parity_gpu import assert_close, run_pass_kv, run_pass_q

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("mode", ["partials", "running"])
def test_pass_kv_100_ragged_sequences_cp4(mode):
    # ~200 Q runs and ~200 KV runs per shard: several launches per ring step
    lens = [int(x) for x in np.random.default_rng(31).integers(1, 400, size=100)]
    run_pass_kv(lens, 4, 16, 1, 128, "bf16", seed=31, mode=mode, ranks=[0, 3])


def test_pass_kv_70_sequences_fp32_gqa_d64():
    lens = [int(x) for x in np.random.default_rng(32).integers(1, 120, size=70)]
    run_pass_kv(lens, 2, 8, 2, 64, "f32", seed=32, mode="partials", ranks=[1])


def test_pass_q_40_sequences_with_cached_prefixes():
    # each KV shard holds 4 runs per sequence (two cached chunks, two new ones): 160 runs
    rng = np.random.default_rng(33)
    P = [int(x) for x in rng.integers(0, 300, size=40)]
    T = [int(x) for x in rng.integers(1, 90, size=40)]
    run_pass_q(P, T, 2, 16, 1, 128, seed=33)


def _custom(q_segs, kv_segs, tq, tk, n_h, n_kv, d, dtype, causal, accumulate, seed):
    """cp_partial_attn on hand-built segment tables against the oracle over the same keys."""
    from context_ring_attention_amd import binding as cp
    std = 1.0 / np.sqrt(d) if dtype == "f32" else 1.0
    scale = scale_of(d)
    # shard row r holds global token r of one sequence laid out by the tables
    q = device_tensor(seed, si.TID_Q, np.arange(tq), (n_h, d), std, dtype)
    k = device_tensor(seed, si.TID_K, np.arange(tk), (n_kv, d), std, dtype)
    v = device_tensor(seed, si.TID_V, np.arange(tk), (n_kv, d), std, dtype)
    o = torch.full((tq, n_h, d), float("nan"), device="cuda")
    lse = torch.full((tq, n_h), float("nan"), device="cuda")

    def expand(segs, n):
        seq = np.full(n, -1, np.int32)
        pos = np.full(n, -1, np.int64)
        for s, p, ln, loc in segs:
            seq[loc:loc + ln] = s
            pos[loc:loc + ln] = np.arange(p, p + ln)
        return seq, pos
    q_seq, q_pos = expand(q_segs, tq)
    k_seq, k_pos = expand(kv_segs, tk)
    qf = oracle_view(seed, si.TID_Q, np.arange(tq), (n_h, d), std, dtype)
    kf = oracle_view(seed, si.TID_K, np.arange(tk), (n_kv, d), std, dtype)
    vf = oracle_view(seed, si.TID_V, np.arange(tk), (n_kv, d), std, dtype)
    covered = np.flatnonzero(q_seq >= 0)
    kin = np.flatnonzero(k_seq >= 0)
    if accumulate:
        # a running partial over a first half of the keys, then this call folds in the rest
        half = kin[: len(kin) // 2]
        rest = kin[len(kin) // 2:]
        o0, l0 = oracle.attention(qf, kf[half], vf[half], n_h, n_kv, q_seq, q_pos, k_seq[half],
                                  k_pos[half], causal, scale)
        o.copy_(torch.from_numpy(o0.astype(np.float32)))
        lse.copy_(torch.from_numpy(l0.astype(np.float32)))
        kv_used = [sg for sg in kv_segs if sg[3] >= (rest[0] if len(rest) else tk)]
    else:
        kv_used = kv_segs
    log(f"custom tables: {len(q_segs)} Q runs, {len(kv_used)} KV runs, {dtype}, causal={causal}, "
        f"accumulate={accumulate}")
    cp.partial_attn(q, k, v, q_segs, kv_used, causal, scale, o, lse, accumulate=accumulate)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qf, kf[kin], vf[kin], n_h, n_kv, q_seq, q_pos, k_seq[kin],
                                    k_pos[kin], causal, scale)
    sel = torch.from_numpy(covered).cuda()
    assert_close(o[sel], lse[sel], o_ref[covered], l_ref[covered], dtype, "custom tables")
    unused = np.flatnonzero(q_seq < 0)
    if len(unused):   # rows outside every Q run are never written
        assert bool(torch.isnan(o[torch.from_numpy(unused).cuda()]).all())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
def test_one_sequence_with_150_kv_runs(dtype, causal):
    """One sequence whose KV shard holds 150 runs of 2 keys, stored in reverse order: the Q rows
    take the KV runs in three launches (64 + 64 + 22), the later two folding into the first."""
    T = 300
    q_segs = [(0, 0, T, 0)]
    kv_segs = [(0, 2 * i, 2, T - 2 * (i + 1)) for i in range(T // 2)]   # position 2i at row T-2i-2
    _custom(q_segs, kv_segs, T, T, 16, 1, 128 if dtype == "bf16" else 64, dtype, causal, False, 34)


def test_one_sequence_with_130_q_runs_and_a_running_partial():
    """130 Q runs of 3 tokens of one sequence in shuffled storage order (three groups of Q runs),
    folding 90 KV runs into a running partial (accumulate = 1)."""
    rng = np.random.default_rng(35)
    order = rng.permutation(130)
    q_segs = [(0, 3 * int(p), 3, 3 * i) for i, p in enumerate(order)]
    kv_segs = [(0, 3 * i + 0, 3, 3 * i) for i in range(130)]             # keys stored in order
    kv_rows = 390
    _custom(q_segs, kv_segs, 390, kv_rows, 16, 1, 128, "bf16", True, True, 35)


def test_runs_of_other_sequences_and_empty_runs_among_many():
    """80 sequences, Q runs interleaved with zero-length runs and a sequence without KV runs
    (its rows get O = 0, LSE = -inf)."""
    rng = np.random.default_rng(36)
    lens = [int(x) for x in rng.integers(1, 30, size=80)]
    q_segs, kv_segs, loc = [], [], 0
    for s, L in enumerate(lens):
        q_segs.append((s, 0, L, loc))
        if s % 7 == 3:
            q_segs.append((s, L, 0, loc + L))          # an empty run
        if s != 11:                                    # sequence 11 has no keys here
            kv_segs.append((s, 0, L, loc))
        loc += L
    _custom(q_segs, kv_segs, loc, loc, 8, 2, 64, "bf16", True, False, 36)
