"""Pins for the fp64 oracle, each against something other than the oracle itself.

- exactness of the merge over arbitrary splits of the visible keys ("lossless, exact" ring
  variants, "Context Parallelism for Scalable Million-Token Inference" review, §2);
- closed forms: uniform values, zero query, one-hot key, first token;
- a dense brute force (explicit [T, T] score and mask matrices, written independently);
- the GQA head grouping (consecutive heads share a KV head, "Context Parallelism과 Expert
  Parallelism" §8.2).
"""
import math

import numpy as np
import pytest

import oracle
from synth_inputs import normal_tokens

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _batch(seqlens, n_h, n_kv, d, seed, std=1.0):
    T = int(sum(seqlens))
    q = normal_tokens(seed, 1, np.arange(T), (n_h, d), std).numpy()
    k = normal_tokens(seed, 2, np.arange(T), (n_kv, d), std).numpy()
    v = normal_tokens(seed, 3, np.arange(T), (n_kv, d), std).numpy()
    seq = np.concatenate([np.full(L, i, np.int32) for i, L in enumerate(seqlens)])
    pos = np.concatenate([np.arange(L, dtype=np.int64) for L in seqlens])
    return q, k, v, seq, pos


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_merge_of_any_key_partition_equals_unsharded(seed):
    rng = np.random.default_rng(100 + seed)
    seqlens = [20, 28]
    n_h, n_kv, d = 4, 2, 16
    q, k, v, seq, pos = _batch(seqlens, n_h, n_kv, d, seed)
    scale = 1.0 / math.sqrt(d)
    o_full, lse_full = oracle.attention(q, k, v, n_h, n_kv, seq, pos, seq, pos, True, scale)
    T = q.shape[0]
    for n_sub in [1, 2, 3, 5, 9, 17]:
        # subset 0 stays empty, subset n_sub-1 (if > 1) gets exactly one key
        assign = rng.integers(1 if n_sub > 1 else 0, n_sub, size=T)
        if n_sub > 2:
            assign[assign == n_sub - 1] = 1
            assign[rng.integers(0, T)] = n_sub - 1
        parts_o, parts_l = [], []
        for s in rng.permutation(n_sub):
            idx = np.flatnonzero(assign == s)
            o_p, l_p = oracle.attention(q, k[idx], v[idx], n_h, n_kv, seq, pos, seq[idx], pos[idx],
                                        True, scale)
            parts_o.append(o_p.reshape(-1, d))
            parts_l.append(l_p.reshape(-1))
        o_m, l_m = oracle.merge(parts_o, parts_l)
        assert np.max(np.abs(o_m - o_full.reshape(-1, d))) < 1e-12
        assert np.max(np.abs(l_m - lse_full.reshape(-1))) < 1e-12


def test_uniform_values_give_that_value_for_every_row_and_shard():
    seqlens = [17, 33]
    n_h, n_kv, d = 4, 1, 8
    q, k, _, seq, pos = _batch(seqlens, n_h, n_kv, d, 3)
    vec = np.linspace(-1.5, 2.5, d).astype(np.float32)
    v = np.broadcast_to(vec, (q.shape[0], n_kv, d)).copy()
    o, _ = oracle.attention(q, k, v, n_h, n_kv, seq, pos, seq, pos, True, 0.3)
    assert np.max(np.abs(o - vec)) < 1e-14
    half = np.arange(q.shape[0]) % 2 == 0
    o_p, l_p = oracle.attention(q, k[half], v[half], n_h, n_kv, seq, pos, seq[half], pos[half],
                                True, 0.3)
    seen = np.isfinite(l_p)
    assert np.max(np.abs(o_p[seen] - vec)) < 1e-14
    assert np.all(o_p[~seen] == 0.0)


def test_zero_query_gives_running_mean_and_log_count():
    L = 40
    n_h, n_kv, d = 2, 1, 8
    _, k, v, seq, pos = _batch([L], n_h, n_kv, d, 4)
    q = np.zeros((L, n_h, d), np.float32)
    o, lse = oracle.attention(q, k, v, n_h, n_kv, seq, pos, seq, pos, True, 0.125)
    vv = v[:, 0, :].astype(np.float64)
    running_mean = np.cumsum(vv, axis=0) / np.arange(1, L + 1)[:, None]
    for h in range(n_h):
        assert np.max(np.abs(o[:, h, :] - running_mean)) < 1e-13
        assert np.max(np.abs(lse[:, h] - np.log(np.arange(1, L + 1)))) < 1e-13


@pytest.mark.parametrize("a", [-3.0, 0.7, 5.0])
def test_one_hot_key_closed_form(a):
    L, d = 30, 16
    jstar = 7
    _, _, v, seq, pos = _batch([L], 1, 1, d, 5)
    k = np.zeros((L, 1, d), np.float32)
    k[jstar, 0, 3] = 2.0
    q = np.zeros((L, 1, d), np.float32)
    scale = 0.25
    q[:, 0, 3] = a / (2.0 * scale)
    a = scale * 2.0 * float(q[0, 0, 3])     # the score the stored fp32 query really gives
    o, lse = oracle.attention(q, k, v, 1, 1, seq, pos, seq, pos, True, scale)
    vv = v[:, 0, :].astype(np.float64)
    for p in range(L):
        n = p + 1
        if p < jstar:
            exp_o = vv[: p + 1].mean(axis=0)
            exp_l = math.log(n)
        else:
            ea = math.exp(a)
            exp_o = (ea * vv[jstar] + vv[: p + 1].sum(axis=0) - vv[jstar]) / (ea + n - 1)
            exp_l = math.log(ea + n - 1)
        assert np.max(np.abs(o[p, 0] - exp_o)) < 1e-13
        assert abs(lse[p, 0] - exp_l) < 1e-13


def test_first_token_of_each_sequence_sees_only_itself():
    seqlens = [5, 9, 3]
    n_h, n_kv, d = 4, 2, 8
    q, k, v, seq, pos = _batch(seqlens, n_h, n_kv, d, 6)
    scale = 0.35
    o, lse = oracle.attention(q, k, v, n_h, n_kv, seq, pos, seq, pos, True, scale)
    starts = np.cumsum([0] + seqlens[:-1])
    for t in starts:
        for h in range(n_h):
            g = h // (n_h // n_kv)
            assert np.max(np.abs(o[t, h] - v[t, g])) < 1e-15
            s = scale * float(np.dot(q[t, h].astype(np.float64), k[t, g].astype(np.float64)))
            assert abs(lse[t, h] - s) < 1e-13


def _dense_brute_force(q, k, v, head_to_kv, seq, pos, causal, scale):
    """Explicit dense score matrix and explicit 0/1 mask matrix, two-pass softmax (numpy)."""
    T, n_h, d = q.shape
    o = np.zeros((T, n_h, d))
    lse = np.zeros((T, n_h))
    mask = np.zeros((T, T), dtype=bool)
    for i in range(T):
        for j in range(T):
            mask[i, j] = seq[i] == seq[j] and (not causal or pos[j] <= pos[i])
    for h in range(n_h):
        g = head_to_kv[h]
        S = scale * (q[:, h, :].astype(np.float64) @ k[:, g, :].astype(np.float64).T)
        S = np.where(mask, S, -np.inf)
        m = S.max(axis=1)
        P = np.exp(S - m[:, None])
        den = P.sum(axis=1)
        o[:, h, :] = (P @ v[:, g, :].astype(np.float64)) / den[:, None]
        lse[:, h] = m + np.log(den)
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
def test_dense_brute_force_agrees(causal):
    seqlens = [23, 41]
    n_h, n_kv, d = 4, 2, 16
    q, k, v, seq, pos = _batch(seqlens, n_h, n_kv, d, 7)
    head_to_kv = [0, 0, 1, 1]  # consecutive heads share a KV head
    o, lse = oracle.attention(q, k, v, n_h, n_kv, seq, pos, seq, pos, causal, 0.25)
    ob, lb = _dense_brute_force(q, k, v, head_to_kv, seq, pos, causal, 0.25)
    assert np.max(np.abs(o - ob)) < 1e-13
    assert np.max(np.abs(lse - lb)) < 1e-13


def test_gqa_consecutive_heads_share_kv_head():
    L, n_h, n_kv, d = 24, 4, 2, 8
    q, k, v, seq, pos = _batch([L], n_h, n_kv, d, 8)
    k[:, 1, :] = 0.0          # KV head 1 gives every key the same score
    o, _ = oracle.attention(q, k, v, n_h, n_kv, seq, pos, seq, pos, True, 0.5)
    run1 = np.cumsum(v[:, 1, :].astype(np.float64), axis=0) / np.arange(1, L + 1)[:, None]
    run0 = np.cumsum(v[:, 0, :].astype(np.float64), axis=0) / np.arange(1, L + 1)[:, None]
    for h in (2, 3):
        assert np.max(np.abs(o[:, h, :] - run1)) < 1e-13
    for h in (0, 1):
        assert np.max(np.abs(o[1:, h, :] - run0[1:])) > 1e-3   # real softmax, not uniform


def test_partial_over_rows_subset_matches_full():
    seqlens = [50]
    q, k, v, seq, pos = _batch(seqlens, 2, 1, 8, 9)
    o, lse = oracle.attention(q, k, v, 2, 1, seq, pos, seq, pos, True, 0.3)
    rows = np.array([49, 0, 17, 17])
    o_r, l_r = oracle.attention(q, k, v, 2, 1, seq, pos, seq, pos, True, 0.3, rows=rows)
    assert np.array_equal(o_r, o[rows]) and np.array_equal(l_r, lse[rows])


def test_empty_visible_set_and_merge_of_nothing():
    q, k, v, seq, pos = _batch([6], 2, 1, 4, 10)
    o, lse = oracle.attention(q, k[:0], v[:0], 2, 1, seq, pos, seq[:0], pos[:0], True, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o_m, l_m = oracle.merge([o.reshape(-1, 4), o.reshape(-1, 4)], [lse.reshape(-1), lse.reshape(-1)])
    assert np.all(o_m == 0) and np.all(np.isneginf(l_m))
    # keys of another sequence are invisible
    o2, l2 = oracle.attention(q, k, v, 2, 1, seq, pos, seq + 1, pos, False, 1.0)
    assert np.all(o2 == 0) and np.all(np.isneginf(l2))


def test_merge_single_part_is_identity_and_two_equal_parts_add_ln2():
    rng = np.random.default_rng(11)
    o = rng.standard_normal((10, 8))
    l = rng.standard_normal(10)
    o1, l1 = oracle.merge([o], [l])
    assert np.max(np.abs(o1 - o)) < 1e-15 and np.max(np.abs(l1 - l)) < 1e-15
    o2, l2 = oracle.merge([o, o], [l, l])
    assert np.max(np.abs(o2 - o)) < 1e-15 and np.max(np.abs(l2 - (l + math.log(2)))) < 1e-14


def test_decode_splits_cover_keys_and_merge_exactly():
    L, n_h, d, S = 300, 4, 16, 32
    q1, k, v, seq, pos = _batch([L], n_h, 1, d, 12)
    q = q1[:1]
    qs = np.zeros(1, np.int32)
    qp = np.array([L], np.int64)     # the new token comes after every cached key
    bounds = oracle.split_bounds(L, S)
    assert bounds[0][0] == 0 and bounds[-1][1] == L
    assert all(b[1] == c[0] for b, c in zip(bounds, bounds[1:]))
    assert all(L // S <= hi - lo <= -(-L // S) for lo, hi in bounds)
    o_full, l_full = oracle.attention(q, k, v, n_h, 1, qs, qp, seq, pos, False, 0.2)
    po, pl = [], []
    for lo, hi in bounds:
        o_p, l_p = oracle.attention(q, k[lo:hi], v[lo:hi], n_h, 1, qs, qp, seq[lo:hi], pos[lo:hi],
                                    False, 0.2)
        po.append(o_p.reshape(-1, d))
        pl.append(l_p.reshape(-1))
    o_m, l_m = oracle.merge(po, pl)
    assert np.max(np.abs(o_m - o_full.reshape(-1, d))) < 1e-12
    assert np.max(np.abs(l_m - l_full.reshape(-1))) < 1e-12
    # a split with fewer keys than splits: empty splits merge away
    b2 = oracle.split_bounds(5, 8)
    assert sum(hi - lo for lo, hi in b2) == 5 and sum(hi == lo for lo, hi in b2) == 3


def test_decode_split_table_golden_l300_s32():
    """Hand-worked split table of a length the split count does not divide (L=300, S=32):
    tests/golden/decode_splits_l300_s32.txt."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "decode_splits_l300_s32.txt")
    rows = [tuple(int(x) for x in line.split()) for line in open(path)
            if line.strip() and not line.startswith("#")]
    assert [c for c, _, _ in rows] == list(range(32))
    assert oracle.split_bounds(300, 32) == [(lo, hi) for _, lo, hi in rows]
