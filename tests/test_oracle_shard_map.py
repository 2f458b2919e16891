"""Pins for the oracle's load-balanced shard map (integer, exact).

Source: "Context Parallelism for Scalable Million-Token Inference" (xllm-io review), section 4,
load-balanced sharding (Fig. 2): equal compute and equal KV memory per rank, variable-length
batches supported. The chunk layout (2N chunks, rank r owns r and 2N-1-r) is the reading stated
for the tiny ring workload; tests/golden/shard_map_t256_cp4.txt holds its worked values.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN_DIR = os.path.join(os.path.dirname(__file__), "golden")
GOLDEN = os.path.join(GOLDEN_DIR, "shard_map_t256_cp4.txt")


def _golden(path=GOLDEN):
    rows = []
    with open(path) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x) if x.lstrip("-").isdigit() else x for x in line.split()])
    return rows


def _visible_pairs(q_seq, q_pos, k_seq, k_pos):
    """Brute-force count of causal (query, key) pairs of the same sequence."""
    total = 0
    for s0 in range(0, len(q_pos), 512):
        qs = q_seq[s0:s0 + 512, None]
        qp = q_pos[s0:s0 + 512, None]
        total += int(np.sum((k_seq[None, :] == qs) & (k_pos[None, :] <= qp)))
    return total


def _check_golden_layout(path, T, N):
    gold = _golden(path)
    shards = [oracle.shard_tokens([(0, 0, T)], N, r) for r in range(N)]
    assert sorted(row[0] for row in gold) == list(range(N))
    for row in gold:
        r = row[0]
        seq, pos, glob = shards[r]
        expect = np.r_[np.arange(row[1], row[2]), np.arange(row[3], row[4])]
        assert np.array_equal(pos, expect)
        assert np.array_equal(glob, expect)
        assert np.all(seq == 0)
        counts = []
        for t in range(N):
            s = oracle.pass_kv_shard(N, r, t)
            ks, kp, _ = shards[s]
            counts.append(_visible_pairs(seq, pos, ks, kp))
        assert counts == row[5:9]
        assert sum(counts) == row[9]


def test_golden_t256_cp4_layout_and_pair_counts():
    _check_golden_layout(GOLDEN, 256, 4)


def test_golden_t257_cp4_floor_edges_and_pair_counts():
    """A length 2N does not divide: the hand-worked floor edges put the odd token in chunk 7."""
    _check_golden_layout(os.path.join(GOLDEN_DIR, "shard_map_t257_cp4.txt"), 257, 4)


def test_golden_ring_schedules_cp4():
    """Pass-KV and Pass-Q step tables and Pass-Q slots against the hand-written golden table."""
    N = 4
    for row in _golden(os.path.join(GOLDEN_DIR, "ring_schedule_cp4.txt")):
        kind, who, steps = row[0], row[1], row[2:2 + N]
        if kind == "pass_kv":
            assert [oracle.pass_kv_shard(N, who, t) for t in range(N)] == steps
        else:
            assert [oracle.pass_q_query(N, who, t) for t in range(N)] == steps
            assert [oracle.pass_q_slot(N, q, who) for q in steps] == row[2 + N:]


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8, 16])
def test_ring_schedules_are_rings(N):
    """What the ring itself fixes, for any world size: every rank starts on its own shard, a shard
    held by rank r at step t is held by rank r+1 at step t+1 (it travels one hop per step), and over
    N steps every rank meets every shard once. Pass-Q slots are a bijection onto [0, N^2)."""
    for r in range(N):
        held = [oracle.pass_kv_shard(N, r, t) for t in range(N)]
        assert held[0] == r and sorted(held) == list(range(N))
        for t in range(N - 1):
            assert oracle.pass_kv_shard(N, (r + 1) % N, t + 1) == held[t]
    slots = set()
    for s in range(N):
        hosted = [oracle.pass_q_query(N, s, t) for t in range(N)]
        assert hosted[0] == s and sorted(hosted) == list(range(N))
        for t in range(N - 1):
            assert oracle.pass_q_query(N, (s + 1) % N, t + 1) == hosted[t]
        slots.update(oracle.pass_q_slot(N, q, s) for q in hosted)
    assert slots == set(range(N * N))
    for bad in ((N, 0), (-1, 0), (0, -1)):
        with pytest.raises(ValueError):
            oracle.pass_kv_shard(N, *bad)


@pytest.mark.parametrize("L,N", [(256, 4), (257, 4), (7, 4), (3, 2), (1000, 8), (1, 1), (0, 3)])
def test_ranks_partition_every_range_with_balanced_counts(L, N):
    allpos = []
    sizes = []
    for r in range(N):
        seq, pos, glob = oracle.shard_tokens([(0, 0, L)], N, r)
        allpos.append(pos)
        sizes.append(len(pos))
    allpos = np.concatenate(allpos) if allpos else np.zeros(0)
    assert np.array_equal(np.sort(allpos), np.arange(L))
    # floor chunk edges: chunk sizes differ by at most one, so ranks differ by at most two
    assert max(sizes) - min(sizes) <= 2


def test_equal_compute_per_rank_when_divisible():
    L, N = 4096, 4
    C = L // (2 * N)
    shards = [oracle.shard_tokens([(0, 0, L)], N, r) for r in range(N)]
    for r in range(N):
        qs, qp, _ = shards[r]
        ks = np.concatenate([shards[s][0] for s in range(N)])
        kp = np.concatenate([shards[s][1] for s in range(N)])
        assert _visible_pairs(qs, qp, ks, kp) == 2 * N * C * C + C


def test_persistent_kv_layout_per_rank():
    # cached prefix [0, P) and new tokens [P, P+T) are sharded separately
    P, T, N = 120 * 1024, 8 * 1024, 4
    for r in range(N):
        qs, qp, _ = oracle.shard_tokens([(0, P, P + T)], N, r)
        ks, kp, kg = oracle.shard_tokens([(0, 0, P), (0, P, P + T)], N, r)
        assert len(qp) == 2048 and len(kp) == 32768
        assert np.array_equal(kg, kp)
        c_new = T // 8
        assert qp[0] == P + r * c_new and qp[-1] == P + (8 - r) * c_new - 1
        assert np.sum(kp < P) == 2 * 15360 and np.sum(kp >= P) == 2 * 1024


def test_varlen_batch_global_index_and_segments():
    lens = [64 * 1024, 192 * 1024, 256 * 1024, 512 * 1024]
    N = 8
    base = np.cumsum([0] + lens[:-1])
    sizes = []
    for r in (0, 5, 7):
        seq, pos, glob = oracle.shard_tokens([(i, 0, L) for i, L in enumerate(lens)], N, r)
        sizes.append(len(pos))
        assert np.array_equal(glob, base[seq] + pos)
        # per sequence, chunk r then chunk 2N-1-r of C = L / 2N tokens each
        for i, L in enumerate(lens):
            C = L // (2 * N)
            expect = np.r_[np.arange(r * C, (r + 1) * C), np.arange((2 * N - 1 - r) * C, (2 * N - r) * C)]
            assert np.array_equal(pos[seq == i], expect)
    assert sizes == [131072] * 3


# ------------------------------------------------------------------------ property-based, vs the library
from hypothesis import given, settings, strategies as st  # noqa: E402


@st.composite
def _batches(draw):
    n_seq = draw(st.integers(1, 5))
    ids = draw(st.permutations(list(range(n_seq + draw(st.integers(0, 2))))))[:n_seq]
    ranges = []
    for sid in ids:
        L = draw(st.integers(0, 3000))
        if draw(st.booleans()) and L > 1:          # a cached prefix and new tokens, as two ranges
            P = draw(st.integers(1, L - 1))
            ranges += [(sid, 0, P), (sid, P, L)]
        else:
            ranges.append((sid, 0, L))
    return ranges, draw(st.integers(1, 8))


@settings(max_examples=150, deadline=None)
@given(_batches())
def test_library_shard_map_matches_oracle_for_random_batches(batch):
    from context_ring_attention_amd import binding as cp
    ranges, N = batch
    seen = []
    for r in range(N):
        segs, toks = cp.shard_map(ranges, N, r)
        seq, pos, glob = oracle.shard_tokens(ranges, N, r)
        lib_seq = np.concatenate([np.full(n, s, np.int64) for s, _, n, _ in segs]) if segs else np.zeros(0, np.int64)
        lib_pos = np.concatenate([np.arange(p, p + n) for _, p, n, _ in segs]) if segs else np.zeros(0, np.int64)
        assert np.array_equal(lib_seq, seq) and np.array_equal(lib_pos, pos)
        assert np.array_equal(toks, glob)
        seen.append(glob)
    allg = np.concatenate(seen) if seen else np.zeros(0, np.int64)
    assert len(np.unique(allg)) == len(allg)      # no token owned twice
