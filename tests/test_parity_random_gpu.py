"""Seeded random small configurations of the ring paths against the oracle.

Each case draws sequence lengths (ragged, down to one token), a CP world, a head ratio, D_H,
input dtype, the causal flag and the ring variant (Pass-KV with partials or a running merge, or
Pass-Q over a cached prefix), then checks one rank's merged result, and its partials where the
mode keeps them, element by element against the oracle (larger running-mode rings with a ring
workspace on sampled rows) ("Context Parallelism for Scalable
Million-Token Inference", §3 core formulas; the oracle's readings are the ones the other parity
tests use).
"""
import numpy as np
import pytest

from test_parity_gpu import run_decode, run_pass_kv, run_pass_q

pytestmark = pytest.mark.gpu


def _draw_cases(n_cases, seed=2026):
    rng = np.random.default_rng(seed)
    heads = [(16, 1), (8, 2), (4, 4), (32, 4), (12, 3)]
    cases = []
    for i in range(n_cases):
        n_h, n_kv = heads[rng.integers(len(heads))]
        d = int(rng.choice([64, 128]))
        N = int(rng.choice([1, 2, 3, 4, 8]))
        if rng.random() < 0.3:  # Pass-Q over a cached prefix
            n_seq = int(rng.integers(1, 4))
            P = [int(x) for x in rng.integers(0, 1200, size=n_seq)]
            T = [int(x) for x in rng.integers(1, 400, size=n_seq)]
            cases.append(("pass_q", dict(P=P, T=T, N=N, n_h=n_h, n_kv=n_kv, d=d, seed=100 + i)))
        else:
            n_seq = int(rng.integers(1, 5))
            seqs = [int(x) for x in rng.integers(1, 1500, size=n_seq)]
            dtype = "f32" if rng.random() < 0.2 else "bf16"
            causal = bool(rng.random() < 0.8)
            mode = str(rng.choice(["partials", "running"]))
            rank = int(rng.integers(N))
            cases.append(("pass_kv", dict(seqs=seqs, N=N, n_h=n_h, n_kv=n_kv, d=d, dtype=dtype,
                                          seed=100 + i, causal=causal, ranks=[rank], mode=mode)))
    return cases


CASES = _draw_cases(20)


@pytest.mark.parametrize("kind,kw", CASES, ids=[f"{k}-{i}" for i, (k, _) in enumerate(CASES)])
def test_random_config(kind, kw):
    if kind == "pass_q":
        run_pass_q(**kw)
    else:
        run_pass_kv(**kw)


def _draw_split_cases(n_cases, seed=2029):
    """Running-mode rings with a ring workspace, large enough that steps of the smaller head ratios
    split over their keys; checked on sampled rows."""
    rng = np.random.default_rng(seed)
    heads = [(4, 1), (2, 1), (1, 1), (8, 2), (4, 4), (16, 1)]
    cases = []
    for i in range(n_cases):
        n_h, n_kv = heads[rng.integers(len(heads))]
        N = int(rng.choice([2, 4]))
        total = int(rng.integers(16000, 64000))
        cuts = sorted(int(x) for x in rng.integers(1, total, size=int(rng.integers(0, 3))))
        seqs = [b - a for a, b in zip([0] + cuts, cuts + [total]) if b > a]
        cases.append(dict(seqs=seqs, N=N, n_h=n_h,
                          n_kv=n_kv, d=int(rng.choice([64, 128])), dtype="bf16", seed=400 + i,
                          causal=bool(rng.random() < 0.8), ranks=[int(rng.integers(N))],
                          mode=str(rng.choice(["running", "running_out"])),
                          ws=int(rng.choice([1, 2, 3, 7])), n_sample=256))
    return cases


SPLIT_CASES = _draw_split_cases(8)


@pytest.mark.parametrize("kw", SPLIT_CASES, ids=[f"split-{i}" for i in range(len(SPLIT_CASES))])
def test_random_split_ring_config(kw):
    run_pass_kv(**kw)


def _draw_decode_cases(n_cases, seed=2027):
    rng = np.random.default_rng(seed)
    heads = [(16, 1), (8, 2), (40, 2), (4, 4)]
    cases = []
    for i in range(n_cases):
        n_h, n_kv = heads[rng.integers(len(heads))]
        B = int(rng.choice([1, 2, 5, 9, 33]))
        lengths = [int(x) for x in rng.integers(0, 3000, size=B)]
        n_splits = int(rng.choice([1, 7, 64, 256]))
        cases.append(dict(lengths=lengths, n_h=n_h, n_kv=n_kv, d=int(rng.choice([64, 128])),
                          n_splits=n_splits, seed=200 + i, out=str(rng.choice(["f32", "bf16"])),
                          check_splits=[0, n_splits - 1]))
    return cases


DECODE_CASES = _draw_decode_cases(10)


@pytest.mark.parametrize("kw", DECODE_CASES, ids=[f"decode-{i}" for i in range(len(DECODE_CASES))])
def test_random_decode_config(kw):
    run_decode(**kw)


def _draw_backward_cases(n_cases, seed=2028):
    rng = np.random.default_rng(seed)
    heads = [(16, 1), (8, 2), (4, 4), (12, 3)]
    cases = []
    for i in range(n_cases):
        n_h, n_kv = heads[rng.integers(len(heads))]
        n_seq = int(rng.integers(1, 4))
        cases.append(dict(seqs=[int(x) for x in rng.integers(1, 900, size=n_seq)],
                          N=int(rng.choice([1, 2, 3, 4])), n_h=n_h, n_kv=n_kv,
                          d=int(rng.choice([64, 128])), seed=300 + i,
                          causal=bool(rng.random() < 0.8),
                          dtype="f32" if rng.random() < 0.2 else "bf16",
                          ws=bool(rng.random() < 0.7)))
    return cases


BACKWARD_CASES = _draw_backward_cases(20)


@pytest.mark.parametrize("kw", BACKWARD_CASES, ids=[f"backward-{i}" for i in range(len(BACKWARD_CASES))])
def test_random_backward_config(kw):
    """Every rank's ring backward (dQ per rank, dK/dV per shard over all ranks) against the oracle
    ("Context Parallelism과 Expert Parallelism", §6), with and without the backward workspace."""
    from test_parity_bwd_gpu import run_bwd
    kw = dict(kw)
    run_bwd(kw.pop("seqs"), kw.pop("N"), kw.pop("n_h"), kw.pop("n_kv"), kw.pop("d"), **kw)
