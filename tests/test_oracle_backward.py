"""Pins for the oracle's attention backward (fp64), each against something other than its formula.

The backward of context parallelism sends every rank's K/V gradient contributions back to the
owners of those K/V chunks ("Context Parallelism과 Expert Parallelism", §6); each ring step's
contribution is the gradient of the partial attention over that step's keys, taken with the
final (merged) softmax. Pinned by:
- central finite differences of the forward oracle (the gradient of L = sum(dO * O));
- torch autograd on a dense fp64 formulation (explicit score and mask matrices);
- exactness of the sharding: contributions over any partition of the keys sum to the unsharded
  gradient (the reduce-scatter is a sum);
- closed forms: uniform V gives dQ = dK = 0; a zero query gives uniform weights, so
  dV_j = sum over the rows that see key j of dO / (number of keys the row sees); every row's
  weights sum to one, so sum_j dV_j = sum_i dO_i;
- GQA ownership: gradients of one KV head come only from its query heads.
"""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _dyadic(rng, shape, denom=8, lim=16):
    """Values m / denom with small integers m: exact in fp32, so are x +- 2^-12."""
    return (rng.integers(-lim, lim + 1, size=shape) / denom).astype(np.float32)


def _problem(seed, seqlens=(5, 7), n_h=4, n_kv=2, d=4):
    rng = np.random.default_rng(seed)
    T = sum(seqlens)
    q = _dyadic(rng, (T, n_h, d))
    k = _dyadic(rng, (T, n_kv, d))
    v = _dyadic(rng, (T, n_kv, d))
    g = _dyadic(rng, (T, n_h, d))
    seq = np.concatenate([np.full(L, i, np.int32) for i, L in enumerate(seqlens)])
    pos = np.concatenate([np.arange(L, dtype=np.int64) for L in seqlens])
    return q, k, v, g, seq, pos


def _forward_loss(q, k, v, g, n_h, n_kv, seq, pos, causal, scale):
    o, _ = oracle.attention(q, k, v, n_h, n_kv, seq, pos, seq, pos, causal, scale)
    return float(np.sum(o * g.astype(np.float64)))


def _backward(q, k, v, g, n_h, n_kv, seq, pos, causal, scale, keys=None):
    o, lse = oracle.attention(q, k, v, n_h, n_kv, seq, pos, seq, pos, causal, scale)
    if keys is None:
        keys = np.arange(k.shape[0])
    dq, dk, dv = oracle.attention_backward(q, k[keys], v[keys], n_h, n_kv, seq, pos, seq[keys],
                                           pos[keys], causal, scale, o, lse, g)
    return dq, dk, dv


@pytest.mark.parametrize("causal", [True, False])
def test_finite_differences_of_the_forward(causal):
    n_h, n_kv, scale = 4, 2, 0.5
    q, k, v, g, seq, pos = _problem(1)
    dq, dk, dv = _backward(q, k, v, g, n_h, n_kv, seq, pos, causal, scale)
    h = 2.0 ** -12
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros(x.shape)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            lp = _forward_loss(**{**args, name: xp}, g=g, n_h=n_h, n_kv=n_kv, seq=seq, pos=pos,
                               causal=causal, scale=scale)
            lm = _forward_loss(**{**args, name: xm}, g=g, n_h=n_h, n_kv=n_kv, seq=seq, pos=pos,
                               causal=causal, scale=scale)
            fd[idx] = (lp - lm) / (2 * h)
        err = float(np.max(np.abs(fd - grad)))
        assert err < 2e-6 * max(1.0, float(np.max(np.abs(grad)))), (name, err)


def _torch_dense(q, k, v, g, n_h, n_kv, seq, pos, causal, scale):
    """Autograd of an explicit dense masked attention (fp64)."""
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    T = q.shape[0]
    st, pt = torch.tensor(seq), torch.tensor(pos)
    mask = st[:, None] == st[None, :]
    if causal:
        mask = mask & (pt[None, :] <= pt[:, None])
    group = n_h // n_kv
    outs = []
    for h in range(n_h):
        S = scale * (qt[:, h, :] @ kt[:, h // group, :].T)
        S = S.masked_fill(~mask, float("-inf"))
        outs.append(torch.softmax(S, dim=1) @ vt[:, h // group, :])
    O = torch.stack(outs, dim=1)
    (O * torch.tensor(g, dtype=torch.float64)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("seed,causal", [(2, True), (3, False), (4, True)])
def test_matches_torch_autograd_on_a_dense_formulation(seed, causal):
    rng = np.random.default_rng(seed)
    seqlens, n_h, n_kv, d, scale = (9, 14, 3), 4, 2, 8, 1.0 / math.sqrt(8)
    T = sum(seqlens)
    q = rng.standard_normal((T, n_h, d)).astype(np.float32)
    k = rng.standard_normal((T, n_kv, d)).astype(np.float32)
    v = rng.standard_normal((T, n_kv, d)).astype(np.float32)
    g = rng.standard_normal((T, n_h, d)).astype(np.float32)
    seq = np.concatenate([np.full(L, i, np.int32) for i, L in enumerate(seqlens)])
    pos = np.concatenate([np.arange(L, dtype=np.int64) for L in seqlens])
    dq, dk, dv = _backward(q, k, v, g, n_h, n_kv, seq, pos, causal, scale)
    tq, tk, tv = _torch_dense(q, k, v, g, n_h, n_kv, seq, pos, causal, scale)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - b)) < 1e-12


@pytest.mark.parametrize("n_parts", [2, 3, 7])
def test_contributions_over_a_key_partition_sum_to_the_full_gradient(n_parts):
    rng = np.random.default_rng(10 + n_parts)
    seqlens, n_h, n_kv, d, scale = (11, 17), 4, 1, 8, 0.3
    T = sum(seqlens)
    q = rng.standard_normal((T, n_h, d)).astype(np.float32)
    k = rng.standard_normal((T, n_kv, d)).astype(np.float32)
    v = rng.standard_normal((T, n_kv, d)).astype(np.float32)
    g = rng.standard_normal((T, n_h, d)).astype(np.float32)
    seq = np.concatenate([np.full(L, i, np.int32) for i, L in enumerate(seqlens)])
    pos = np.concatenate([np.arange(L, dtype=np.int64) for L in seqlens])
    dq, dk, dv = _backward(q, k, v, g, n_h, n_kv, seq, pos, True, scale)
    assign = rng.integers(0, n_parts, size=T)
    dq_sum = np.zeros_like(dq)
    dk_all, dv_all = np.zeros_like(dk), np.zeros_like(dv)
    for s in range(n_parts):
        keys = np.flatnonzero(assign == s)
        pq, pk, pv = _backward(q, k, v, g, n_h, n_kv, seq, pos, True, scale, keys=keys)
        dq_sum += pq
        dk_all[keys] = pk
        dv_all[keys] = pv
    assert np.max(np.abs(dq_sum - dq)) < 1e-12
    assert np.max(np.abs(dk_all - dk)) < 1e-12 and np.max(np.abs(dv_all - dv)) < 1e-12


def test_uniform_values_give_zero_score_gradients_and_dv_sums_to_do():
    rng = np.random.default_rng(20)
    seqlens, n_h, n_kv, d, scale = (13, 6), 2, 1, 8, 0.4
    T = sum(seqlens)
    q = rng.standard_normal((T, n_h, d)).astype(np.float32)
    k = rng.standard_normal((T, n_kv, d)).astype(np.float32)
    vec = np.linspace(-2.0, 1.5, d).astype(np.float32)
    v = np.broadcast_to(vec, (T, n_kv, d)).copy()
    g = rng.standard_normal((T, n_h, d)).astype(np.float32)
    seq = np.concatenate([np.full(L, i, np.int32) for i, L in enumerate(seqlens)])
    pos = np.concatenate([np.arange(L, dtype=np.int64) for L in seqlens])
    dq, dk, dv = _backward(q, k, v, g, n_h, n_kv, seq, pos, True, scale)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    # every row's weights sum to one: the value gradients add up to the output gradients
    assert np.max(np.abs(dv.sum(axis=(0, 1)) - g.astype(np.float64).sum(axis=(0, 1)))) < 1e-12


def test_zero_query_gives_uniform_weights():
    rng = np.random.default_rng(21)
    L, n_h, n_kv, d, scale = 15, 2, 1, 8, 0.7
    q = np.zeros((L, n_h, d), np.float32)
    k = rng.standard_normal((L, n_kv, d)).astype(np.float32)
    v = rng.standard_normal((L, n_kv, d)).astype(np.float32)
    g = rng.standard_normal((L, n_h, d)).astype(np.float32)
    seq = np.zeros(L, np.int32)
    pos = np.arange(L, dtype=np.int64)
    _, _, dv = _backward(q, k, v, g, n_h, n_kv, seq, pos, True, scale)
    # row i sees keys 0..i with weight 1/(i+1): dV_j = sum_{i >= j} sum_h dO[i,h] / (i+1)
    gg = g.astype(np.float64).sum(axis=1)
    expect = np.array([sum(gg[i] / (i + 1) for i in range(j, L)) for j in range(L)])
    assert np.max(np.abs(dv[:, 0, :] - expect)) < 1e-13


def test_gqa_gradients_come_from_the_heads_of_the_group():
    rng = np.random.default_rng(22)
    L, n_h, n_kv, d, scale = 12, 4, 2, 8, 0.5
    q = rng.standard_normal((L, n_h, d)).astype(np.float32)
    k = rng.standard_normal((L, n_kv, d)).astype(np.float32)
    v = rng.standard_normal((L, n_kv, d)).astype(np.float32)
    g = rng.standard_normal((L, n_h, d)).astype(np.float32)
    g[:, 2:, :] = 0.0            # no gradient on the heads of KV head 1
    seq = np.zeros(L, np.int32)
    pos = np.arange(L, dtype=np.int64)
    dq, dk, dv = _backward(q, k, v, g, n_h, n_kv, seq, pos, True, scale)
    assert np.all(dk[:, 1, :] == 0.0) and np.all(dv[:, 1, :] == 0.0) and np.all(dq[:, 2:, :] == 0.0)
    assert np.max(np.abs(dk[:, 0, :])) > 1e-3 and np.max(np.abs(dv[:, 0, :])) > 1e-3


def test_rows_without_keys_contribute_nothing():
    rng = np.random.default_rng(23)
    L, n_h, n_kv, d = 6, 2, 1, 4
    q = rng.standard_normal((L, n_h, d)).astype(np.float32)
    k = rng.standard_normal((L, n_kv, d)).astype(np.float32)
    v = rng.standard_normal((L, n_kv, d)).astype(np.float32)
    g = rng.standard_normal((L, n_h, d)).astype(np.float32)
    seq = np.zeros(L, np.int32)
    pos = np.arange(L, dtype=np.int64)
    o = np.zeros((L, n_h, d))
    lse = np.full((L, n_h), -np.inf)
    dq, dk, dv = oracle.attention_backward(q, k, v, n_h, n_kv, seq, pos, seq, pos, True, 1.0, o, lse, g)
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0)
