"""Algorithm 1 (ring Pass-KV vs Pass-Q selection) of "Context Parallelism for Scalable
Million-Token Inference" (xllm-io review), section "核心公式": Pass-KV when the KV-cache miss rate exceeds
2 N_KV / N_H or when SendRecv hides behind attention compute, Pass-Q otherwise.

Pinned against the page's own figures: the threshold is 12.5% for 128 query heads and 8 KV heads;
the measured switch point is T=6400 new tokens on P=121600 cached (5%, the Pass-KV vs Pass-Q
latency table)."""
import pytest

from context_ring_attention_amd import binding as cp

FAST = dict(link_bytes_per_s=1e15, attn_flops_per_s=1e12)   # transfer always hidden
SLOW = dict(link_bytes_per_s=1.0, attn_flops_per_s=1e18)    # transfer never hidden


def test_condition_one_threshold_is_two_nkv_over_nh():
    # 128 query heads, 8 KV heads: threshold 2 * 8 / 128 = 12.5% of the total context
    total = 128000
    above = int(total * 0.13)
    below = int(total * 0.12)
    assert cp.select_ring_variant(above, total - above, 4, 128, 8, 128, 2, **SLOW) == ("pass_kv", 1)
    assert cp.select_ring_variant(below, total - below, 4, 128, 8, 128, 2, **SLOW) == ("pass_q", 0)
    # exactly at the threshold is not "above"
    assert cp.select_ring_variant(16000, 112000, 4, 128, 8, 128, 2, **SLOW) == ("pass_q", 0)
    # per-GPU head share 16:1 gives the same threshold
    assert cp.select_ring_variant(16001, 111999, 4, 16, 1, 128, 2, **SLOW) == ("pass_kv", 1)


def test_condition_two_hidden_transfer_picks_pass_kv():
    # the persistent-KV workload (8K new on 120K cached, miss 6.25%): condition 1 fails, so the
    # choice follows whether one KV shard's transfer hides behind one step's attention
    assert cp.select_ring_variant(8192, 122880, 4, 16, 1, 128, 2, **FAST) == ("pass_kv", 2)
    assert cp.select_ring_variant(8192, 122880, 4, 16, 1, 128, 2, **SLOW) == ("pass_q", 0)


def test_switch_point_of_the_measurements_is_where_the_models_cross():
    # At the page's measured switch point (T=6400, P=121600) the two conditions balance: choose
    # link and compute rates that make transfer time == compute time there, then check that a
    # little more new work (T=7000) picks Pass-KV and a little less (T=5800) picks Pass-Q.
    N, n_h, n_kv, d, e = 4, 128, 8, 128, 2
    T, P = 6400, 121600
    kv_bytes = 2.0 * (T + P) / N * n_kv * d * e
    flops = 4.0 * d * n_h * (T / N) * ((T + P) / N - T / (2.0 * N))
    link, rate = kv_bytes, flops       # one second each at the switch point
    assert cp.select_ring_variant(7000, 128000 - 7000, N, n_h, n_kv, d, e, link, rate)[0] == "pass_kv"
    assert cp.select_ring_variant(5800, 128000 - 5800, N, n_h, n_kv, d, e, link, rate)[0] == "pass_q"


def test_selector_rejects_bad_arguments():
    with pytest.raises(cp.CpError):
        cp.select_ring_variant(0, 10, 4, 16, 1, 128, 2, **FAST)
    with pytest.raises(cp.CpError):
        cp.select_ring_variant(10, 10, 4, 6, 4, 128, 2, **FAST)
    with pytest.raises(cp.CpError):
        cp.select_ring_variant(10, 10, 4, 16, 1, 128, 2, link_bytes_per_s=0.0, attn_flops_per_s=1.0)
