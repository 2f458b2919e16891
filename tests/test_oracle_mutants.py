"""The oracle's pins are not vacuous: plausible mistakes planted in a copy of oracle.c must each
fail at least one of them (CPU only).

Each mutant is one textual change of oracle.c (a dropped term, a wrong sign or index, a
transposed operand, a wrong chunk or split rule), compiled with gcc into a temporary library.
All oracle calls are routed through it, and the pins of test_oracle.py and
test_oracle_shard_map.py run unchanged. The replaced text must occur in oracle.c, so a later
edit of the oracle cannot silently turn a mutant into a no-op. Every mutant keeps all memory
accesses in bounds.
"""
import subprocess

import pytest

import oracle
import test_oracle as T
import test_oracle_backward as B
import test_oracle_shard_map as S

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

MUTANTS = [
    ("causal mask also hides the query's own key", "k_pos[j] > q_pos[t]", "k_pos[j] >= q_pos[t]"),
    ("causal mask ignored", "if (causal && k_pos[j] > q_pos[t]) continue;", ""),
    ("sequence boundaries ignored", "if (k_seq[j] != q_seq[t]) continue;", ""),
    ("GQA heads interleaved instead of consecutive", "int g = h / group;", "int g = h % n_kv;"),
    ("softmax scale dropped", "s *= scale;", "s *= 1.0;"),
    ("LSE without the max", "lse[r * n_h + h] = m + log(l);", "lse[r * n_h + h] = log(l);"),
    ("output not normalised", "out[d] = acc[d] / l;", "out[d] = acc[d];"),
    ("values read from K", "acc[d] += w * (double)vv[d];", "acc[d] += w * (double)kv[d];"),
    ("empty visible set gives LSE 0", "lse[r * n_h + h] = -INFINITY;", "lse[r * n_h + h] = 0.0;"),
    ("query rows read head-major", "const float* qv = q + (t * n_h + h) * (int64_t)d_h;",
     "const float* qv = q + (h * tq + t) * (int64_t)d_h;"),
    ("merge weights not shifted by the max", "double w = exp(lse_parts[i][r] - M);",
     "double w = exp(lse_parts[i][r]);"),
    ("merged LSE without the max", "lse[r] = M + log(wsum);", "lse[r] = log(wsum);"),
    ("merged O not normalised", "o[r * d_h + d] /= wsum;", "o[r * d_h + d] /= 1.0;"),
    ("second chunk not mirrored", "int64_t picks[2] = {rank, n_chunks - 1 - rank};",
     "int64_t picks[2] = {rank, rank + cp_world};"),
    ("mirrored chunk off by one", "int64_t picks[2] = {rank, n_chunks - 1 - rank};",
     "int64_t picks[2] = {rank, (n_chunks - rank) % n_chunks};"),
    ("global index ignores earlier sequences", "base[s] = base[s - 1] + seq_len[s - 1];", "base[s] = 0;"),
    ("decode splits drop the remainder", "*hi = ((int64_t)(c + 1) * len) / n_splits;",
     "*hi = *lo + len / n_splits;"),
    ("decode split edges rounded up",
     "*lo = ((int64_t)c * len) / n_splits;\n  *hi = ((int64_t)(c + 1) * len) / n_splits;",
     "*lo = ((int64_t)c * len + n_splits - 1) / n_splits;\n"
     "  *hi = ((int64_t)(c + 1) * len + n_splits - 1) / n_splits;"),
    ("chunk edges rounded up",
     "int64_t lo = a + (c * len) / n_chunks;\n      int64_t hi = a + ((c + 1) * len) / n_chunks;",
     "int64_t lo = a + (c * len + n_chunks - 1) / n_chunks;\n"
     "      int64_t hi = a + ((c + 1) * len + n_chunks - 1) / n_chunks;"),
    ("Pass-KV ring runs backwards", "return ring_mod(rank - step, cp_world);",
     "return ring_mod(rank + step, cp_world);"),
    ("Pass-Q hosts the KV shard's own Q at every step", "return ring_mod(kv_shard - step, cp_world);",
     "return kv_shard;"),
    ("Pass-Q slots transposed", "return q_shard * cp_world + kv_shard;",
     "return kv_shard * cp_world + q_shard;"),
    ("backward: score gradient with the wrong sign", "double ds = p * (dp - D);",
     "double ds = p * (D - dp);"),
    ("backward: dQ without the scale", "dqr[d] += scale * ds * (double)kv[d];",
     "dqr[d] += ds * (double)kv[d];"),
    ("backward: dK from the key instead of the query", "dkr[d] += scale * ds * (double)qv[d];",
     "dkr[d] += scale * ds * (double)kv[d];"),
    ("backward: weights without the final LSE", "double p = exp(s * scale - L);",
     "double p = exp(s * scale);"),
    ("backward: dV from the score gradient", "dvr[d] += p * (double)gv[d];",
     "dvr[d] += ds * (double)gv[d];"),
    ("backward: D from dO alone", "D += (double)d_o[r * d_h + d] * o[r * d_h + d];",
     "D += (double)d_o[r * d_h + d];"),
    ("backward: causal mask ignored", "if (causal && q_pos[t] < k_pos[j]) continue;", ""),
    ("backward: GQA heads interleaved", "int kvh = h / group;", "int kvh = h % n_kv;"),
    ("backward: dK/dV from the wrong query heads", "if (h / group != g) continue;",
     "if (h % n_kv != g) continue;"),
]

PINS = [
    ("merge of key partitions", lambda: T.test_merge_of_any_key_partition_equals_unsharded(0)),
    ("uniform values", T.test_uniform_values_give_that_value_for_every_row_and_shard),
    ("zero query", T.test_zero_query_gives_running_mean_and_log_count),
    ("one-hot key a=0.7", lambda: T.test_one_hot_key_closed_form(0.7)),
    ("one-hot key a=5", lambda: T.test_one_hot_key_closed_form(5.0)),
    ("first token", T.test_first_token_of_each_sequence_sees_only_itself),
    ("dense brute force, causal", lambda: T.test_dense_brute_force_agrees(True)),
    ("dense brute force, full", lambda: T.test_dense_brute_force_agrees(False)),
    ("GQA grouping", T.test_gqa_consecutive_heads_share_kv_head),
    ("row subset", T.test_partial_over_rows_subset_matches_full),
    ("empty set and empty merge", T.test_empty_visible_set_and_merge_of_nothing),
    ("merge identity and ln 2", T.test_merge_single_part_is_identity_and_two_equal_parts_add_ln2),
    ("decode splits", T.test_decode_splits_cover_keys_and_merge_exactly),
    ("golden decode split table", T.test_decode_split_table_golden_l300_s32),
    ("backward finite differences", lambda: B.test_finite_differences_of_the_forward(True)),
    ("backward autograd", lambda: B.test_matches_torch_autograd_on_a_dense_formulation(2, True)),
    ("backward partition sums", lambda: B.test_contributions_over_a_key_partition_sum_to_the_full_gradient(3)),
    ("backward uniform V", B.test_uniform_values_give_zero_score_gradients_and_dv_sums_to_do),
    ("backward zero query", B.test_zero_query_gives_uniform_weights),
    ("backward GQA", B.test_gqa_gradients_come_from_the_heads_of_the_group),
    ("golden shard map", S.test_golden_t256_cp4_layout_and_pair_counts),
    ("golden shard map, T=257", S.test_golden_t257_cp4_floor_edges_and_pair_counts),
    ("golden ring schedules", S.test_golden_ring_schedules_cp4),
    ("rings, N=5", lambda: S.test_ring_schedules_are_rings(5)),
    ("ranks partition ranges", lambda: S.test_ranks_partition_every_range_with_balanced_counts(257, 4)),
    ("equal compute per rank", S.test_equal_compute_per_rank_when_divisible),
    ("persistent-KV layout", S.test_persistent_kv_layout_per_rank),
    ("varlen global index", S.test_varlen_batch_global_index_and_segments),
]


def _failing_pins():
    failed = []
    for name, pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, RuntimeError, IndexError):
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_every_pin():
    oracle.use_library(None)
    assert _failing_pins() == []


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(what, old, new, tmp_path):
    src = open(oracle._SRC).read()
    assert old in src, f"mutant '{what}' no longer applies to oracle.c"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-I", oracle._HERE,
                    "-o", str(lib), str(mutated), "-lm"], check=True)
    oracle.use_library(str(lib))
    try:
        failed = _failing_pins()
    finally:
        oracle.use_library(None)
    print(f"{what}: caught by {failed}")
    assert failed, f"no pin catches the planted mistake: {what}"
