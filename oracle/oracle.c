/*
 * oracle.c -- plain, slow, fp64 CPU oracle for one context-parallel rank's exact attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py may load or call this library. It shares no code, header, table or helper with the
 * HIP path in context_ring_attention_amd/, and it never includes anything from there.
 *
 * Pages cited (titles as published):
 *   [CPEP]  "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두 축"
 *           (m1ser4ble.github.io blog post).
 *   [CPMTI] "Context Parallelism for Scalable Million-Token Inference"
 *           (xllm-io.github.io paper review of arXiv 2411.01783).
 *
 * Every function is the plain definition written out: no blocking, no online rescaling, no
 * fusion. Arithmetic is fp64 on inputs widened exactly from their fp32 (or bf16-rounded fp32)
 * values. Threads only split independent output rows (OpenMP); each row is computed serially.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------------------------
 * Load-balanced sharding.  [CPMTI §4 "负载均衡分片策略" with Fig. 2; the figure itself is not in the
 * page text]: every CP rank gets about equal attention compute and equal KV memory, and a batch
 * may hold sequences of different lengths.  Reading taken (the figure is missing): a range
 * [a, b) of length L is cut into 2N chunks, chunk c = [a + floor(c*L/2N), a + floor((c+1)*L/2N)),
 * and rank r owns chunk r followed by chunk 2N-1-r.  Ranges are visited in the order given.
 * The global index of (seq s, position p) is base[s] + p, where base[s] is the sum of the
 * lengths of sequences 0..s-1 and the length of a sequence is the largest range end given for it.
 * ------------------------------------------------------------------------------------------ */
int orc_shard_tokens(int n_ranges, const int32_t* seq_id, const int64_t* range_begin,
                     const int64_t* range_end, int cp_world, int rank, int32_t* tok_seq,
                     int64_t* tok_pos, int64_t* tok_global, int64_t max_tokens,
                     int64_t* n_tokens) {
  if (n_ranges < 0 || cp_world < 1 || rank < 0 || rank >= cp_world) return -1;
  int n_seq = 0;
  for (int i = 0; i < n_ranges; ++i) {
    int s = seq_id ? seq_id[i] : i;
    if (s < 0 || range_begin[i] < 0 || range_end[i] < range_begin[i]) return -1;
    if (s + 1 > n_seq) n_seq = s + 1;
  }
  int64_t* seq_len = (int64_t*)calloc((size_t)n_seq + 1, sizeof(int64_t));
  int64_t* base = (int64_t*)calloc((size_t)n_seq + 1, sizeof(int64_t));
  for (int i = 0; i < n_ranges; ++i) {
    int s = seq_id ? seq_id[i] : i;
    if (range_end[i] > seq_len[s]) seq_len[s] = range_end[i];
  }
  for (int s = 1; s <= n_seq; ++s) base[s] = base[s - 1] + seq_len[s - 1];

  int64_t count = 0;
  int64_t n_chunks = 2 * (int64_t)cp_world;
  for (int i = 0; i < n_ranges; ++i) {
    int s = seq_id ? seq_id[i] : i;
    int64_t a = range_begin[i];
    int64_t len = range_end[i] - range_begin[i];
    int64_t picks[2] = {rank, n_chunks - 1 - rank};
    for (int w = 0; w < 2; ++w) {
      int64_t c = picks[w];
      int64_t lo = a + (c * len) / n_chunks;
      int64_t hi = a + ((c + 1) * len) / n_chunks;
      for (int64_t p = lo; p < hi; ++p) {
        if (count < max_tokens) {
          if (tok_seq) tok_seq[count] = s;
          if (tok_pos) tok_pos[count] = p;
          if (tok_global) tok_global[count] = base[s] + p;
        }
        ++count;
      }
    }
  }
  free(seq_len);
  free(base);
  *n_tokens = count;
  return count <= max_tokens ? 0 : 1;
}

/* ------------------------------------------------------------------------------------------
 * Attention of query tokens over a set of keys.
 *
 * [CPEP §5.1]: the output of token t is softmax(q_t K^T) V over the keys it may see; under the
 *   causal mask q_t sees k_1..k_t (itself included) and never a later key.
 * [CPEP §5.2]: prefill has many query rows against the keys; decode has one new query against
 *   the whole cached K/V.
 * [CPEP §8.2]: in GQA, consecutive query heads share one K/V head (Q_0..Q_7 -> K_0, ...), so
 *   head h uses KV head h / (N_H / N_KV).
 * [CPMTI §3 "核心公式"]: Q is [T, N_H, D_H]; K and V are [T+P, N_KV, D_H].
 *
 * Readings (the pages leave these open): the scores carry an explicit scale (1/sqrt(D_H) in the
 * configurations; scale = 1 is the page's literal formula); key j is visible to query t iff
 * they belong to the same sequence and, when causal, pos(j) <= pos(t).  The key set passed in
 * may be any subset of a sequence (one KV shard, one decode split): the result is then the
 * partial attention over that subset, with LSE = m + ln(sum exp(s_j - m)) in natural log.  An
 * empty visible set gives O = 0 and LSE = -inf.
 *
 * q: [tq, n_h, d_h], k, v: [tk, n_kv, d_h] (fp32 values, widened to fp64).
 * rows (optional): the query tokens to compute; outputs are then [n_rows, n_h, d_h] / [n_rows, n_h].
 * ------------------------------------------------------------------------------------------ */
int orc_attention(const float* q, const float* k, const float* v, int64_t tq, int64_t tk,
                  int n_h, int n_kv, int d_h, const int32_t* q_seq, const int64_t* q_pos,
                  const int32_t* k_seq, const int64_t* k_pos, int causal, double scale,
                  const int64_t* rows, int64_t n_rows, double* o, double* lse) {
  if (n_h < 1 || n_kv < 1 || n_h % n_kv != 0 || d_h < 1) return -1;
  int group = n_h / n_kv;
  int64_t n_out = rows ? n_rows : tq;
  int64_t total = n_out * (int64_t)n_h;
  int bad = 0;

#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t idx = 0; idx < total; ++idx) {
    int64_t r = idx / n_h;
    int h = (int)(idx % n_h);
    int64_t t = rows ? rows[r] : r;
    if (t < 0 || t >= tq) {
      bad = 1;
      continue;
    }
    int g = h / group;
    const float* qv = q + (t * n_h + h) * (int64_t)d_h;
    double* out = o + (r * n_h + h) * (int64_t)d_h;
    double* acc = (double*)calloc((size_t)d_h, sizeof(double));

    /* pass 1: the largest visible score */
    double m = -INFINITY;
    int64_t visible = 0;
    for (int64_t j = 0; j < tk; ++j) {
      if (k_seq[j] != q_seq[t]) continue;
      if (causal && k_pos[j] > q_pos[t]) continue;
      const float* kv = k + (j * n_kv + g) * (int64_t)d_h;
      double s = 0.0;
      for (int d = 0; d < d_h; ++d) s += (double)qv[d] * (double)kv[d];
      s *= scale;
      if (s > m) m = s;
      ++visible;
    }
    if (visible == 0) {
      for (int d = 0; d < d_h; ++d) out[d] = 0.0;
      lse[r * n_h + h] = -INFINITY;
      free(acc);
      continue;
    }

    /* pass 2: softmax weights and the weighted sum of values */
    double l = 0.0;
    for (int64_t j = 0; j < tk; ++j) {
      if (k_seq[j] != q_seq[t]) continue;
      if (causal && k_pos[j] > q_pos[t]) continue;
      const float* kv = k + (j * n_kv + g) * (int64_t)d_h;
      const float* vv = v + (j * n_kv + g) * (int64_t)d_h;
      double s = 0.0;
      for (int d = 0; d < d_h; ++d) s += (double)qv[d] * (double)kv[d];
      s *= scale;
      double w = exp(s - m);
      l += w;
      for (int d = 0; d < d_h; ++d) acc[d] += w * (double)vv[d];
    }
    for (int d = 0; d < d_h; ++d) out[d] = acc[d] / l;
    lse[r * n_h + h] = m + log(l);
    free(acc);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------------------------
 * Merge of partial attention results.  [CPMTI §3 "核心公式" (Pass-Q ends with an All2All merge of
 * partial attention results) and §5 "关键实现细节" item 3 (merge attention)]; the page does not
 * print the formula but calls both ring variants lossless and exact [CPMTI §2 "解决方案概述"].
 * Reading: the combine that is exact for any split of a row's visible keys,
 *   M = max_i LSE_i,  w_i = exp(LSE_i - M),  LSE = M + ln(sum_i w_i),  O = sum_i w_i O_i / sum_i w_i,
 * with M = -inf (no part saw a key) giving O = 0 and LSE = -inf.
 * o_parts[i]: [rows, d_h], lse_parts[i]: [rows].
 * ------------------------------------------------------------------------------------------ */
void orc_merge(int n_parts, const double* const* o_parts, const double* const* lse_parts,
               int64_t rows, int d_h, double* o, double* lse) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double M = -INFINITY;
    for (int i = 0; i < n_parts; ++i)
      if (lse_parts[i][r] > M) M = lse_parts[i][r];
    if (M == -INFINITY) {
      for (int d = 0; d < d_h; ++d) o[r * d_h + d] = 0.0;
      lse[r] = -INFINITY;
      continue;
    }
    double wsum = 0.0;
    for (int d = 0; d < d_h; ++d) o[r * d_h + d] = 0.0;
    for (int i = 0; i < n_parts; ++i) {
      double w = exp(lse_parts[i][r] - M);
      wsum += w;
      for (int d = 0; d < d_h; ++d) o[r * d_h + d] += w * o_parts[i][r * d_h + d];
    }
    for (int d = 0; d < d_h; ++d) o[r * d_h + d] /= wsum;
    lse[r] = M + log(wsum);
  }
}

/* ------------------------------------------------------------------------------------------
 * Decode split bounds.  [CPMTI §5 "软件栈": Flash Decoding with 256 splits for decode.]
 * Reading: split c of a request with L cached keys covers [floor(c*L/S), floor((c+1)*L/S)).
 * ------------------------------------------------------------------------------------------ */
void orc_split_bounds(int64_t len, int n_splits, int c, int64_t* lo, int64_t* hi) {
  *lo = ((int64_t)c * len) / n_splits;
  *hi = ((int64_t)(c + 1) * len) / n_splits;
}

/* ------------------------------------------------------------------------------------------
 * Ring schedules.  [CPMTI §3 "核心公式", Fig. 3]: in ring Pass-KV each rank keeps its Q shard while
 * the KV shards travel around the ring of N ranks for N-1 rounds; in ring Pass-Q the KV shards
 * stay on their ranks, the Q shards travel, and an All2All then returns every partial result to
 * the rank that owns its Q shard, where the partials are merged.
 * Readings (the page fixes neither the direction nor the storage order; O and LSE do not depend
 * on them): a shard moves from rank r to rank r+1 at every step, so at step t
 *   - Pass-KV: rank r holds the KV shard that started on rank (r - t) mod N;
 *   - Pass-Q: the rank that owns KV shard s hosts the Q shard that started on rank (s - t) mod N;
 * and the partial of Q shard q against KV shard s is stored in slot q*N + s.
 * ------------------------------------------------------------------------------------------ */
static int ring_mod(int a, int n) { return ((a % n) + n) % n; }

int orc_pass_kv_shard(int cp_world, int rank, int step) {
  if (cp_world < 1 || rank < 0 || rank >= cp_world || step < 0) return -1;
  return ring_mod(rank - step, cp_world);
}

int orc_pass_q_query(int cp_world, int kv_shard, int step) {
  if (cp_world < 1 || kv_shard < 0 || kv_shard >= cp_world || step < 0) return -1;
  return ring_mod(kv_shard - step, cp_world);
}

int orc_pass_q_slot(int cp_world, int q_shard, int kv_shard) {
  if (cp_world < 1 || q_shard < 0 || q_shard >= cp_world || kv_shard < 0 || kv_shard >= cp_world)
    return -1;
  return q_shard * cp_world + kv_shard;
}

/* ------------------------------------------------------------------------------------------
 * Backward of the partial attention of query tokens over a set of keys.
 * [CPEP §6]: with CP the forward gathers K/V for each rank's Q chunk, and the backward sends the
 * K/V gradient contributions back to the ranks that own those K/V chunks (a reduce-scatter, i.e.
 * a sum per chunk).  On the ring, each step's gradient contribution is that of the step's key
 * subset.
 * Definition (the gradient of O = softmax(scale * q.K^T) V written out, [CPEP §5.1]): for row
 * (t, h) with the FINAL output O and log-sum-exp LSE over all the keys the row sees (every shard),
 * and every key j of the given subset visible to it,
 *   p_j  = exp(s_j - LSE)                  (its softmax weight in the full attention)
 *   dp_j = sum_d dO[d] V[j][d]
 *   D    = sum_d dO[d] O[d]                (= sum over all visible keys of p_j dp_j)
 *   ds_j = p_j (dp_j - D)
 *   dQ[t][h]  += scale * ds_j * K[j]
 *   dK[j][g]  += scale * ds_j * Q[t][h]     (g = the row's KV head)
 *   dV[j][g]  += p_j * dO[t][h]
 * Summed over a partition of the keys these contributions give the full gradient, which is what
 * makes the per-shard reduce-scatter exact.  Rows with LSE = -inf saw no key and contribute 0.
 * q: [tq, n_h, d_h]; k, v: [tk, n_kv, d_h] (fp32 values); o: [tq, n_h, d_h] and lse: [tq, n_h]
 * (fp64, the final forward results); d_o: [tq, n_h, d_h] (fp32 values).  Outputs (fp64, written,
 * not accumulated): dq [tq, n_h, d_h], dk and dv [tk, n_kv, d_h].
 * Plain loops in two passes over the same per-pair terms: pass 1 (rows in parallel) sums dQ of
 * each row over its visible keys; pass 2 (keys in parallel) sums dK and dV of each key over the
 * rows that see it.  The score gradient of a (row, key) pair is computed the same way in both.
 * ------------------------------------------------------------------------------------------ */
/* Terms of one visible (row t, head h; key j) pair of the backward: p = exp(s - LSE) and
 * ds = p * (dO.V[j] - D).  kvh is the row's KV head; D = dO.O of the row. */
static void bwd_pair(const float* qv, const float* gv, const float* kv, const float* vv, int d_h,
                     double scale, double L, double D, double* p_out, double* ds_out) {
  double s = 0.0, dp = 0.0;
  for (int d = 0; d < d_h; ++d) {
    s += (double)qv[d] * (double)kv[d];
    dp += (double)gv[d] * (double)vv[d];
  }
  double p = exp(s * scale - L);
  double ds = p * (dp - D);
  *p_out = p;
  *ds_out = ds;
}

int orc_attention_backward(const float* q, const float* k, const float* v, int64_t tq, int64_t tk,
                           int n_h, int n_kv, int d_h, const int32_t* q_seq, const int64_t* q_pos,
                           const int32_t* k_seq, const int64_t* k_pos, int causal, double scale,
                           const double* o, const double* lse, const float* d_o, double* dq,
                           double* dk, double* dv) {
  if (n_h < 1 || n_kv < 1 || n_h % n_kv != 0 || d_h < 1) return -1;
  int group = n_h / n_kv;
  /* D of every row */
  double* Drow = (double*)calloc((size_t)(tq * n_h) + 1, sizeof(double));
  for (int64_t r = 0; r < tq * n_h; ++r) {
    double D = 0.0;
    for (int d = 0; d < d_h; ++d) D += (double)d_o[r * d_h + d] * o[r * d_h + d];
    Drow[r] = D;
  }
  /* pass 1: dQ of each row over its visible keys */
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < tq * n_h; ++r) {
    int64_t t = r / n_h;
    int h = (int)(r % n_h);
    int kvh = h / group; /* the row's KV head */
    double* dqr = dq + r * (int64_t)d_h;
    for (int d = 0; d < d_h; ++d) dqr[d] = 0.0;
    double L = lse[r];
    if (L == -INFINITY) continue;
    const float* qv = q + r * (int64_t)d_h;
    const float* gv = d_o + r * (int64_t)d_h;
    for (int64_t j = 0; j < tk; ++j) {
      if (k_seq[j] != q_seq[t]) continue;
      if (causal && q_pos[t] < k_pos[j]) continue; /* a later key is invisible */
      const float* kv = k + (j * n_kv + kvh) * (int64_t)d_h;
      const float* vv = v + (j * n_kv + kvh) * (int64_t)d_h;
      double p, ds;
      bwd_pair(qv, gv, kv, vv, d_h, scale, L, Drow[r], &p, &ds);
      for (int d = 0; d < d_h; ++d) dqr[d] += scale * ds * (double)kv[d];
    }
  }
  /* pass 2: dK and dV of each key over the rows that see it */
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t c = 0; c < tk * n_kv; ++c) {
    int64_t j = c / n_kv;
    int g = (int)(c % n_kv);
    double* dkr = dk + c * (int64_t)d_h;
    double* dvr = dv + c * (int64_t)d_h;
    for (int d = 0; d < d_h; ++d) dkr[d] = dvr[d] = 0.0;
    const float* kv = k + c * (int64_t)d_h;
    const float* vv = v + c * (int64_t)d_h;
    for (int64_t t = 0; t < tq; ++t) {
      if (k_seq[j] != q_seq[t]) continue;
      if (causal && q_pos[t] < k_pos[j]) continue;
      for (int h = 0; h < n_h; ++h) {
        if (h / group != g) continue; /* only the query heads of this KV head */
        int64_t r = t * n_h + h;
        double L = lse[r];
        if (L == -INFINITY) continue;
        const float* qv = q + r * (int64_t)d_h;
        const float* gv = d_o + r * (int64_t)d_h;
        double p, ds;
        bwd_pair(qv, gv, kv, vv, d_h, scale, L, Drow[r], &p, &ds);
        for (int d = 0; d < d_h; ++d) {
          dkr[d] += scale * ds * (double)qv[d];
          dvr[d] += p * (double)gv[d];
        }
      }
    }
  }
  free(Drow);
  return 0;
}
