/*
 * oracle.h -- fp64 CPU oracle for one context-parallel rank's exact attention.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg, never by the product path. Shares nothing with the HIP library.
 * Definitions and the pages they follow are documented in oracle.c.
 */
#ifndef CP_ORACLE_H
#define CP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int orc_num_threads(void);

/* Tokens owned by `rank` under load-balanced sharding, in local order.
   Returns 0, 1 if max_tokens was too small (n_tokens still set), -1 on bad arguments. */
int orc_shard_tokens(int n_ranges, const int32_t* seq_id, const int64_t* range_begin,
                     const int64_t* range_end, int cp_world, int rank, int32_t* tok_seq,
                     int64_t* tok_pos, int64_t* tok_global, int64_t max_tokens,
                     int64_t* n_tokens);

/* Exact (partial) attention of query tokens over the given keys, fp64. */
int orc_attention(const float* q, const float* k, const float* v, int64_t tq, int64_t tk,
                  int n_h, int n_kv, int d_h, const int32_t* q_seq, const int64_t* q_pos,
                  const int32_t* k_seq, const int64_t* k_pos, int causal, double scale,
                  const int64_t* rows, int64_t n_rows, double* o, double* lse);

/* LSE-weighted merge of n partial (O, LSE) results, fp64. */
void orc_merge(int n_parts, const double* const* o_parts, const double* const* lse_parts,
               int64_t rows, int d_h, double* o, double* lse);

/* Key range [lo, hi) of decode split c out of n_splits for a request with len cached keys. */
void orc_split_bounds(int64_t len, int n_splits, int c, int64_t* lo, int64_t* hi);

/* Gradients (fp64) of the partial attention of query tokens over the given keys, from the final
   forward output o and lse and the output gradient d_o. Returns -1 on bad arguments. */
int orc_attention_backward(const float* q, const float* k, const float* v, int64_t tq, int64_t tk,
                           int n_h, int n_kv, int d_h, const int32_t* q_seq, const int64_t* q_pos,
                           const int32_t* k_seq, const int64_t* k_pos, int causal, double scale,
                           const double* o, const double* lse, const float* d_o, double* dq,
                           double* dk, double* dv);

/* Ring schedules: KV shard rank `rank` holds at Pass-KV step `step`; Q shard hosted by the owner of
   KV shard `kv_shard` at Pass-Q step `step`; storage slot of the partial (q_shard, kv_shard).
   Each returns -1 on bad arguments. */
int orc_pass_kv_shard(int cp_world, int rank, int step);
int orc_pass_q_query(int cp_world, int kv_shard, int step);
int orc_pass_q_slot(int cp_world, int q_shard, int kv_shard);

#ifdef __cplusplus
}
#endif
#endif
