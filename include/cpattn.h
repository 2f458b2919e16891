/*
 * cpattn.h -- C ABI of the MI355X (gfx950) context-parallel ring attention library.
 *
 * One context-parallel (CP) rank's exact GQA attention: a query shard attends, block by block, to
 * each key/value shard of the ring; each step yields a partial output plus its log-sum-exp, and
 * the partials are merged without loss. Decode splits the KV cache and merges the same way.
 *
 * Pages cited (titles as published):
 *   [CPEP]  "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두 축"
 *           (m1ser4ble.github.io blog post).
 *   [CPMTI] "Context Parallelism for Scalable Million-Token Inference"
 *           (xllm-io.github.io review of arXiv 2411.01783).
 *
 * Conventions for every entry point:
 *  - Memory is owned by the caller. The library never allocates, frees or synchronises device
 *    memory; "device" pointers must point to memory on the current HIP device.
 *  - Calls enqueue work on `stream` (a hipStream_t; NULL = the default stream) and return. The
 *    return value reports argument validation and launch errors only; faults during execution
 *    show up at the caller's next synchronisation.
 *  - On a negative status nothing was launched and no output was written; cp_last_error() holds
 *    a message (thread-local).
 *  - Layouts are dense and row-major: Q [T_q, N_H, D_H], K and V [T_k, N_KV, D_H] ([CPMTI §3
 *    "核心公式"]). Query head h reads KV head h / (N_H / N_KV): consecutive heads share a KV head
 *    ([CPEP §8.2]).
 *  - Scores are softmax_scale * q.k; LSE is the natural-log log-sum-exp of those scores over the
 *    keys a row saw. A row that saw no key has O = 0 and LSE = -inf.
 *  - Supported: D_H in {64, 128}; inputs fp32 or bf16; token counts below 2^31.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CP_OK = 0,
  CP_E_ARG = -1,         /* null pointer, negative size, bad enum value */
  CP_E_SHAPE = -2,       /* inconsistent shapes (N_H % N_KV != 0, segment outside its shard, ...) */
  CP_E_UNSUPPORTED = -3, /* valid but not implemented (D_H not 64/128, dtype combination) */
  CP_E_CAPACITY = -4,    /* an output buffer or a fixed table is too small */
  CP_E_HIP = -5          /* the HIP runtime reported an error at launch */
} cp_status;

typedef enum { CP_F32 = 0, CP_BF16 = 1 } cp_dtype;

/* A run of tokens of one sequence stored contiguously in a shard: shard rows
   [local_start, local_start + len) hold positions [pos_start, pos_start + len) of sequence
   seq_id. Positions count from 0 at the first token of the sequence (cached tokens first). */
typedef struct {
  int32_t seq_id;
  int32_t reserved; /* set to 0 */
  int64_t pos_start;
  int64_t len;
  int64_t local_start;
} cp_segment;

/* Runs of a segment table one kernel launch takes (tables travel in kernel arguments). Longer
   tables are accepted (up to 2^20 runs) and split over several launches: the Q runs in groups of
   whole sequences, each with only its own sequences' KV runs, and KV runs beyond this count of one
   group folded in by further launches in order. */
#define CP_MAX_SEGMENTS 64
/* Largest number of parts cp_merge_lse merges in one call. */
#define CP_MAX_MERGE_PARTS 64

/* ---------------------------------------------------------------------------------------------
 * cp_shard_map -- load-balanced sharding ([CPMTI §4 "负载均衡分片策略", Fig. 2]: each rank gets
 * equal attention compute and equal KV memory; batches of different lengths are supported).
 * Each range [range_begin[i], range_end[i]) of sequence seq_id[i] (seq_id NULL: sequence i) is
 * cut into 2*cp_world chunks with edges begin + floor(c*L/(2*cp_world)); rank `rank` owns chunk
 * `rank` and chunk 2*cp_world-1-rank. Ranges are visited in order, and each owned non-empty chunk
 * becomes one segment, in that order. Host-only, integer, launches nothing.
 *   segs_out:   host, caller-owned, capacity max_segs; *n_segs_out = segments needed.
 *   tokens_out: optional (NULL ok), host, capacity max_tokens: for each local token in order, its
 *               packed global index base[seq] + pos, where base[s] is the sum of the lengths of
 *               sequences 0..s-1 and a sequence's length is the largest range_end given for it.
 *               *n_tokens_out (optional) = local token count.
 * Returns CP_E_CAPACITY (with the counts set) if a buffer is too small, CP_E_ARG on bad ranges,
 * CP_E_UNSUPPORTED if a range is so long that its chunk edges (c * L / 2N) overflow 64 bits.
 * ------------------------------------------------------------------------------------------- */
int cp_shard_map(int n_ranges, const int32_t* seq_id, const int64_t* range_begin,
                 const int64_t* range_end, int cp_world, int rank, cp_segment* segs_out,
                 int max_segs, int* n_segs_out, int64_t* tokens_out, int64_t max_tokens,
                 int64_t* n_tokens_out);

/* ---------------------------------------------------------------------------------------------
 * cp_partial_attn -- one ring step: exact attention of a Q shard over one KV shard, producing
 * the partial output and its LSE ([CPMTI §3 "核心公式": each rank computes the partial attention
 * of its local Q against the KV it holds; [CPEP §5.1] per-token attention and causal mask;
 * [CPEP §4.1]/§6 block-wise attention with online softmax).
 *   q: device [tq, n_h, d_h]; k, v: device [tk, n_kv, d_h]; dtype in_dtype (all three).
 *   q_segs / kv_segs: host tables (any length up to 2^20 runs; see CP_MAX_SEGMENTS) describing
 *     which sequence and positions every shard row holds; rows outside all segments are not read
 *     or written.
 *   causal: key visible iff same sequence and key position <= query position; 0: same sequence.
 *   o: device fp32 [tq, n_h, d_h]; lse: device fp32 [tq, n_h].
 *   accumulate = 0: overwrite (o, lse) with this step's partial.
 *   accumulate = 1: (o, lse) hold a running partial; merge this step into it in place.
 * bf16 inputs run on MFMA with fp32 accumulation (probabilities rounded to bf16 before P.V);
 * fp32 inputs run in fp32 arithmetic throughout.
 * ------------------------------------------------------------------------------------------- */
int cp_partial_attn(const void* q, const void* k, const void* v, int64_t tq, int64_t tk, int n_h,
                    int n_kv, int d_h, cp_dtype in_dtype, const cp_segment* q_segs, int n_q_segs,
                    const cp_segment* kv_segs, int n_kv_segs, int causal, float softmax_scale,
                    float* o, float* lse, int accumulate, void* stream);

/* ---------------------------------------------------------------------------------------------
 * cp_merge_lse -- lossless merge of partial results ([CPMTI §3 "核心公式": Pass-Q ends with an
 * All2All merge of partial attention; §5 "关键实现细节" item 3, merge attention; the variants are
 * exact, §2 "解决方案概述"). Per row: M = max_i LSE_i, w_i = exp(LSE_i - M),
 * O = sum_i w_i O_i / sum_i w_i, LSE = M + ln(sum_i w_i); rows no part saw give O = 0, LSE = -inf.
 *   o_parts, lse_parts: host arrays of n_parts (1..CP_MAX_MERGE_PARTS) device pointers to fp32
 *     [rows, d_h] and [rows]. rows = T_q * N_H.
 *   o_out: device [rows, d_h] in out_dtype (fp32 or bf16, round to nearest even);
 *   lse_out: device fp32 [rows] (may be NULL). Merging in place is allowed: o_out may alias a part's
 *     O when out_dtype is fp32, and lse_out may alias a part's LSE (each row is read before it is
 *     written, by the same wave).
 * ------------------------------------------------------------------------------------------- */
int cp_merge_lse(int n_parts, const float* const* o_parts, const float* const* lse_parts,
                 int64_t rows, int d_h, void* o_out, cp_dtype out_dtype, float* lse_out,
                 void* stream);

/* ---------------------------------------------------------------------------------------------
 * cp_decode_splitkv -- decode attention, one new query token per request against its KV cache,
 * split n_splits ways and merged ([CPMTI §5 "软件栈": Flash Decoding with 256 splits; §4 decode
 * uses ring Pass-Q; [CPEP §5.2] decode: one q against the whole cache).
 *   q: device [batch, n_h, d_h]; k_cache, v_cache: device [sum L_b, n_kv, d_h], request b at rows
 *     [kv_offset[b], kv_offset[b] + kv_len[b]); kv_offset, kv_len: device int64 [batch].
 *   Split c of request b covers cache rows [floor(c*L_b/S), floor((c+1)*L_b/S)); every cached key
 *   is visible (the query comes after the cache).
 *   ws_o: device fp32 [batch, n_splits, n_h, d_h], ws_lse: device fp32 [batch, n_splits, n_h]:
 *     the per-split partials (O normalised over the split's keys, and its LSE). They are merged
 *     in fp32, so the result is the exact combine of the splits ([CPMTI §2]: the ring variants
 *     are lossless). Caller-owned; cp_decode_workspace_bytes gives the size of one buffer holding
 *     ws_o then ws_lse (at byte offset batch*n_splits*n_h*d_h*4). ws_o is 16-byte aligned.
 *   o_out: device [batch, n_h, d_h] in out_dtype; lse_out: device fp32 [batch, n_h] (may be NULL).
 * in_dtype must be CP_BF16. 1 <= n_splits <= 1024.
 * kv_offset and kv_len live in device memory and are read by the kernels, not checked on the host:
 * the caller guarantees kv_offset[b] >= 0 and kv_offset[b] + kv_len[b] <= the cache's rows. A
 * negative kv_len[b] is read as an empty cache (O = 0, LSE = -inf). The workspace holds one call's
 * partials: calls that share it must be ordered (same stream), not overlap.
 * ------------------------------------------------------------------------------------------- */
int cp_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                      const int64_t* kv_offset, const int64_t* kv_len, int batch, int n_h,
                      int n_kv, int d_h, cp_dtype in_dtype, int n_splits, float softmax_scale,
                      float* ws_o, float* ws_lse, void* o_out, cp_dtype out_dtype, float* lse_out,
                      void* stream);
size_t cp_decode_workspace_bytes(int batch, int n_h, int d_h, int n_splits);

/* cp_decode_splitkv_ex -- cp_decode_splitkv with the precision of the split workspace's partial O
 * chosen by the caller: ws_dtype CP_F32 (exactly cp_decode_splitkv) or CP_BF16, which halves the
 * partials' HBM traffic at the price of rounding each split's O to bf16 before the merge (a
 * relative 2^-9 of |V|, the precision the split's bf16 probabilities already carry). The LSEs stay
 * fp32. ws_o: device [batch, n_splits, n_h, d_h] in ws_dtype; cp_decode_workspace_bytes_ex sizes
 * the buffer (ws_lse at byte offset batch*n_splits*n_h*d_h*sizeof(ws_dtype)); returns 0 for a bad
 * ws_dtype. Other arguments and errors as cp_decode_splitkv (CP_E_ARG for a bad ws_dtype). */
int cp_decode_splitkv_ex(const void* q, const void* k_cache, const void* v_cache,
                         const int64_t* kv_offset, const int64_t* kv_len, int batch, int n_h,
                         int n_kv, int d_h, cp_dtype in_dtype, int n_splits, float softmax_scale,
                         cp_dtype ws_dtype, void* ws_o, float* ws_lse, void* o_out,
                         cp_dtype out_dtype, float* lse_out, void* stream);
size_t cp_decode_workspace_bytes_ex(int batch, int n_h, int d_h, int n_splits, cp_dtype ws_dtype);

/* Bytes of the device array cp_decode_splitkv_noalloc keeps its split workspace in (72 MiB: the
 * fp32 workspace of 32 requests x 256 splits x 16 heads x D_H 128 takes 64.5 MiB). */
#define CP_DECODE_NOALLOC_MAX_BYTES (72u * 1024u * 1024u)

/* cp_decode_splitkv_noalloc -- cp_decode_splitkv_ex for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the split workspace lives in a file-scope device array of CP_DECODE_NOALLOC_MAX_BYTES inside
 * the library, not in an argument. Each device the library runs on holds its own copy until the
 * process ends; the call allocates and frees nothing. The caller still passes inputs and outputs.
 * Returns CP_E_CAPACITY (nothing launched) when cp_decode_workspace_bytes_ex(batch, n_h, d_h,
 * n_splits, ws_dtype) exceeds CP_DECODE_NOALLOC_MAX_BYTES; CP_E_HIP if the array's device address
 * cannot be looked up. Every call on a device shares that device's array, which keeps the last
 * call's partials (every split's partial is rewritten, so nothing needs clearing): calls that
 * overlap on one device (different streams, threads or processes) race and must not be issued.
 * Other arguments and errors as cp_decode_splitkv_ex. */
int cp_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int64_t* kv_offset, const int64_t* kv_len, int batch, int n_h,
                              int n_kv, int d_h, cp_dtype in_dtype, int n_splits,
                              float softmax_scale, cp_dtype ws_dtype, void* o_out,
                              cp_dtype out_dtype, float* lse_out, void* stream);

/* cp_ring_workspace_bytes -- size of one partial of the optional workspace of cp_ring_pass_kv's
 * running mode for a Q shard of tq tokens: O, then the LSEs at the next 256-byte boundary, of
 * tq * n_h rows of d_h fp32 values. A workspace of k such partials lets a step split into up to
 * k + 1 parts. Host-only. */
size_t cp_ring_workspace_bytes(int64_t tq, int n_h, int d_h);

/* ---------------------------------------------------------------------------------------------
 * cp_ring_pass_kv -- one rank's ring Pass-KV on one device ([CPMTI §3 "核心公式": each rank keeps
 * its Q shard while KV shards travel the ring for N-1 rounds; §3 Fig. 3). At step t the rank
 * holds KV shard (rank - t) mod cp_world and runs cp_partial_attn on it.
 *   k_shards, v_shards, tk, kv_segs, n_kv_segs: host arrays indexed by shard id [cp_world].
 *   Mode "partials" (o_parts != NULL): step t writes o_parts[t] / lse_parts[t] (device fp32
 *     [tq*n_h*d_h] / [tq*n_h]); the N partials are then merged with cp_merge_lse into o_out. The
 *     steps are independent in this mode, so they share launches (up to 8 per launch).
 *   Mode "running" (o_parts == NULL): steps accumulate into o_acc / lse_acc (device fp32), and
 *     o_out receives the result in out_dtype (o_out may equal o_acc when out_dtype is fp32).
 *   lse_out may be NULL.
 *   workspace, workspace_bytes: optional device scratch for the running mode (NULL or smaller
 *     than one partial: none; 16-byte aligned; ignored in the partials mode), caller-owned, in
 *     partials of cp_ring_workspace_bytes(tq, n_h, d_h) bytes. With bf16 inputs, a step whose Q
 *     shard has fewer 256-row tiles (over all KV heads) than the device has CUs is split over its
 *     keys into p parts: as many as fill the CUs, at most 8, at most one more than the workspace
 *     holds partials, and at least 2048 keys each (every KV run is cut at whole 64-key tiles near
 *     i/p of its length). The parts run in one launch, the first folding into (o_acc, lse_acc),
 *     the others into workspace partials, which are then merged in place. The split depends only
 *     on the shapes, the device's CU count and workspace_bytes. Calls sharing one workspace must
 *     be ordered on one stream.
 * ------------------------------------------------------------------------------------------- */
int cp_ring_pass_kv(const void* q, int64_t tq, const cp_segment* q_segs, int n_q_segs,
                    int cp_world, int rank, const void* const* k_shards,
                    const void* const* v_shards, const int64_t* tk,
                    const cp_segment* const* kv_segs, const int* n_kv_segs, int n_h, int n_kv,
                    int d_h, cp_dtype in_dtype, int causal, float softmax_scale,
                    float* const* o_parts, float* const* lse_parts, float* o_acc, float* lse_acc,
                    void* o_out, cp_dtype out_dtype, float* lse_out, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * cp_ring_pass_q -- ring Pass-Q over all cp_world ranks on one device ([CPMTI §3 "核心公式": KV
 * shards stay on their rank while Q shards travel the ring for N-1 rounds, then an All2All
 * returns every partial to its Q owner, where they are merged). At step t the rank owning KV
 * shard s hosts Q shard q = (s - t) mod cp_world; the partial lands in slot q*cp_world + s (on
 * one device the All2All is this placement). Each Q shard's cp_world partials are then merged in
 * ascending s into o_out[q] / lse_out[q].
 *   q_shards, tq, q_segs, n_q_segs: host arrays [cp_world] (Q shard per rank).
 *   k_shards ... n_kv_segs: host arrays [cp_world] (KV shard per rank).
 *   o_parts, lse_parts: host arrays [cp_world*cp_world] of device fp32 buffers, slot q*N + s
 *     sized for Q shard q.
 *   o_out, lse_out: host arrays [cp_world] of device outputs (lse_out may be NULL, or hold NULLs).
 * The cp_world^2 partials are independent (each has a slot of its own). They are computed in
 * ring-step order, as many per launch as fit the kernel's tables together (at most 8 problems
 * and 64 Q runs and 64 KV runs in total: two steps of a 4-rank ring per launch). Every partial
 * and every merge is validated as by cp_partial_attn / cp_merge_lse before anything is launched.
 * ------------------------------------------------------------------------------------------- */
int cp_ring_pass_q(int cp_world, const void* const* q_shards, const int64_t* tq,
                   const cp_segment* const* q_segs, const int* n_q_segs,
                   const void* const* k_shards, const void* const* v_shards, const int64_t* tk,
                   const cp_segment* const* kv_segs, const int* n_kv_segs, int n_h, int n_kv,
                   int d_h, cp_dtype in_dtype, int causal, float softmax_scale,
                   float* const* o_parts, float* const* lse_parts, void* const* o_out,
                   cp_dtype out_dtype, float* const* lse_out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Backward ([CPEP §6]: with context parallelism the backward returns each rank's K/V gradient
 * contributions to the ranks that own those K/V chunks, a reduce-scatter; on one device that is
 * a sum per KV shard). For a row (token, head) with FINAL output O and LSE (over every shard the
 * row sees) and output gradient dO, and a key j it sees: P = exp(scale * q.k_j - LSE),
 * dS = P (dO.v_j - delta) with delta = dO.O; then dQ += scale * dS k_j, dK_j += scale * dS q,
 * dV_j += P dO. Summed over ring steps (dQ) and over the ranks that visit a KV shard (dK, dV) the
 * contributions are the exact gradient of the whole attention.
 *
 * cp_attn_bwd_delta -- delta[r] = sum_d dO[r][d] * O[r][d] for rows = T_q * N_H.
 *   o: device fp32 [rows, d_h] (the final forward output); d_o: device [rows, d_h] in do_dtype;
 *   delta: device fp32 [rows].
 * ------------------------------------------------------------------------------------------- */
int cp_attn_bwd_delta(const float* o, const void* d_o, cp_dtype do_dtype, int64_t rows, int d_h,
                      float* delta, void* stream);

/* cp_attn_bwd_workspace_bytes -- size of the optional device workspace of cp_partial_attn_bwd and
 * cp_ring_pass_kv_bwd for head dimension d_h (0 if d_h is not 64 or 128): 2048 slots of 128 keys x
 * d_h x 2 fp32 values (256 MiB at d_h = 128). It depends on d_h only, so one allocation serves
 * every shape. Host-only.
 * ------------------------------------------------------------------------------------------- */
size_t cp_attn_bwd_workspace_bytes(int d_h);

/* cp_partial_attn_bwd -- one ring step's backward: the contributions of a Q shard against one KV
 * shard, ADDED into dq, dk and dv (callers zero them first).
 *   q, k, v, tq, tk, n_h, n_kv, d_h, segment tables, causal, softmax_scale: as cp_partial_attn.
 *     bf16 inputs run the products on bf16 MFMA with fp32 accumulation (probabilities and score
 *     gradients rounded to bf16 as operands; the score gradient that dK sums is formed from the
 *     probability rounded to fp16); fp32 inputs run in fp32 arithmetic throughout.
 *   lse: device fp32 [tq, n_h], the final natural-log LSE of each row (-inf: the row saw no key);
 *   delta: device fp32 [tq, n_h] from cp_attn_bwd_delta; d_o: device [tq, n_h, d_h] in in_dtype.
 *   dq: device fp32 [tq, n_h, d_h]; dk, dv: device fp32 [tk, n_kv, d_h]; all 16-byte aligned.
 *   workspace, workspace_bytes: optional device scratch (16-byte aligned; NULL or 0 bytes: none),
 *     caller-owned, at most cp_attn_bwd_workspace_bytes(d_h) of it used. With bf16 inputs and
 *     fewer than 1024 key tiles of 128 keys (over all KV heads) in a launch, the query rows that
 *     see each key tile are divided into up to 16 equal parts (as many as the workspace holds)
 *     worked on by separate workgroups; their dK/dV sums go to the workspace and are then added
 *     into dk and dv in part order. The part count depends only on the shapes and workspace_bytes.
 *     Calls sharing one workspace must be ordered on one stream.
 * Contributions of one call are summed in a fixed order (deterministic); calls that add into the
 * same buffers must be ordered on one stream.
 * ------------------------------------------------------------------------------------------- */
int cp_partial_attn_bwd(const void* q, const void* k, const void* v, int64_t tq, int64_t tk,
                        int n_h, int n_kv, int d_h, cp_dtype in_dtype, const cp_segment* q_segs,
                        int n_q_segs, const cp_segment* kv_segs, int n_kv_segs, int causal,
                        float softmax_scale, const float* lse, const float* delta, const void* d_o,
                        float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                        void* stream);

/* cp_ring_pass_kv_bwd -- one rank's ring Pass-KV backward on one device: delta of the rank's rows
 * into `delta` (device fp32 [tq, n_h], caller-owned), then at step t the contributions against KV
 * shard (rank - t) mod cp_world, added into dq and into that shard's dk_shards[s] / dv_shards[s]
 * (device fp32 [tk[s], n_kv, d_h]). o, lse: the rank's final forward output and LSE; d_o in in_dtype.
 * workspace, workspace_bytes: as cp_partial_attn_bwd (shared by the steps, which run in order).
 * Other arguments as cp_ring_pass_kv. Every step is validated before the first launch.
 * ------------------------------------------------------------------------------------------- */
int cp_ring_pass_kv_bwd(const void* q, int64_t tq, const cp_segment* q_segs, int n_q_segs,
                        int cp_world, int rank, const void* const* k_shards,
                        const void* const* v_shards, const int64_t* tk,
                        const cp_segment* const* kv_segs, const int* n_kv_segs, int n_h, int n_kv,
                        int d_h, cp_dtype in_dtype, int causal, float softmax_scale, const float* o,
                        const float* lse, const void* d_o, float* delta, float* dq,
                        float* const* dk_shards, float* const* dv_shards, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * cp_select_ring_variant -- runtime choice between ring Pass-KV and ring Pass-Q ([CPMTI §3
 * "核心公式", Algorithm 1]): Pass-KV when the KV-cache miss rate T / (T + P) exceeds
 * 2 * N_KV / N_H (condition 1), or when the SendRecv of one ring step can be hidden behind that
 * step's attention compute (condition 2); Pass-Q otherwise. Host-only, launches nothing.
 *   new_tokens T >= 1, cached_tokens P >= 0; elem_bytes: bytes per K/V element.
 *   link_bytes_per_s, attn_flops_per_s: the caller's estimates of the ring link bandwidth and of
 *     the attention throughput (> 0). Condition 2 compares, per ring step and rank, the time to
 *     pass one KV shard, 2 * (T + P) / N * N_KV * D_H * elem_bytes bytes, with the causal
 *     attention work of one step, 4 * D_H * N_H * (T / N) * ((T + P) / N - T / (2N)) flops (the new
 *     tokens against one shard of the context, half of the new-token block being masked).
 *   *variant_out: CP_PASS_KV or CP_PASS_Q. *reason_out (optional): 1 = miss rate above the
 *     threshold, 2 = transfer hidden by compute, 0 = neither (Pass-Q).
 * ------------------------------------------------------------------------------------------- */
typedef enum { CP_PASS_KV = 0, CP_PASS_Q = 1 } cp_ring_variant;
int cp_select_ring_variant(int64_t new_tokens, int64_t cached_tokens, int cp_world, int n_h,
                           int n_kv, int d_h, int elem_bytes, double link_bytes_per_s,
                           double attn_flops_per_s, int* variant_out, int* reason_out);

/* Human-readable name of a cp_status value. */
const char* cp_status_string(int status);
/* Message of the last failing call on this thread ("" if none). */
const char* cp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CPATTN_H */
