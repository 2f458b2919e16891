// cp_internal.h -- types shared by the host API (api.cpp) and the gfx950 kernels.
//
// Pages cited: [CPEP] "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두
// 축"; [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (paper review).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cpattn.h"

namespace cpk {

// Compact copy of cp_segment for kernel arguments (validated to fit int32 on the host).
struct Seg {
  int32_t seq;
  int32_t pos;  // position of the first token of the run within its sequence
  int32_t len;  // tokens in the run
  int32_t loc;  // first shard row of the run
};

constexpr int kMaxSegs = CP_MAX_SEGMENTS;
constexpr int kMaxParts = CP_MAX_MERGE_PARTS;

// Arguments of one partial-attention launch, covering up to kMaxProblems independent problems
// (a Q shard against a KV shard each, e.g. the ranks of one ring step) whose segment tables are
// pooled. Rows of a Q shard are handled per KV head group as a flat row space per Q segment: row r
// of segment i is token loc + r / group, query head g*group + r % group (consecutive heads share
// KV head g, [CPEP §8.2]). Each workgroup takes one tile of rows; tiles are numbered in processing
// order: slots 0..n_q_segs-1 visit the Q segments in `order`, and inside a segment tiles go from
// the last (largest positions, most causal work) to the first, so the heaviest tiles start first.
constexpr int kMaxProblems = 8;
struct AttnParams {
  const void* q[kMaxProblems];
  const void* k[kMaxProblems];
  const void* v[kMaxProblems];
  float* o[kMaxProblems];
  float* lse[kMaxProblems];
  int32_t n_h;
  int32_t n_kv;
  int32_t group;       // n_h / n_kv
  int32_t causal;
  int32_t accumulate;
  int32_t n_q_segs;    // Q segments of all problems
  int32_t total_tiles;
  float scale;         // softmax scale
  float scale_log2;    // softmax scale * log2(e)
  int32_t tile_prefix[kMaxSegs + 1];  // tiles before processing slot i
  int8_t order[kMaxSegs];             // Q segment of processing slot i
  int8_t q_prob[kMaxSegs];            // problem of Q segment i
  int8_t kv_lo[kMaxProblems];         // KV segments of problem i: [kv_lo[i], kv_hi[i])
  int8_t kv_hi[kMaxProblems];
  Seg qs[kMaxSegs];
  Seg ks[kMaxSegs];
};
static_assert(sizeof(AttnParams) <= 4096, "kernel arguments are limited to 4 KB");

struct MergeParams {
  const float* o_parts[kMaxParts];
  const float* lse_parts[kMaxParts];
  void* o_out;
  float* lse_out;
  int64_t rows;
  int32_t n_parts;
  int32_t d_h;
  int32_t out_bf16;
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const int64_t* kv_offset;
  const int64_t* kv_len;
  void* ws_o;  // [batch, n_splits, n_h, d_h], fp32 (or bf16 if ws_bf16)
  float* ws_lse;
  void* o_out;
  float* lse_out;
  int32_t batch;
  int32_t n_h;
  int32_t n_kv;
  int32_t group;
  int32_t n_splits;
  int32_t out_bf16;
  int32_t ws_bf16;
  float scale;
  float scale_log2;
  // > 0: the persistent split kernel, each wave walking up to this many units (host-chosen)
  int32_t units_per_wave;
};

// Units a persistent decode wave can hold finished partials of (registers).
constexpr int kDecodeMaxUnits = 8;

// Arguments of one backward launch pair (dQ kernel, then dK/dV kernel) for one Q shard against
// one KV shard. Q tiles (256 rows) are numbered over the Q runs in `q_order`, the last tile of a run
// first; KV tiles (128 keys) over the KV runs in `kv_order`, the first tile of a run first (the
// causally heaviest tiles start first either way).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  const float* lse;    // final log-sum-exp of each (token, head), natural log
  const float* delta;  // dO . O of each (token, head)
  float* dq;           // [tq, n_h, d_h] fp32, accumulated
  float* dk;           // [tk, n_kv, d_h] fp32, accumulated
  float* dv;
  int32_t n_h;
  int32_t n_kv;
  int32_t group;
  int32_t causal;
  float scale;
  float scale_log2;
  int32_t n_q_segs;
  int32_t n_kv_segs;
  int32_t q_tiles;
  int32_t kv_tiles;
  int32_t q_prefix[kMaxSegs + 1];
  int32_t kv_prefix[kMaxSegs + 1];
  int8_t q_order[kMaxSegs];
  int8_t kv_order[kMaxSegs];
  Seg qs[kMaxSegs];
  Seg ks[kMaxSegs];
};
static_assert(sizeof(BwdParams) <= 4096, "kernel arguments are limited to 4 KB");
constexpr int kBwdQRows = 256;  // query rows per dQ workgroup
constexpr int kBwdKeys = 128;   // keys per dK/dV workgroup

// Launchers (defined next to their kernels). Each returns the HIP launch status.
hipError_t launch_attn_f32(const AttnParams& p, int d_h, hipStream_t stream);
hipError_t launch_attn_bf16(const AttnParams& p, int d_h, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
// O = 0, LSE = -inf for `rows` rows of d_h fp32 values (o 16-byte aligned).
hipError_t launch_fill_running(float* o, float* lse, int64_t rows, int d_h, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int d_h, hipStream_t stream);
// Device address of the allocation-free decode workspace (CP_DECODE_NOALLOC_MAX_BYTES) on the
// current device; looked up once per device, then cached.
hipError_t decode_scratch(void** out);
hipError_t launch_bwd(const BwdParams& p, int d_h, hipStream_t stream);
hipError_t launch_bwd_delta(const float* o, const void* d_o, bool do_bf16, int64_t rows, int d_h,
                            float* delta, hipStream_t stream);

// Rows per workgroup tile of each attention kernel (the host plans tiles with these).
constexpr int kTileRowsF32 = 64;
#ifndef CP_BF16_TILE_ROWS
#define CP_BF16_TILE_ROWS 256
#endif
constexpr int kTileRowsBf16 = CP_BF16_TILE_ROWS;

}  // namespace cpk
