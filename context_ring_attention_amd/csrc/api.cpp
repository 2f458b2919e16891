// api.cpp -- the C ABI declared in include/cpattn.h: validation, the load-balanced shard map,
// launch planning, and the ring schedules played out on one device.
//
// Pages cited: [CPEP] "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두
// 축"; [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (paper review).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <string>
#include <vector>

#include "cp_internal.h"
#include "cpattn.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return CP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kI32Max = 0x7fffffff;

// Validates a segment table against a shard of `rows` rows and packs it for the kernels.
int pack_segments(const cp_segment* segs, int n, int64_t rows, const char* what, cpk::Seg* out) {
  if (n < 0 || n > cpk::kMaxSegs)
    return fail(CP_E_CAPACITY, "%s: %d segments (1..%d supported)", what, n, cpk::kMaxSegs);
  if (n > 0 && !segs) return fail(CP_E_ARG, "%s: segment table is NULL", what);
  for (int i = 0; i < n; ++i) {
    const cp_segment& s = segs[i];
    if (s.seq_id < 0 || s.pos_start < 0 || s.len < 0 || s.local_start < 0)
      return fail(CP_E_SHAPE, "%s[%d]: negative field", what, i);
    // (written so that no sum of two caller values can overflow)
    if (s.len > rows || s.local_start > rows - s.len)
      return fail(CP_E_SHAPE, "%s[%d]: rows [%lld, +%lld) outside the shard of %lld rows", what, i,
                  (long long)s.local_start, (long long)s.len, (long long)rows);
    if (s.len > kI32Max || s.pos_start > kI32Max - s.len)
      return fail(CP_E_UNSUPPORTED, "%s[%d]: positions beyond 2^31", what, i);
    out[i] = cpk::Seg{s.seq_id, (int32_t)s.pos_start, (int32_t)s.len, (int32_t)s.local_start};
  }
  return CP_OK;
}

// Orders the Q runs (of all problems) by the causal work of their heaviest (last) tile,
// heaviest first, and numbers the workgroup tiles accordingly (see AttnParams).
void plan_tiles(cpk::AttnParams& p, int rows_per_tile) {
  std::vector<std::pair<int64_t, int>> work;
  for (int i = 0; i < p.n_q_segs; ++i) {
    const cpk::Seg& q = p.qs[i];
    const int pr = p.q_prob[i];
    const int64_t last = (int64_t)q.pos + q.len - 1;
    int64_t w = 0;
    for (int j = p.kv_lo[pr]; j < p.kv_hi[pr]; ++j) {
      const cpk::Seg& k = p.ks[j];
      if (k.seq != q.seq) continue;
      int64_t n = p.causal ? std::min<int64_t>(k.len, std::max<int64_t>(0, last - k.pos + 1)) : k.len;
      w += n;
    }
    work.push_back({w, i});
  }
  std::stable_sort(work.begin(), work.end(),
                   [](const std::pair<int64_t, int>& a, const std::pair<int64_t, int>& b) { return a.first > b.first; });
  p.tile_prefix[0] = 0;
  for (int s = 0; s < p.n_q_segs; ++s) {
    const int i = work[s].second;
    p.order[s] = (int8_t)i;
    const int64_t rows = (int64_t)p.qs[i].len * p.group;
    p.tile_prefix[s + 1] = p.tile_prefix[s] + (int)((rows + rows_per_tile - 1) / rows_per_tile);
  }
  p.total_tiles = p.tile_prefix[p.n_q_segs];
}

int check_heads(int n_h, int n_kv, int d_h) {
  if (n_h < 1 || n_kv < 1) return fail(CP_E_ARG, "n_h=%d n_kv=%d must be >= 1", n_h, n_kv);
  if (n_h % n_kv != 0) return fail(CP_E_SHAPE, "n_h=%d is not a multiple of n_kv=%d", n_h, n_kv);
  if (d_h != 64 && d_h != 128) return fail(CP_E_UNSUPPORTED, "d_h=%d (64 or 128 supported)", d_h);
  if (n_kv > 65535) return fail(CP_E_UNSUPPORTED, "n_kv=%d too large", n_kv);
  return CP_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CP_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// One partial attention: a Q shard (with its segment table) against a KV shard.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  int64_t tq, tk;
  const cp_segment* q_segs;
  int n_q_segs;
  const cp_segment* kv_segs;
  int n_kv_segs;
  float* o;
  float* lse;
};

// Argument checks of a set of partial attentions (nothing is launched).
int validate_problems(const Problem* probs, int n_probs, int n_h, int n_kv, int d_h,
                      cp_dtype in_dtype, float softmax_scale, int accumulate) {
  int st = check_heads(n_h, n_kv, d_h);
  if (st) return st;
  if (in_dtype != CP_F32 && in_dtype != CP_BF16) return fail(CP_E_ARG, "in_dtype=%d", (int)in_dtype);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CP_E_ARG, "softmax_scale must be finite and > 0");
  if (accumulate != 0 && accumulate != 1) return fail(CP_E_ARG, "accumulate=%d", accumulate);
  const int64_t group = n_h / n_kv;
  for (int i = 0; i < n_probs; ++i) {
    const Problem& pr = probs[i];
    if (pr.tq < 0 || pr.tk < 0) return fail(CP_E_ARG, "negative token count");
    if (pr.tq > kI32Max || pr.tk > kI32Max) return fail(CP_E_UNSUPPORTED, "token counts beyond 2^31");
    cpk::Seg scratch[cpk::kMaxSegs];
    st = pack_segments(pr.q_segs, pr.n_q_segs, pr.tq, "q_segs", scratch);
    if (st) return st;
    st = pack_segments(pr.kv_segs, pr.n_kv_segs, pr.tk, "kv_segs", scratch);
    if (st) return st;
    // the kernels index a Q run's (token, head-in-group) rows in 32 bits
    for (int j = 0; j < pr.n_q_segs; ++j)
      if (pr.q_segs[j].len > 0 && pr.q_segs[j].len * group > kI32Max)
        return fail(CP_E_UNSUPPORTED, "q_segs[%d]: %lld tokens x %lld heads per KV head exceed 2^31 rows",
                    j, (long long)pr.q_segs[j].len, (long long)group);
    if (pr.n_q_segs > 0 && (!pr.q || !pr.o || !pr.lse)) return fail(CP_E_ARG, "q, o or lse is NULL");
    if (pr.n_kv_segs > 0 && (!pr.k || !pr.v)) return fail(CP_E_ARG, "k or v is NULL");
    if (!aligned16(pr.q) || !aligned16(pr.k) || !aligned16(pr.v) || !aligned16(pr.o))
      return fail(CP_E_ARG, "q, k, v and o must be 16-byte aligned");
  }
  return CP_OK;
}

// Argument checks of cp_merge_lse (nothing is launched).
int validate_merge(int n_parts, const float* const* o_parts, const float* const* lse_parts,
                   int64_t rows, int d_h, const void* o_out, cp_dtype out_dtype) {
  if (n_parts < 1 || n_parts > cpk::kMaxParts)
    return fail(CP_E_CAPACITY, "n_parts=%d (1..%d supported)", n_parts, cpk::kMaxParts);
  if (!o_parts || !lse_parts) return fail(CP_E_ARG, "part arrays are NULL");
  if (rows < 0) return fail(CP_E_ARG, "rows=%lld", (long long)rows);
  if (d_h != 64 && d_h != 128) return fail(CP_E_UNSUPPORTED, "d_h=%d (64 or 128 supported)", d_h);
  if (out_dtype != CP_F32 && out_dtype != CP_BF16) return fail(CP_E_ARG, "out_dtype=%d", (int)out_dtype);
  if (rows > ((int64_t)1 << 40)) return fail(CP_E_UNSUPPORTED, "rows=%lld", (long long)rows);
  for (int i = 0; i < n_parts; ++i) {
    if (!o_parts[i] || !lse_parts[i]) return fail(CP_E_ARG, "part %d is NULL", i);
    if (!aligned16(o_parts[i])) return fail(CP_E_ARG, "o_parts[%d] must be 16-byte aligned", i);
  }
  if (!o_out || !aligned16(o_out)) return fail(CP_E_ARG, "o_out is NULL or not 16-byte aligned");
  if (out_dtype == CP_BF16)
    for (int i = 0; i < n_parts; ++i)
      if ((const void*)o_parts[i] == o_out) return fail(CP_E_ARG, "bf16 output cannot alias a part");
  return CP_OK;
}

// Validates, then launches independent partial attentions, as few launches as the pooled segment
// tables allow (problems are packed in order; a problem always fits a launch on its own).
int partial_attn_problems(const Problem* probs, int n_probs, int n_h, int n_kv, int d_h,
                          cp_dtype in_dtype, int causal, float softmax_scale, int accumulate,
                          void* stream, const char* what) {
  int st = validate_problems(probs, n_probs, n_h, n_kv, d_h, in_dtype, softmax_scale, accumulate);
  if (st) return st;
  const bool bf16 = in_dtype == CP_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int next = 0;
  while (next < n_probs) {
    cpk::AttnParams p{};
    p.n_h = n_h;
    p.n_kv = n_kv;
    p.group = n_h / n_kv;
    p.causal = causal ? 1 : 0;
    p.accumulate = accumulate;
    p.scale = softmax_scale;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    int nq = 0, nk = 0, np = 0;
    while (next < n_probs && np < cpk::kMaxProblems &&
           nq + probs[next].n_q_segs <= cpk::kMaxSegs && nk + probs[next].n_kv_segs <= cpk::kMaxSegs) {
      const Problem& pr = probs[next++];
      pack_segments(pr.q_segs, pr.n_q_segs, pr.tq, "q_segs", p.qs + nq);
      pack_segments(pr.kv_segs, pr.n_kv_segs, pr.tk, "kv_segs", p.ks + nk);
      for (int i = 0; i < pr.n_q_segs; ++i) p.q_prob[nq + i] = (int8_t)np;
      p.kv_lo[np] = (int8_t)nk;
      p.kv_hi[np] = (int8_t)(nk + pr.n_kv_segs);
      p.q[np] = pr.q;
      p.k[np] = pr.k;
      p.v[np] = pr.v;
      p.o[np] = pr.o;
      p.lse[np] = pr.lse;
      nq += pr.n_q_segs;
      nk += pr.n_kv_segs;
      ++np;
    }
    p.n_q_segs = nq;
    plan_tiles(p, bf16 ? cpk::kTileRowsBf16 : cpk::kTileRowsF32);
    if (p.total_tiles == 0) continue;
    const hipError_t e = bf16 ? cpk::launch_attn_bf16(p, d_h, s) : cpk::launch_attn_f32(p, d_h, s);
    st = launch_status(e, what);
    if (st) return st;
  }
  return ok();
}

}  // namespace

extern "C" {

const char* cp_status_string(int status) {
  switch (status) {
    case CP_OK: return "CP_OK";
    case CP_E_ARG: return "CP_E_ARG";
    case CP_E_SHAPE: return "CP_E_SHAPE";
    case CP_E_UNSUPPORTED: return "CP_E_UNSUPPORTED";
    case CP_E_CAPACITY: return "CP_E_CAPACITY";
    case CP_E_HIP: return "CP_E_HIP";
    default: return "CP_E_UNKNOWN";
  }
}

const char* cp_last_error(void) { return g_last_error.c_str(); }

// Load-balanced sharding ([CPMTI §4 "负载均衡分片策略", Fig. 2]): 2N chunks per range with floor
// edges; rank r takes chunk r then chunk 2N-1-r, so with a causal mask each rank pairs an early
// (cheap) chunk with a late (expensive) one and every rank gets the same work and KV size.
int cp_shard_map(int n_ranges, const int32_t* seq_id, const int64_t* range_begin,
                 const int64_t* range_end, int cp_world, int rank, cp_segment* segs_out,
                 int max_segs, int* n_segs_out, int64_t* tokens_out, int64_t max_tokens,
                 int64_t* n_tokens_out) {
  if (n_ranges < 0) return fail(CP_E_ARG, "n_ranges=%d", n_ranges);
  if (n_ranges > 0 && (!range_begin || !range_end)) return fail(CP_E_ARG, "range arrays are NULL");
  if (cp_world < 1) return fail(CP_E_ARG, "cp_world=%d", cp_world);
  if (rank < 0 || rank >= cp_world) return fail(CP_E_ARG, "rank=%d outside [0, %d)", rank, cp_world);
  if (!n_segs_out) return fail(CP_E_ARG, "n_segs_out is NULL");
  if (max_segs < 0 || max_tokens < 0) return fail(CP_E_ARG, "negative capacity");

  std::map<int32_t, int64_t> seq_len;
  for (int i = 0; i < n_ranges; ++i) {
    const int32_t s = seq_id ? seq_id[i] : i;
    if (s < 0) return fail(CP_E_ARG, "seq_id[%d]=%d", i, s);
    if (range_begin[i] < 0 || range_end[i] < range_begin[i])
      return fail(CP_E_ARG, "range %d: [%lld, %lld)", i, (long long)range_begin[i], (long long)range_end[i]);
    int64_t& L = seq_len[s];
    L = std::max(L, range_end[i]);
  }
  std::map<int32_t, int64_t> seq_base;
  int64_t acc = 0;
  for (const auto& kv : seq_len) {  // ascending sequence id
    seq_base[kv.first] = acc;
    acc += kv.second;
  }
  // sequences without a range have length 0 and do not shift later bases

  const int64_t n_chunks = 2 * (int64_t)cp_world;
  // chunk edges are computed as c * L / (2N) in 64 bits
  for (int i = 0; i < n_ranges; ++i)
    if (range_end[i] - range_begin[i] > INT64_MAX / n_chunks)
      return fail(CP_E_UNSUPPORTED, "range %d: length %lld too large for %lld chunks", i,
                  (long long)(range_end[i] - range_begin[i]), (long long)n_chunks);
  int n_segs = 0;
  int64_t n_tok = 0;
  for (int i = 0; i < n_ranges; ++i) {
    const int32_t s = seq_id ? seq_id[i] : i;
    const int64_t a = range_begin[i];
    const int64_t L = range_end[i] - range_begin[i];
    const int64_t owned[2] = {rank, n_chunks - 1 - rank};
    for (int w = 0; w < 2; ++w) {
      const int64_t lo = a + owned[w] * L / n_chunks;
      const int64_t hi = a + (owned[w] + 1) * L / n_chunks;
      if (hi <= lo) continue;
      if (segs_out && n_segs < max_segs) {
        cp_segment& g = segs_out[n_segs];
        g.seq_id = s;
        g.reserved = 0;
        g.pos_start = lo;
        g.len = hi - lo;
        g.local_start = n_tok;
      }
      if (tokens_out)
        for (int64_t p = lo; p < hi; ++p)
          if (n_tok + (p - lo) < max_tokens) tokens_out[n_tok + (p - lo)] = seq_base[s] + p;
      ++n_segs;
      n_tok += hi - lo;
    }
  }
  *n_segs_out = n_segs;
  if (n_tokens_out) *n_tokens_out = n_tok;
  if (n_segs > max_segs || (segs_out == nullptr && n_segs > 0))
    return fail(CP_E_CAPACITY, "need %d segments, capacity %d", n_segs, segs_out ? max_segs : 0);
  if (tokens_out && n_tok > max_tokens)
    return fail(CP_E_CAPACITY, "need %lld tokens, capacity %lld", (long long)n_tok, (long long)max_tokens);
  return ok();
}

int cp_partial_attn(const void* q, const void* k, const void* v, int64_t tq, int64_t tk, int n_h,
                    int n_kv, int d_h, cp_dtype in_dtype, const cp_segment* q_segs, int n_q_segs,
                    const cp_segment* kv_segs, int n_kv_segs, int causal, float softmax_scale,
                    float* o, float* lse, int accumulate, void* stream) {
  const Problem pr{q, k, v, tq, tk, q_segs, n_q_segs, kv_segs, n_kv_segs, o, lse};
  return partial_attn_problems(&pr, 1, n_h, n_kv, d_h, in_dtype, causal, softmax_scale, accumulate,
                               stream, "cp_partial_attn");
}

int cp_merge_lse(int n_parts, const float* const* o_parts, const float* const* lse_parts,
                 int64_t rows, int d_h, void* o_out, cp_dtype out_dtype, float* lse_out,
                 void* stream) {
  const int st = validate_merge(n_parts, o_parts, lse_parts, rows, d_h, o_out, out_dtype);
  if (st) return st;
  cpk::MergeParams p{};
  for (int i = 0; i < n_parts; ++i) {
    p.o_parts[i] = o_parts[i];
    p.lse_parts[i] = lse_parts[i];
  }
  p.o_out = o_out;
  p.lse_out = lse_out;
  p.rows = rows;
  p.n_parts = n_parts;
  p.d_h = d_h;
  p.out_bf16 = out_dtype == CP_BF16;
  if (rows == 0) return ok();
  return launch_status(cpk::launch_merge(p, static_cast<hipStream_t>(stream)), "cp_merge_lse");
}

size_t cp_decode_workspace_bytes(int batch, int n_h, int d_h, int n_splits) {
  if (batch < 0 || n_h < 0 || d_h < 0 || n_splits < 0) return 0;
  const size_t parts = (size_t)batch * n_splits * n_h;
  return parts * d_h * 2 + parts * sizeof(float);  // bf16 partial O, then fp32 LSE
}

int cp_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                      const int64_t* kv_offset, const int64_t* kv_len, int batch, int n_h,
                      int n_kv, int d_h, cp_dtype in_dtype, int n_splits, float softmax_scale,
                      void* ws_o, float* ws_lse, void* o_out, cp_dtype out_dtype, float* lse_out,
                      void* stream) {
  int st = check_heads(n_h, n_kv, d_h);
  if (st) return st;
  if (in_dtype != CP_BF16) return fail(CP_E_UNSUPPORTED, "decode supports bf16 inputs only");
  if (out_dtype != CP_F32 && out_dtype != CP_BF16) return fail(CP_E_ARG, "out_dtype=%d", (int)out_dtype);
  if (batch < 0 || batch > 65535) return fail(CP_E_UNSUPPORTED, "batch=%d (0..65535)", batch);
  if (n_splits < 1 || n_splits > 1024) return fail(CP_E_UNSUPPORTED, "n_splits=%d (1..1024)", n_splits);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CP_E_ARG, "softmax_scale must be finite and > 0");
  const int group = n_h / n_kv;
  if ((int64_t)n_kv * ((group + 15) / 16) > 65535) return fail(CP_E_UNSUPPORTED, "too many head blocks");
  if (batch == 0) return ok();
  if (!q || !k_cache || !v_cache || !kv_offset || !kv_len || !ws_o || !ws_lse || !o_out)
    return fail(CP_E_ARG, "NULL pointer argument");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(ws_o) || !aligned16(o_out))
    return fail(CP_E_ARG, "q, caches, ws_o and o_out must be 16-byte aligned");
  cpk::DecodeParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.kv_offset = kv_offset;
  p.kv_len = kv_len;
  p.ws_o = ws_o;
  p.ws_lse = ws_lse;
  p.o_out = o_out;
  p.lse_out = lse_out;
  p.batch = batch;
  p.n_h = n_h;
  p.n_kv = n_kv;
  p.group = group;
  p.n_splits = n_splits;
  p.out_bf16 = out_dtype == CP_BF16;
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  return launch_status(cpk::launch_decode(p, d_h, static_cast<hipStream_t>(stream)), "cp_decode_splitkv");
}

// Ring Pass-KV ([CPMTI §3 "核心公式"; Fig. 3]): the rank keeps its Q shard; at step t it holds the
// KV shard that started on rank (rank - t) mod N.
int cp_ring_pass_kv(const void* q, int64_t tq, const cp_segment* q_segs, int n_q_segs,
                    int cp_world, int rank, const void* const* k_shards,
                    const void* const* v_shards, const int64_t* tk,
                    const cp_segment* const* kv_segs, const int* n_kv_segs, int n_h, int n_kv,
                    int d_h, cp_dtype in_dtype, int causal, float softmax_scale,
                    float* const* o_parts, float* const* lse_parts, float* o_acc, float* lse_acc,
                    void* o_out, cp_dtype out_dtype, float* lse_out, void* stream) {
  if (cp_world < 1 || cp_world > cpk::kMaxParts) return fail(CP_E_ARG, "cp_world=%d", cp_world);
  if (rank < 0 || rank >= cp_world) return fail(CP_E_ARG, "rank=%d", rank);
  if (!k_shards || !v_shards || !tk || !kv_segs || !n_kv_segs) return fail(CP_E_ARG, "shard arrays are NULL");
  const bool partials = o_parts != nullptr;
  if (partials && !lse_parts) return fail(CP_E_ARG, "lse_parts is NULL");
  if (!partials && (!o_acc || !lse_acc)) return fail(CP_E_ARG, "running mode needs o_acc and lse_acc");
  if (!o_out) return fail(CP_E_ARG, "o_out is NULL");
  // Step t holds KV shard (rank - t) mod N. Every step and the final merge are validated before
  // the first launch, so a failing call launches nothing.
  std::vector<Problem> steps(cp_world);
  for (int t = 0; t < cp_world; ++t) {
    const int s = ((rank - t) % cp_world + cp_world) % cp_world;
    steps[t] = Problem{q, k_shards[s], v_shards[s], tq, tk[s], q_segs, n_q_segs, kv_segs[s],
                       n_kv_segs[s], partials ? o_parts[t] : o_acc, partials ? lse_parts[t] : lse_acc};
  }
  int st = validate_problems(steps.data(), cp_world, n_h, n_kv, d_h, in_dtype, softmax_scale, 0);
  if (st) return st;
  const int64_t rows = tq * (int64_t)n_h;
  const bool fold_only = !partials && o_out == o_acc && out_dtype == CP_F32 &&
                         (lse_out == nullptr || lse_out == lse_acc);
  const float* op[1] = {o_acc};
  const float* lp[1] = {lse_acc};
  if (partials)
    st = validate_merge(cp_world, o_parts, lse_parts, rows, d_h, o_out, out_dtype);
  else if (!fold_only)
    st = validate_merge(1, op, lp, rows, d_h, o_out, out_dtype);
  if (st) return st;
  for (int t = 0; t < cp_world; ++t) {
    const int acc = (!partials && t > 0) ? 1 : 0;
    st = partial_attn_problems(&steps[t], 1, n_h, n_kv, d_h, in_dtype, causal, softmax_scale, acc,
                               stream, "cp_ring_pass_kv");
    if (st) return st;
  }
  if (partials)
    return cp_merge_lse(cp_world, o_parts, lse_parts, rows, d_h, o_out, out_dtype, lse_out, stream);
  if (fold_only) return ok();
  return cp_merge_lse(1, op, lp, rows, d_h, o_out, out_dtype, lse_out, stream);
}

// Ring Pass-Q ([CPMTI §3 "核心公式"]): KV shards stay put, Q shards travel; afterwards an All2All
// returns each partial to its Q owner, which merges them ([CPMTI §5 "关键实现细节" item 3]).
int cp_ring_pass_q(int cp_world, const void* const* q_shards, const int64_t* tq,
                   const cp_segment* const* q_segs, const int* n_q_segs,
                   const void* const* k_shards, const void* const* v_shards, const int64_t* tk,
                   const cp_segment* const* kv_segs, const int* n_kv_segs, int n_h, int n_kv,
                   int d_h, cp_dtype in_dtype, int causal, float softmax_scale,
                   float* const* o_parts, float* const* lse_parts, void* const* o_out,
                   cp_dtype out_dtype, float* const* lse_out, void* stream) {
  if (cp_world < 1 || cp_world > cpk::kMaxParts) return fail(CP_E_ARG, "cp_world=%d", cp_world);
  if (!q_shards || !tq || !q_segs || !n_q_segs || !k_shards || !v_shards || !tk || !kv_segs ||
      !n_kv_segs || !o_parts || !lse_parts || !o_out)
    return fail(CP_E_ARG, "NULL array argument");
  const int N = cp_world;
  // Step t: the rank holding KV shard s computes Q shard (s - t) mod N against it. The N partials
  // of a step are independent and go to the GPU as one launch. All N*N partials and the N merges
  // are validated before the first launch.
  std::vector<Problem> all((size_t)N * N);
  for (int t = 0; t < N; ++t)
    for (int s = 0; s < N; ++s) {
      const int qi = ((s - t) % N + N) % N;
      const int slot = qi * N + s;
      all[(size_t)t * N + s] = Problem{q_shards[qi], k_shards[s], v_shards[s], tq[qi], tk[s],
                                       q_segs[qi], n_q_segs[qi], kv_segs[s], n_kv_segs[s],
                                       o_parts[slot], lse_parts[slot]};
    }
  int vst = validate_problems(all.data(), N * N, n_h, n_kv, d_h, in_dtype, softmax_scale, 0);
  if (vst) return vst;
  for (int qi = 0; qi < N; ++qi) {
    vst = validate_merge(N, o_parts + (size_t)qi * N, lse_parts + (size_t)qi * N, tq[qi] * (int64_t)n_h,
                         d_h, o_out[qi], out_dtype);
    if (vst) return vst;
  }
  for (int t = 0; t < N; ++t) {
    const int st = partial_attn_problems(all.data() + (size_t)t * N, N, n_h, n_kv, d_h, in_dtype,
                                         causal, softmax_scale, 0, stream, "cp_ring_pass_q");
    if (st) return st;
  }
  for (int qi = 0; qi < N; ++qi) {
    const int st = cp_merge_lse(N, o_parts + (size_t)qi * N, lse_parts + (size_t)qi * N,
                                tq[qi] * (int64_t)n_h, d_h, o_out[qi], out_dtype,
                                lse_out ? lse_out[qi] : nullptr, stream);
    if (st) return st;
  }
  return ok();
}

// Algorithm 1 of [CPMTI §3 "核心公式"]: Pass-KV if the KV-cache miss rate exceeds 2 N_KV / N_H or
// if a ring step's KV transfer hides behind its attention compute; Pass-Q otherwise.
int cp_select_ring_variant(int64_t new_tokens, int64_t cached_tokens, int cp_world, int n_h,
                           int n_kv, int d_h, int elem_bytes, double link_bytes_per_s,
                           double attn_flops_per_s, int* variant_out, int* reason_out) {
  if (!variant_out) return fail(CP_E_ARG, "variant_out is NULL");
  if (new_tokens < 1 || cached_tokens < 0) return fail(CP_E_ARG, "need T >= 1 and P >= 0");
  if (cp_world < 1 || n_h < 1 || n_kv < 1 || d_h < 1 || elem_bytes < 1)
    return fail(CP_E_ARG, "sizes must be positive");
  if (n_h % n_kv != 0) return fail(CP_E_SHAPE, "n_h=%d is not a multiple of n_kv=%d", n_h, n_kv);
  if (!(link_bytes_per_s > 0) || !(attn_flops_per_s > 0))
    return fail(CP_E_ARG, "bandwidth and throughput estimates must be > 0");
  const double T = (double)new_tokens, P = (double)cached_tokens, N = (double)cp_world;
  const double miss = T / (T + P);
  const double threshold = 2.0 * n_kv / n_h;
  int reason = 0;
  if (miss > threshold) {
    reason = 1;
  } else {
    const double kv_bytes = 2.0 * (T + P) / N * n_kv * d_h * elem_bytes;
    const double flops = 4.0 * d_h * n_h * (T / N) * ((T + P) / N - T / (2.0 * N));
    if (kv_bytes / link_bytes_per_s <= flops / attn_flops_per_s) reason = 2;
  }
  *variant_out = reason ? CP_PASS_KV : CP_PASS_Q;
  if (reason_out) *reason_out = reason;
  return ok();
}

}  // extern "C"
