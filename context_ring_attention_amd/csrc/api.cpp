// api.cpp -- the C ABI declared in include/cpattn.h: validation, the load-balanced shard map,
// launch planning, and the ring schedules played out on one device.
//
// Pages cited: [CPEP] "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두
// 축"; [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (paper review).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "attn_bwd.h"
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
size_t round_up256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int64_t kI32Max = 0x7fffffff;

// Segment tables longer than this are rejected (a sanity bound; tables of any length up to it are
// split over as many launches as needed).
constexpr int kMaxTableSegs = 1 << 20;

// Validates a segment table against a shard of `rows` rows (nothing is packed or launched).
int check_segments(const cp_segment* segs, int n, int64_t rows, const char* what) {
  if (n < 0 || n > kMaxTableSegs)
    return fail(CP_E_CAPACITY, "%s: %d segments (0..%d supported)", what, n, kMaxTableSegs);
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
  }
  return CP_OK;
}

// The kernels' compact copy of a validated segment.
cpk::Seg to_seg(const cp_segment& s) {
  return cpk::Seg{s.seq_id, (int32_t)s.pos_start, (int32_t)s.len, (int32_t)s.local_start};
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
    st = check_segments(pr.q_segs, pr.n_q_segs, pr.tq, "q_segs");
    if (st) return st;
    st = check_segments(pr.kv_segs, pr.n_kv_segs, pr.tk, "kv_segs");
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

// One launchable piece of a partial attention: a subset of a problem's Q runs (at most
// kMaxSegs) against a subset of its KV runs (at most kMaxSegs), in one accumulation phase.
// Phase 0 takes the caller's accumulate flag; later phases fold into what phase 0 wrote.
struct Piece {
  const Problem* pr;
  std::vector<cp_segment> q, kv;
  int phase;
};

// Splits a problem whose tables exceed one launch. Q runs are grouped by sequence (in order of
// first appearance) and packed into groups of at most kMaxSegs runs; a group takes only the KV
// runs of its own sequences (runs of other sequences are never visible to it). A group whose KV
// runs exceed kMaxSegs is repeated with the next kMaxSegs KV runs in phase 1, 2, ...: each Q row
// then merges the partials of its KV runs in order, as a ring step does. Rows stay disjoint
// between the pieces of one phase.
void split_problem(const Problem& pr, std::vector<Piece>& out) {
  const int cap = cpk::kMaxSegs;
  if (pr.n_q_segs <= cap && pr.n_kv_segs <= cap) {
    out.push_back(Piece{&pr, std::vector<cp_segment>(pr.q_segs, pr.q_segs + pr.n_q_segs),
                        std::vector<cp_segment>(pr.kv_segs, pr.kv_segs + pr.n_kv_segs), 0});
    return;
  }
  std::map<int32_t, std::vector<cp_segment>> kv_by_seq;
  for (int j = 0; j < pr.n_kv_segs; ++j)
    if (pr.kv_segs[j].len > 0) kv_by_seq[pr.kv_segs[j].seq_id].push_back(pr.kv_segs[j]);
  std::vector<int32_t> seq_order;
  std::map<int32_t, std::vector<cp_segment>> q_by_seq;
  for (int i = 0; i < pr.n_q_segs; ++i) {
    const cp_segment& q = pr.q_segs[i];
    if (q.len == 0) continue;
    auto it = q_by_seq.find(q.seq_id);
    if (it == q_by_seq.end()) {
      seq_order.push_back(q.seq_id);
      it = q_by_seq.emplace(q.seq_id, std::vector<cp_segment>()).first;
    }
    it->second.push_back(q);
  }
  // Groups of whole sequences while they fit; a sequence with more Q runs than one launch takes
  // is cut into chunks of kMaxSegs runs, each with all of that sequence's KV runs.
  struct Group {
    std::vector<cp_segment> q, kv;
  };
  std::vector<Group> groups;
  Group cur;
  auto flush = [&]() {
    if (!cur.q.empty()) groups.push_back(std::move(cur));
    cur = Group();
  };
  for (int32_t sid : seq_order) {
    const std::vector<cp_segment>& qs = q_by_seq[sid];
    const std::vector<cp_segment>& ks = kv_by_seq[sid];
    const int kv_first = (int)std::min<size_t>(ks.size(), cap);  // what phase 0 would add
    if (qs.size() <= (size_t)cap && ks.size() <= (size_t)cap) {
      if (cur.q.size() + qs.size() > (size_t)cap || cur.kv.size() + kv_first > (size_t)cap) flush();
      cur.q.insert(cur.q.end(), qs.begin(), qs.end());
      cur.kv.insert(cur.kv.end(), ks.begin(), ks.end());
      continue;
    }
    flush();
    for (size_t a = 0; a < qs.size(); a += cap) {
      Group g;
      g.q.assign(qs.begin() + a, qs.begin() + std::min(qs.size(), a + cap));
      g.kv = ks;
      groups.push_back(std::move(g));
    }
  }
  flush();
  for (const Group& g : groups) {
    if (g.kv.empty()) {  // no visible key: phase 0 still writes the empty result (or keeps it)
      out.push_back(Piece{&pr, g.q, {}, 0});
      continue;
    }
    for (size_t b = 0, ph = 0; b < g.kv.size(); b += cap, ++ph)
      out.push_back(Piece{&pr, g.q,
                          std::vector<cp_segment>(g.kv.begin() + b, g.kv.begin() + std::min(g.kv.size(), b + cap)),
                          (int)ph});
  }
}

// Validates, then launches independent partial attentions, as few launches as the pooled segment
// tables allow (pieces are packed in order; a piece always fits a launch on its own). Problems
// whose tables exceed one launch are split (split_problem); their later phases run after every
// phase-0 launch, in order, on the same stream.
int partial_attn_problems(const Problem* probs, int n_probs, int n_h, int n_kv, int d_h,
                          cp_dtype in_dtype, int causal, float softmax_scale, int accumulate,
                          void* stream, const char* what) {
  int st = validate_problems(probs, n_probs, n_h, n_kv, d_h, in_dtype, softmax_scale, accumulate);
  if (st) return st;
  const bool bf16 = in_dtype == CP_BF16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<Piece> pieces;
  for (int i = 0; i < n_probs; ++i) split_problem(probs[i], pieces);
  int n_phases = 0;
  for (const Piece& pc : pieces) n_phases = std::max(n_phases, pc.phase + 1);
  for (int phase = 0; phase < n_phases; ++phase) {
    std::vector<const Piece*> todo;
    for (const Piece& pc : pieces)
      if (pc.phase == phase) todo.push_back(&pc);
    size_t next = 0;
    while (next < todo.size()) {
      cpk::AttnParams p{};
      p.n_h = n_h;
      p.n_kv = n_kv;
      p.group = n_h / n_kv;
      p.causal = causal ? 1 : 0;
      p.accumulate = phase == 0 ? accumulate : 1;
      p.scale = softmax_scale;
      p.scale_log2 = softmax_scale * 1.4426950408889634f;
      int nq = 0, nk = 0, np = 0;
      while (next < todo.size() && np < cpk::kMaxProblems &&
             nq + (int)todo[next]->q.size() <= cpk::kMaxSegs &&
             nk + (int)todo[next]->kv.size() <= cpk::kMaxSegs) {
        const Piece& pc = *todo[next++];
        for (size_t i = 0; i < pc.q.size(); ++i) {
          p.qs[nq + i] = to_seg(pc.q[i]);
          p.q_prob[nq + i] = (int8_t)np;
        }
        for (size_t j = 0; j < pc.kv.size(); ++j) p.ks[nk + j] = to_seg(pc.kv[j]);
        p.kv_lo[np] = (int8_t)nk;
        p.kv_hi[np] = (int8_t)(nk + pc.kv.size());
        p.q[np] = pc.pr->q;
        p.k[np] = pc.pr->k;
        p.v[np] = pc.pr->v;
        p.o[np] = pc.pr->o;
        p.lse[np] = pc.pr->lse;
        nq += (int)pc.q.size();
        nk += (int)pc.kv.size();
        ++np;
      }
      p.n_q_segs = nq;
      plan_tiles(p, bf16 ? cpk::kTileRowsBf16 : cpk::kTileRowsF32);
      if (p.total_tiles == 0) continue;
      const hipError_t e = bf16 ? cpk::launch_attn_bf16(p, d_h, s) : cpk::launch_attn_f32(p, d_h, s);
      st = launch_status(e, what);
      if (st) return st;
    }
  }
  return ok();
}

// Tile plan of one backward launch pair over one piece's tables: Q runs ordered by the causal
// work of their last tile (dQ workgroups, last tile of a run first), KV runs by the work of their
// first tile (dK/dV workgroups, first tile of a run first), heaviest first.
void plan_bwd(cpk::BwdParams& p, const Piece& pc, int q_rows_per_tile, int keys_per_tile) {
  p.n_q_segs = (int)pc.q.size();
  p.n_kv_segs = (int)pc.kv.size();
  for (int i = 0; i < p.n_q_segs; ++i) p.qs[i] = to_seg(pc.q[i]);
  for (int j = 0; j < p.n_kv_segs; ++j) p.ks[j] = to_seg(pc.kv[j]);
  std::vector<std::pair<int64_t, int>> qw, kw;
  for (int i = 0; i < p.n_q_segs; ++i) {
    const cpk::Seg& q = p.qs[i];
    const int64_t last = (int64_t)q.pos + q.len - 1;
    int64_t w = 0;
    for (int j = 0; j < p.n_kv_segs; ++j) {
      const cpk::Seg& k = p.ks[j];
      if (k.seq != q.seq) continue;
      w += p.causal ? std::min<int64_t>(k.len, std::max<int64_t>(0, last - k.pos + 1)) : k.len;
    }
    qw.push_back({w, i});
  }
  for (int j = 0; j < p.n_kv_segs; ++j) {
    const cpk::Seg& k = p.ks[j];
    int64_t w = 0;
    for (int i = 0; i < p.n_q_segs; ++i) {
      const cpk::Seg& q = p.qs[i];
      if (q.seq != k.seq) continue;
      w += p.causal ? std::min<int64_t>(q.len, std::max<int64_t>(0, (int64_t)q.pos + q.len - k.pos)) : q.len;
    }
    kw.push_back({w, j});
  }
  auto heavier = [](const std::pair<int64_t, int>& a, const std::pair<int64_t, int>& b) { return a.first > b.first; };
  std::stable_sort(qw.begin(), qw.end(), heavier);
  std::stable_sort(kw.begin(), kw.end(), heavier);
  p.q_prefix[0] = 0;
  for (int s2 = 0; s2 < p.n_q_segs; ++s2) {
    const int i = qw[s2].second;
    p.q_order[s2] = (int8_t)i;
    const int64_t rows = (int64_t)p.qs[i].len * p.group;
    p.q_prefix[s2 + 1] = p.q_prefix[s2] + (int)((rows + q_rows_per_tile - 1) / q_rows_per_tile);
  }
  p.q_tiles = p.q_prefix[p.n_q_segs];
  p.kv_prefix[0] = 0;
  for (int s2 = 0; s2 < p.n_kv_segs; ++s2) {
    const int j = kw[s2].second;
    p.kv_order[s2] = (int8_t)j;
    p.kv_prefix[s2 + 1] = p.kv_prefix[s2] + (p.ks[j].len + keys_per_tile - 1) / keys_per_tile;
  }
  p.kv_tiles = p.kv_prefix[p.n_kv_segs];
}

// Argument checks of one backward step beyond those of its forward problem.
int validate_bwd_extra(const float* lse, const float* delta, const void* d_o, const float* dq,
                       const float* dk, const float* dv, cp_dtype in_dtype, int n_q_segs, int n_kv_segs) {
  if (in_dtype != CP_BF16 && in_dtype != CP_F32) return fail(CP_E_ARG, "in_dtype=%d", (int)in_dtype);
  if (n_q_segs > 0 && (!lse || !delta || !d_o || !dq)) return fail(CP_E_ARG, "lse, delta, d_o or dq is NULL");
  if (n_kv_segs > 0 && (!dk || !dv)) return fail(CP_E_ARG, "dk or dv is NULL");
  if (!aligned16(d_o) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(CP_E_ARG, "d_o, dq, dk and dv must be 16-byte aligned");
  return CP_OK;
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

size_t cp_decode_workspace_bytes_ex(int batch, int n_h, int d_h, int n_splits, cp_dtype ws_dtype) {
  if (batch < 0 || n_h < 0 || d_h < 0 || n_splits < 0) return 0;
  if (ws_dtype != CP_F32 && ws_dtype != CP_BF16) return 0;
  const size_t parts = (size_t)batch * n_splits * n_h;
  const size_t elt = ws_dtype == CP_BF16 ? 2 : 4;
  return parts * d_h * elt + parts * sizeof(float);  // partial O, then fp32 LSE
}

size_t cp_decode_workspace_bytes(int batch, int n_h, int d_h, int n_splits) {
  return cp_decode_workspace_bytes_ex(batch, n_h, d_h, n_splits, CP_F32);
}

}  // extern "C"

namespace {

int device_cus();

// Argument checks of a decode call, apart from the workspace (nothing is launched).
int validate_decode(int batch, int n_h, int n_kv, int d_h, cp_dtype in_dtype, int n_splits,
                    float softmax_scale, cp_dtype ws_dtype, cp_dtype out_dtype) {
  int st = check_heads(n_h, n_kv, d_h);
  if (st) return st;
  if (in_dtype != CP_BF16) return fail(CP_E_UNSUPPORTED, "decode supports bf16 inputs only");
  if (out_dtype != CP_F32 && out_dtype != CP_BF16) return fail(CP_E_ARG, "out_dtype=%d", (int)out_dtype);
  if (ws_dtype != CP_F32 && ws_dtype != CP_BF16) return fail(CP_E_ARG, "ws_dtype=%d", (int)ws_dtype);
  if (batch < 0 || batch > 65535) return fail(CP_E_UNSUPPORTED, "batch=%d (0..65535)", batch);
  if (n_splits < 1 || n_splits > 1024) return fail(CP_E_UNSUPPORTED, "n_splits=%d (1..1024)", n_splits);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CP_E_ARG, "softmax_scale must be finite and > 0");
  const int group = n_h / n_kv;
  if ((int64_t)n_kv * ((group + 15) / 16) > 65535) return fail(CP_E_UNSUPPORTED, "too many head blocks");
  // the merge grid has one workgroup per (request, head) in one 32-bit dimension, 256 threads each
  if ((int64_t)batch * n_h * 256 > (int64_t)UINT32_MAX)
    return fail(CP_E_UNSUPPORTED, "batch * n_h = %lld too large", (long long)batch * n_h);
  return CP_OK;
}

}  // namespace

extern "C" {

int cp_decode_splitkv_ex(const void* q, const void* k_cache, const void* v_cache,
                         const int64_t* kv_offset, const int64_t* kv_len, int batch, int n_h,
                         int n_kv, int d_h, cp_dtype in_dtype, int n_splits, float softmax_scale,
                         cp_dtype ws_dtype, void* ws_o, float* ws_lse, void* o_out,
                         cp_dtype out_dtype, float* lse_out, void* stream) {
  int st = validate_decode(batch, n_h, n_kv, d_h, in_dtype, n_splits, softmax_scale, ws_dtype, out_dtype);
  if (st) return st;
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
  p.group = n_h / n_kv;
  p.n_splits = n_splits;
  p.out_bf16 = out_dtype == CP_BF16;
  p.ws_bf16 = ws_dtype == CP_BF16;
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  // Large batches take the persistent split kernel: one-wave workgroups, one per SIMD in each of
  // as many rounds as needed for at most kDecodeMaxUnits (request, split, head block) units per
  // wave, the units spread evenly over whole rounds; each wave stores its partials at its end.
  // Used from 4 units per wave up (fewer measured no faster). Requests are ranked by lanes, so at
  // most 64 of them; the unit count stays far inside int.
  const int64_t units = (int64_t)batch * n_splits * n_kv * ((p.group + 15) / 16);
  const int64_t slots = 4 * (int64_t)device_cus();
  int64_t per_wave = 0;
  if (slots > 0) {
    const int64_t rounds = (units + cpk::kDecodeMaxUnits * slots - 1) / (cpk::kDecodeMaxUnits * slots);
    per_wave = (units + rounds * slots - 1) / (rounds * slots);
  }
  p.units_per_wave = (batch <= 64 && per_wave >= 4 && units <= (1 << 24)) ? (int)per_wave : 0;
  return launch_status(cpk::launch_decode(p, d_h, static_cast<hipStream_t>(stream)), "cp_decode_splitkv");
}

int cp_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int64_t* kv_offset, const int64_t* kv_len, int batch, int n_h,
                              int n_kv, int d_h, cp_dtype in_dtype, int n_splits,
                              float softmax_scale, cp_dtype ws_dtype, void* o_out,
                              cp_dtype out_dtype, float* lse_out, void* stream) {
  int st = validate_decode(batch, n_h, n_kv, d_h, in_dtype, n_splits, softmax_scale, ws_dtype, out_dtype);
  if (st) return st;
  const size_t need = cp_decode_workspace_bytes_ex(batch, n_h, d_h, n_splits, ws_dtype);
  if (need > (size_t)CP_DECODE_NOALLOC_MAX_BYTES)
    return fail(CP_E_CAPACITY, "the split workspace needs %zu bytes; the library's scratch array holds %zu",
                need, (size_t)CP_DECODE_NOALLOC_MAX_BYTES);
  if (batch == 0) return ok();
  void* ws = nullptr;
  const hipError_t e = cpk::decode_scratch(&ws);
  if (e != hipSuccess) return fail(CP_E_HIP, "cp_decode_splitkv_noalloc: scratch lookup: %s", hipGetErrorString(e));
  const size_t o_bytes = (size_t)batch * n_splits * n_h * d_h * (ws_dtype == CP_BF16 ? 2 : 4);
  float* ws_lse = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + o_bytes);
  return cp_decode_splitkv_ex(q, k_cache, v_cache, kv_offset, kv_len, batch, n_h, n_kv, d_h,
                              in_dtype, n_splits, softmax_scale, ws_dtype, ws, ws_lse, o_out,
                              out_dtype, lse_out, stream);
}

int cp_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                      const int64_t* kv_offset, const int64_t* kv_len, int batch, int n_h,
                      int n_kv, int d_h, cp_dtype in_dtype, int n_splits, float softmax_scale,
                      float* ws_o, float* ws_lse, void* o_out, cp_dtype out_dtype, float* lse_out,
                      void* stream) {
  return cp_decode_splitkv_ex(q, k_cache, v_cache, kv_offset, kv_len, batch, n_h, n_kv, d_h,
                              in_dtype, n_splits, softmax_scale, CP_F32, ws_o, ws_lse, o_out,
                              out_dtype, lse_out, stream);
}

// delta = dO . O per row, the row term of the softmax gradient ([CPEP §6] backward).
int cp_attn_bwd_delta(const float* o, const void* d_o, cp_dtype do_dtype, int64_t rows, int d_h,
                      float* delta, void* stream) {
  if (rows < 0) return fail(CP_E_ARG, "rows=%lld", (long long)rows);
  if (d_h != 64 && d_h != 128) return fail(CP_E_UNSUPPORTED, "d_h=%d (64 or 128 supported)", d_h);
  if (do_dtype != CP_F32 && do_dtype != CP_BF16) return fail(CP_E_ARG, "do_dtype=%d", (int)do_dtype);
  if (rows > ((int64_t)1 << 40)) return fail(CP_E_UNSUPPORTED, "rows=%lld", (long long)rows);
  if (rows == 0) return ok();
  if (!o || !d_o || !delta) return fail(CP_E_ARG, "NULL pointer argument");
  return launch_status(cpk::launch_bwd_delta(o, d_o, do_dtype == CP_BF16, rows, d_h, delta,
                                             static_cast<hipStream_t>(stream)),
                       "cp_attn_bwd_delta");
}

// One ring step's backward ([CPEP §6]): gradient contributions of a Q shard against one KV shard,
// added into dq (the Q shard's) and dk, dv (the KV shard's, summed over the ranks that visit it).
size_t cp_attn_bwd_workspace_bytes(int d_h) {
  if (d_h != 64 && d_h != 128) return 0;
  return (size_t)cpk::kBwdMaxSlots * cpk::bwd_slot_bytes(d_h);
}

int cp_partial_attn_bwd(const void* q, const void* k, const void* v, int64_t tq, int64_t tk,
                        int n_h, int n_kv, int d_h, cp_dtype in_dtype, const cp_segment* q_segs,
                        int n_q_segs, const cp_segment* kv_segs, int n_kv_segs, int causal,
                        float softmax_scale, const float* lse, const float* delta, const void* d_o,
                        float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const Problem pr{q, k, v, tq, tk, q_segs, n_q_segs, kv_segs, n_kv_segs, dq, const_cast<float*>(lse)};
  int st = validate_problems(&pr, 1, n_h, n_kv, d_h, in_dtype, softmax_scale, 0);
  if (st) return st;
  st = validate_bwd_extra(lse, delta, d_o, dq, dk, dv, in_dtype, n_q_segs, n_kv_segs);
  if (st) return st;
  if (workspace && !aligned16(workspace)) return fail(CP_E_ARG, "workspace must be 16-byte aligned");
  std::vector<Piece> pieces;
  split_problem(pr, pieces);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (const Piece& pc : pieces) {  // pieces may share rows or keys: one launch pair each, in order
    cpk::BwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.d_o = d_o;
    p.lse = lse;
    p.delta = delta;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.n_h = n_h;
    p.n_kv = n_kv;
    p.group = n_h / n_kv;
    p.causal = causal ? 1 : 0;
    p.scale = softmax_scale;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    const bool bf16 = in_dtype == CP_BF16;
    plan_bwd(p, pc, bf16 ? cpk::kBwdQRows : cpk::kBwdF32Rows, bf16 ? cpk::kBwdKeys : cpk::kBwdF32Keys);
    if (p.q_tiles == 0 || p.kv_tiles == 0) continue;  // no pair of this piece can be visible
    // With a workspace, a launch with fewer key tiles than the split target divides each tile's
    // query rows into up to kBwdMaxParts parts (as many as the workspace holds).
    cpk::BwdSplit sp{nullptr, 1};
    const int64_t tiles = (int64_t)p.kv_tiles * n_kv;
    if (bf16 && workspace && tiles < cpk::kBwdSplitTarget) {
      int64_t parts = std::min<int64_t>(cpk::kBwdMaxParts, (cpk::kBwdSplitTarget + tiles - 1) / tiles);
      parts = std::min<int64_t>(parts, (int64_t)(workspace_bytes / cpk::bwd_slot_bytes(d_h)) / tiles);
      if (parts > 1) sp = cpk::BwdSplit{static_cast<float*>(workspace), (int32_t)parts};
    }
    st = launch_status(bf16 ? cpk::launch_bwd_split(p, sp, d_h, s) : cpk::launch_bwd_f32(p, d_h, s),
                       "cp_partial_attn_bwd");
    if (st) return st;
  }
  return ok();
}

// Ring Pass-KV backward on one device ([CPEP §6]; [CPMTI §3 Fig. 3]): delta of the rank's rows,
// then at step t the rank's contributions against KV shard (rank - t) mod N, its dK/dV added into
// that shard's accumulators (on one device the reduce-scatter is this sum).
int cp_ring_pass_kv_bwd(const void* q, int64_t tq, const cp_segment* q_segs, int n_q_segs,
                        int cp_world, int rank, const void* const* k_shards,
                        const void* const* v_shards, const int64_t* tk,
                        const cp_segment* const* kv_segs, const int* n_kv_segs, int n_h, int n_kv,
                        int d_h, cp_dtype in_dtype, int causal, float softmax_scale, const float* o,
                        const float* lse, const void* d_o, float* delta, float* dq,
                        float* const* dk_shards, float* const* dv_shards, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (cp_world < 1 || cp_world > cpk::kMaxParts) return fail(CP_E_ARG, "cp_world=%d", cp_world);
  if (rank < 0 || rank >= cp_world) return fail(CP_E_ARG, "rank=%d", rank);
  if (!k_shards || !v_shards || !tk || !kv_segs || !n_kv_segs || !dk_shards || !dv_shards)
    return fail(CP_E_ARG, "shard arrays are NULL");
  if (!o && tq > 0) return fail(CP_E_ARG, "o is NULL");
  std::vector<Problem> steps(cp_world);
  for (int t = 0; t < cp_world; ++t) {
    const int s = ((rank - t) % cp_world + cp_world) % cp_world;
    steps[t] = Problem{q, k_shards[s], v_shards[s], tq, tk[s], q_segs, n_q_segs, kv_segs[s],
                       n_kv_segs[s], dq, const_cast<float*>(lse)};
  }
  int st = validate_problems(steps.data(), cp_world, n_h, n_kv, d_h, in_dtype, softmax_scale, 0);
  if (st) return st;
  for (int t = 0; t < cp_world; ++t) {
    const int s = ((rank - t) % cp_world + cp_world) % cp_world;
    st = validate_bwd_extra(lse, delta, d_o, dq, dk_shards[s], dv_shards[s], in_dtype, n_q_segs,
                            n_kv_segs[s]);
    if (st) return st;
  }
  if (workspace && !aligned16(workspace)) return fail(CP_E_ARG, "workspace must be 16-byte aligned");
  st = cp_attn_bwd_delta(o, d_o, in_dtype, tq * (int64_t)n_h, d_h, delta, stream);
  if (st) return st;
  for (int t = 0; t < cp_world; ++t) {
    const int s = ((rank - t) % cp_world + cp_world) % cp_world;
    st = cp_partial_attn_bwd(q, k_shards[s], v_shards[s], tq, tk[s], n_h, n_kv, d_h, in_dtype,
                             q_segs, n_q_segs, kv_segs[s], n_kv_segs[s], causal, softmax_scale, lse,
                             delta, d_o, dq, dk_shards[s], dv_shards[s], workspace,
                             workspace_bytes, stream);
    if (st) return st;
  }
  return ok();
}

// Ring Pass-KV ([CPMTI §3 "核心公式"; Fig. 3]): the rank keeps its Q shard; at step t it holds the
// KV shard that started on rank (rank - t) mod N.
// Most parts one running-mode ring step is split into (and one launch carries).
constexpr int kMaxRingSplit = 8;

size_t cp_ring_workspace_bytes(int64_t tq, int n_h, int d_h) {
  if (tq < 0 || n_h <= 0 || d_h <= 0) return 0;
  const size_t rows = (size_t)tq * (size_t)n_h;
  return round_up256(rows * (size_t)d_h * sizeof(float)) + round_up256(rows * sizeof(float));
}

namespace {

// CUs of the current device (looked up once per device).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
  cache[dev] = cus;
  return cus;
}

// The keys of one ring step divided into `parts` pieces: every KV run is cut at whole numbers
// of 64-key tiles near i/parts of its length; piece i of every run goes to out[i] (empty pieces
// are dropped, so a run of fewer than 64 * parts keys lands in fewer pieces).
void split_kv_runs(const cp_segment* runs, int n, int parts, std::vector<std::vector<cp_segment>>& out) {
  out.assign(parts, std::vector<cp_segment>());
  for (int j = 0; j < n; ++j) {
    const cp_segment& r = runs[j];
    for (int i = 0; i < parts; ++i) {
      const int64_t b0 = i == 0 ? 0 : r.len * i / parts / 64 * 64;
      const int64_t b1 = i == parts - 1 ? r.len : r.len * (i + 1) / parts / 64 * 64;
      if (b1 <= b0) continue;
      cp_segment x = r;
      x.pos_start = r.pos_start + b0;
      x.local_start = r.local_start + b0;
      x.len = b1 - b0;
      out[i].push_back(x);
    }
  }
}

}  // namespace

int cp_ring_pass_kv(const void* q, int64_t tq, const cp_segment* q_segs, int n_q_segs,
                    int cp_world, int rank, const void* const* k_shards,
                    const void* const* v_shards, const int64_t* tk,
                    const cp_segment* const* kv_segs, const int* n_kv_segs, int n_h, int n_kv,
                    int d_h, cp_dtype in_dtype, int causal, float softmax_scale,
                    float* const* o_parts, float* const* lse_parts, float* o_acc, float* lse_acc,
                    void* o_out, cp_dtype out_dtype, float* lse_out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (cp_world < 1 || cp_world > cpk::kMaxParts) return fail(CP_E_ARG, "cp_world=%d", cp_world);
  if (rank < 0 || rank >= cp_world) return fail(CP_E_ARG, "rank=%d", rank);
  if (!k_shards || !v_shards || !tk || !kv_segs || !n_kv_segs) return fail(CP_E_ARG, "shard arrays are NULL");
  const bool partials = o_parts != nullptr;
  if (partials && !lse_parts) return fail(CP_E_ARG, "lse_parts is NULL");
  if (!partials && (!o_acc || !lse_acc)) return fail(CP_E_ARG, "running mode needs o_acc and lse_acc");
  if (!o_out) return fail(CP_E_ARG, "o_out is NULL");
  if (workspace && !aligned16(workspace)) return fail(CP_E_ARG, "workspace must be 16-byte aligned");
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
  if (partials) {
    // The steps write separate partials, so on one device (every shard resident) they are
    // independent: they go to the GPU together, up to 8 problems per launch. A rank's small Q shard
    // then fills the chip where one step alone would not.
    st = partial_attn_problems(steps.data(), cp_world, n_h, n_kv, d_h, in_dtype, causal,
                               softmax_scale, 0, stream, "cp_ring_pass_kv");
    if (st) return st;
    return cp_merge_lse(cp_world, o_parts, lse_parts, rows, d_h, o_out, out_dtype, lse_out, stream);
  }
  // Running mode: each step folds into (o_acc, lse_acc), so the steps run in ring order. A step
  // whose Q tiles cannot fill the CUs is split over its keys when a workspace is given: its parts
  // go to the GPU in one launch, the first folding into the running result and each other one
  // into a workspace partial (both from an empty result), and the partials are then merged into
  // (o_acc, lse_acc) in place.
  const size_t part_bytes = cp_ring_workspace_bytes(tq, n_h, d_h);
  const int64_t ws_parts = workspace && part_bytes > 0 ? (int64_t)(workspace_bytes / part_bytes) : 0;
  int64_t q_tiles = 0;
  for (int i = 0; i < n_q_segs; ++i)
    q_tiles += (q_segs[i].len * (n_h / n_kv) + cpk::kTileRowsBf16 - 1) / cpk::kTileRowsBf16;
  q_tiles *= n_kv;
  const int cus = ws_parts > 0 && in_dtype == CP_BF16 ? device_cus() : 0;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto ws_o = [&](int i) {  // O of workspace partial i (i >= 1), then its LSEs
    return reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + (size_t)(i - 1) * part_bytes);
  };
  auto ws_lse = [&](int i) {
    return reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(ws_o(i)) +
                                    round_up256((size_t)rows * d_h * sizeof(float)));
  };
  bool filled = false;  // (o_acc, lse_acc) holds a result (or the empty one)
  for (int t = 0; t < cp_world; ++t) {
    const Problem& pr = steps[t];
    int64_t keys = 0;
    for (int j = 0; j < pr.n_kv_segs; ++j) keys += pr.kv_segs[j].len;
    // parts: enough to fill the CUs, at least 2048 keys each, at most kMaxRingSplit
    int64_t parts = 1;
    if (cus > 0 && q_tiles > 0 && q_tiles < cus)
      parts = std::min<int64_t>({(int64_t)kMaxRingSplit, (cus + q_tiles - 1) / q_tiles, keys / 2048,
                                 ws_parts + 1});
    std::vector<std::vector<cp_segment>> pk;
    if (parts > 1) split_kv_runs(pr.kv_segs, pr.n_kv_segs, (int)parts, pk);
    int used = 0;  // non-empty parts, in order
    for (const auto& v : pk) used += v.empty() ? 0 : 1;
    if (used < 2) {  // not split
      st = partial_attn_problems(&pr, 1, n_h, n_kv, d_h, in_dtype, causal, softmax_scale,
                                 filled ? 1 : 0, stream, "cp_ring_pass_kv");
      if (st) return st;
      filled = true;
      continue;
    }
    std::vector<Problem> probs;
    std::vector<const float*> mo, ml;
    for (const auto& v : pk) {
      if (v.empty()) continue;
      Problem x = pr;
      x.kv_segs = v.data();
      x.n_kv_segs = (int)v.size();
      const int i = (int)probs.size();
      if (i > 0) {
        x.o = ws_o(i);
        x.lse = ws_lse(i);
      }
      probs.push_back(x);
      mo.push_back(x.o);
      ml.push_back(x.lse);
    }
    if (!filled) {
      st = launch_status(cpk::launch_fill_running(o_acc, lse_acc, rows, d_h, hs), "cp_ring_pass_kv");
      if (st) return st;
      filled = true;
    }
    for (int i = 1; i < (int)probs.size(); ++i) {
      st = launch_status(cpk::launch_fill_running(ws_o(i), ws_lse(i), rows, d_h, hs), "cp_ring_pass_kv");
      if (st) return st;
    }
    st = partial_attn_problems(probs.data(), (int)probs.size(), n_h, n_kv, d_h, in_dtype, causal,
                               softmax_scale, 1, stream, "cp_ring_pass_kv");
    if (st) return st;
    st = cp_merge_lse((int)probs.size(), mo.data(), ml.data(), rows, d_h, o_acc, CP_F32, lse_acc, stream);
    if (st) return st;
  }
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
  // Step t: the rank holding KV shard s computes Q shard (s - t) mod N against it. Every one of the
  // N*N partials lands in a slot of its own, so on one GPU they are all independent: they go to the
  // GPU in ring-step order, as many problems per launch as the kernel's tables take (two steps of
  // a 4-rank ring per launch). All N*N partials and the N merges are validated before the first
  // launch.
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
  {
    const int st = partial_attn_problems(all.data(), N * N, n_h, n_kv, d_h, in_dtype, causal,
                                         softmax_scale, 0, stream, "cp_ring_pass_q");
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
