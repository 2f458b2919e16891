// decode.hip -- split-KV decode: one new query token per request against its cached K/V,
// split S ways into partial (O, LSE) results that are then merged.
//
// [CPMTI §5 "软件栈"]: decode uses Flash Decoding with 256 splits; [CPMTI §4 "解码阶段CP"]: decode
// runs ring Pass-Q, i.e. partials over KV shards merged afterwards; [CPEP §5.2]: at decode one
// query reads the whole KV cache; [CPEP §8.2]: the query heads of a group share their KV head.
//
// The split kernel streams K and V once from HBM (the work is bandwidth-bound: 16 query heads
// against one KV head give 16 flops per byte of cache). One wave owns one (request, split,
// 16-head block) and walks its keys in blocks of 32; for small batches four waves share a split,
// each taking a quarter of its keys, and combine their results in LDS; for large batches (4 or
// more such units per SIMD) one wave per SIMD, in one or more rounds, walks up to 8 units in
// turn, keeps their partials in registers and stores them all at its end, so that the partial
// writes do not mix with the K/V read stream. The walk of a unit is the same in all three forms:
//  - K and V blocks are loaded with whole-row 16-byte non-temporal accesses (the cache is read
//    once; the loads must not evict the split partials the merge reads back) and staged in LDS
//    in their row-major layout;
//  - S^T = K q^T on v_mfma_f32_16x16x32_bf16: 16 keys x 16 heads per MFMA, q^T held in
//    registers;
//  - V comes back from LDS as the V^T operand of O^T += V^T P^T via ds_read_b64_tr_b16;
//  - the next block's K and V loads are issued before the current block's math, and the first
//    block's loads are in flight together with the query's.
// Each split's partial O is normalised (a convex combination of V rows) and stored in the
// workspace in fp32 (the default: the merge then rounds nothing), or in bf16 when the caller asks
// for the half-size workspace; its LSE is always fp32. The merge kernel then combines the S
// partials of each (request, head) with the same LSE-weighted rule as cp_merge_lse.
//
// Pages cited: [CPEP] "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두
// 축"; [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (paper review).
#include <mutex>

#include "device_common.h"

namespace cpk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
// Native vector for 16-byte staging (arrays of HIP's uint4 struct are not promoted to registers).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct DecCfg {
  static constexpr int kBK = 32;                 // keys per block
  // Padded LDS rows: K rows are read 16 bytes per lane by 16 lanes on 16 rows (stride 4 mod 64
  // dwords keeps them on disjoint bank quads); V rows by the transposing loads, 8 rows x 32
  // bytes per half-wave (stride 8 mod 64 dwords keeps the eight runs disjoint).
  static constexpr int kStrideK = D * 2 + 16;
  static constexpr int kStrideV = D * 2 + 32;
  static constexpr int kStageBytes = kBK * (kStrideK + kStrideV);  // one wave's K and V block
  static constexpr int kKSteps = D / 32;         // MFMA k-steps over the head dimension
  static constexpr int kDBlocks = D / 16;        // 16-row blocks of O^T
  static constexpr int kChunks = D / 8;          // 16-byte chunks per key row
  static constexpr int kVLoads = kBK * kChunks / 64;
};

// Rank of request i by cached length, longest first (ties by index); batch <= 64, one request per
// lane.
__device__ __forceinline__ int request_rank(const DecodeParams& p, int i) {
  const int64_t li = i < p.batch ? p.kv_len[i] : -1;
  int rank = 0;
  for (int j = 0; j < p.batch; ++j) {
    const int64_t lj = p.kv_len[j];
    rank += (lj > li) || (lj == li && j < i);
  }
  return rank;
}

// The request of rank `want`, from every lane's request_rank (wave-uniform call; batch <= 64).
__device__ __forceinline__ int request_of_rank(const DecodeParams& p, int lane, int lane_rank, int want) {
  const unsigned long long hit = __ballot(lane < p.batch && lane_rank == want);
  return __ffsll(hit) - 1;
}

// One wave walks keys [wlo, wlo + n) of request b for the 16 query heads h0.. of KV head g and
// leaves the running max m (base-2 units, the same in every lane of a head column), the lane's
// part of the row sum l, and the unnormalised O^T accumulators. ks / vs: the wave's own staging
// LDS (its accesses are ordered among themselves, so no barrier is needed).
template <int D>
__device__ __forceinline__ void decode_walk(const DecodeParams& p, unsigned char* ks, unsigned char* vs,
                                            int lane, int b, int g, int h0, int64_t wlo, int n,
                                            float& m, float& l, f32x4 (&oacc)[D / 16]) {
  using C = DecCfg<D>;
  const int col = lane & 15;  // head column of the 16x16 blocks
  const int grp = lane >> 4;  // 0..3: k slice of the operands, row group of the accumulator
  const int64_t base = p.kv_offset[b];
  const __bf16* __restrict__ Kc = static_cast<const __bf16*>(p.k);
  const __bf16* __restrict__ Vc = static_cast<const __bf16*>(p.v);

  // q^T operand: lane holds q[head h0+col][st*32 + grp*8 + e] (the K operand uses the same
  // permutation of the head dimension, so the MFMA's reduction covers every d once)
  const int hig = h0 + col;
  const bool head_ok = hig < p.group;
  const int head = g * p.group + (head_ok ? hig : 0);
  bf16x8 qreg[C::kKSteps];
  {
    const __bf16* qp = static_cast<const __bf16*>(p.q) + ((int64_t)b * p.n_h + head) * D + grp * 8;
#pragma unroll
    for (int st = 0; st < C::kKSteps; ++st) {
      qreg[st] = *reinterpret_cast<const bf16x8*>(qp + st * 32);
      if (!head_ok) qreg[st] = bf16x8{};
    }
  }

  // Loads of one 32-key block: every instruction reads four whole key rows (16 lanes x 16
  // bytes per row), non-temporal (the cache is streamed once).
  const __bf16* Kr = Kc + (base + wlo) * p.n_kv * D + (int64_t)g * D;
  const __bf16* Vr = Vc + (base + wlo) * p.n_kv * D + (int64_t)g * D;
  const int64_t row_stride = (int64_t)p.n_kv * D;
  u32x4 kr[C::kVLoads], vr[C::kVLoads];
#define CP_DEC_LOAD(KB0)                                                             \
  _Pragma("unroll") for (int i = 0; i < C::kVLoads; ++i) {                           \
    const int idx = i * 64 + lane;                                                   \
    const int key = min((KB0) + idx / C::kChunks, n - 1);                            \
    const int64_t off = key * row_stride + (idx % C::kChunks) * 8;                   \
    vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vr + off));    \
    kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kr + off));    \
  }
#define CP_DEC_STORE()                                                               \
  _Pragma("unroll") for (int i = 0; i < C::kVLoads; ++i) {                           \
    const int idx = i * 64 + lane;                                                   \
    const int row = idx / C::kChunks, c16 = (idx % C::kChunks) * 16;                 \
    *reinterpret_cast<u32x4*>(vs + row * C::kStrideV + c16) = vr[i];                 \
    *reinterpret_cast<u32x4*>(ks + row * C::kStrideK + c16) = kr[i];                 \
  }

  m = -INFINITY;
  l = 0.f;
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tr-read addressing: lane group grp reads 4 key rows, 4 lanes per row, 4 d per lane
  const int j16 = lane & 15;
  const int tr_row = 4 * grp + (j16 >> 2);
  const int tr_col = 4 * (j16 & 3);

  if (n > 0) CP_DEC_LOAD(0);
  // retire the q and first-block loads together before the block loop (keeps the loop's
  // prefetch out of its waits)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (n > 0) CP_DEC_STORE();
  for (int kb0 = 0; kb0 < n; kb0 += C::kBK) {
    const bool has_next = kb0 + C::kBK < n;
    if (has_next) CP_DEC_LOAD(kb0 + C::kBK);

    // S^T (keys x heads) for the two 16-key halves; K operand: key row col, d slice of grp
    f32x4 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < C::kKSteps; ++st) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(ks + (16 * h + col) * C::kStrideK + (st * 32 + grp * 8) * 2);
        s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[st], s[h], 0, 0, 0);
      }
    }
    // keys past the wave's part are masked
    if (kb0 + C::kBK > n) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (kb0 + 16 * h + 4 * grp + v >= n) s[h][v] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[h][v]);
    mx = max_xor32(max_xor16(mx));
    const float mnew = fmaxf(m, mx * p.scale_log2);  // the block always holds a visible key
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    bf16x8 pt;
    float rs = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[h][v], p.scale_log2, -mnew));
        rs += e;
        pt[4 * h + v] = (__bf16)e;
      }
    l = l * alpha + rs;
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) oacc[db] *= alpha;

    // O^T += V^T P^T: operand k = 4h + v <-> key 16h + 4*grp + v
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) {
      const int off = tr_row * C::kStrideV + (db * 16 + tr_col) * 2;
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vs + off));
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vs + off + 16 * C::kStrideV));
      const i16x8 both = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, both), pt,
                                                          oacc[db], 0, 0, 0);
    }
    if (has_next) CP_DEC_STORE();  // after this block's LDS reads (same wave: in order)
  }
#undef CP_DEC_LOAD
#undef CP_DEC_STORE
}

// Stores the partial of (request b, split c, 16-head block h0 of KV head g): the normalised O
// (a lane holds 4-value pieces of head column col's row) and the lane's LSE (natural log), for
// the heads that exist. The workspace layout [batch][n_splits][n_h][D] makes those heads' rows
// one contiguous block. Stored directly, every instruction would write 16 separate pieces; the
// tile goes through the wave's staging LDS `tile` instead (no longer read; the wave's LDS
// accesses are in order) and leaves as whole rows, 16 bytes per lane, each instruction covering
// 1 KB of consecutive bytes.
template <int D, bool WS_BF16>
__device__ __forceinline__ void decode_store(const DecodeParams& p, unsigned char* tile, int lane, int b,
                                             int c, int g, int h0, const f32x4 (&o)[D / 16], float lse) {
  using C = DecCfg<D>;
  const int col = lane & 15;
  const int grp = lane >> 4;
  constexpr int kElt = WS_BF16 ? 2 : 4;        // bytes per stored value
  constexpr int kRowBytes = D * kElt;
  // padded LDS rows: the 16 head rows written by one instruction land on distinct banks
  constexpr int kTStride = kRowBytes + (WS_BF16 ? 32 : 16);
  static_assert(16 * kTStride <= C::kStageBytes, "the tile fits the wave's staging LDS");
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db) {
    unsigned char* dst = tile + col * kTStride + (db * 16 + 4 * grp) * kElt;
    if constexpr (WS_BF16) {
      const bf16x4 o4 = {(__bf16)o[db][0], (__bf16)o[db][1], (__bf16)o[db][2], (__bf16)o[db][3]};
      *reinterpret_cast<bf16x4*>(dst) = o4;
    } else {
      *reinterpret_cast<f32x4*>(dst) = o[db];
    }
  }
  const int n_valid = min(16, p.group - h0);  // heads of this block that exist
  const int64_t prow0 = ((int64_t)b * p.n_splits + c) * p.n_h + g * p.group + h0;
  unsigned char* wo = static_cast<unsigned char*>(p.ws_o) + prow0 * kRowBytes;
  constexpr int kLanesPerRow = kRowBytes / 16;
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += kRowsPerStore) {
    const int r = r0 + lane / kLanesPerRow;
    const int c16 = (lane % kLanesPerRow) * 16;
    if (r < n_valid)
      *reinterpret_cast<u32x4*>(wo + r * kRowBytes + c16) = *reinterpret_cast<const u32x4*>(tile + r * kTStride + c16);
  }
  if (grp == 0 && h0 + col < p.group) p.ws_lse[prow0 + col] = lse;
}

// W waves share one (request, split, 16-head block): wave w takes the w-th of W equal parts of
// the split's keys with LDS of its own, and the W partial results are combined in LDS before
// the split's partial is written. W = 1 for large batches (enough workgroups to fill the chip);
// W = 4 for small ones, where one wave per split would leave most of each CU idle.
template <int D, int W, bool WS_BF16>
__global__ __launch_bounds__(64 * W) void decode_split_kernel(const DecodeParams p) {
  using C = DecCfg<D>;
  // combine area: per wave 16 heads x (D values of O + m + l), in fp32
  constexpr int kCombineBytes = W > 1 ? W * 16 * (D + 2) * 4 : 0;
  constexpr int kLdsBytes = W * C::kStageBytes > kCombineBytes ? W * C::kStageBytes : kCombineBytes;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];

  const int wave = W > 1 ? (int)(threadIdx.x / 64) : 0;
  const int lane = threadIdx.x & 63;
  unsigned char* ks = smem + wave * C::kStageBytes;
  unsigned char* vs = ks + C::kBK * C::kStrideK;

  const int c = blockIdx.x % p.n_splits;  // split (fastest: neighbours stream adjacent keys)
  // Requests are taken longest first, so the last workgroups to be dispatched are the shortest
  // splits and the tail of the launch stays short (for batches of up to 64 requests; the
  // workgroup takes the request of rank blockIdx / S).
  int b = blockIdx.x / p.n_splits;
  if (p.batch <= 64) b = request_of_rank(p, lane, request_rank(p, lane), b);
  const int hblocks = (p.group + 15) / 16;
  const int g = blockIdx.y / hblocks;
  const int h0 = (blockIdx.y % hblocks) * 16;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t L = p.kv_len[b] > 0 ? p.kv_len[b] : 0;  // a negative length reads as an empty cache
  const int64_t lo = ((int64_t)c * L) / p.n_splits;
  const int64_t hi = ((int64_t)(c + 1) * L) / p.n_splits;
  // this wave's part of the split
  const int64_t wlo = lo + ((hi - lo) * wave) / W;
  const int64_t whi = lo + ((hi - lo) * (wave + 1)) / W;

  float m, l;
  f32x4 oacc[C::kDBlocks];
  decode_walk<D>(p, ks, vs, lane, b, g, h0, wlo, (int)(whi - wlo), m, l, oacc);

  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  if constexpr (W > 1) {
    // combine the W parts (m in base-2 units, the same in every lane of a head column)
    float* cm = reinterpret_cast<float*>(smem);  // [W][16] max
    float* cl = cm + W * 16;                     // [W][16] sum
    float* co = cl + W * 16;                     // [W][16][D] unnormalised O
    __syncthreads();                             // every wave is done with its staging LDS
    if (grp == 0) {
      cm[wave * 16 + col] = m;
      cl[wave * 16 + col] = lt;
    }
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) co[(wave * 16 + col) * D + db * 16 + 4 * grp + v] = oacc[db][v];
    __syncthreads();
    if (wave != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, cm[w * 16 + col]);
    float wt[W];
    lt = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = cm[w * 16 + col];
      wt[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);  // a part with no key: 0
      lt += wt[w] * cl[w * 16 + col];
    }
    m = M;
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) o = fmaf(wt[w], co[(w * 16 + col) * D + db * 16 + 4 * grp + v], o);
        oacc[db][v] = o;
      }
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  f32x4 o[C::kDBlocks];
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db) o[db] = oacc[db] * inv;
  decode_store<D, WS_BF16>(p, ks, lane, b, c, g, h0, o, lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY);
}

// Unit `pos` of the persistent split kernel: units are numbered request rank major (longest
// request first), then KV head and head block, then split.
__device__ __forceinline__ void decode_unit_coords(const DecodeParams& p, int lane, int lane_rank, int pos,
                                                   int per_req, int hblocks, int& b, int& c, int& g,
                                                   int& h0) {
  const int r = pos / per_req;
  const int rem = pos - r * per_req;
  const int y = rem / p.n_splits;
  c = rem - y * p.n_splits;
  b = request_of_rank(p, lane, lane_rank, r);
  g = y / hblocks;
  h0 = (y - g * hblocks) * 16;
}

// Large batches (batch <= 64, 4 or more units per SIMD): one-wave workgroups, one per SIMD in each
// of one or more rounds, each walking p.units_per_wave (at most kDecodeMaxUnits) (request, split,
// 16-head block) units in turn, each as decode_split_kernel's
// one-wave walk, and keeps every finished partial (normalised O and LSE) in registers; it stores
// them all when it is done. Units are dealt in a zigzag over the longest-first numbering (wave w
// takes units w, 2G-1-w, 2G+w, ... of a grid of G waves), which gives every wave about the same
// number of keys. The splits and their partials are those of decode_split_kernel; only when the
// partials reach HBM changes: the waves of a round finish together, so the partial writes leave in
// one burst per round instead of mixing with the K/V stream throughout the launch (interleaved
// writes slow the read stream far more than their own bytes cost).
template <int D, bool WS_BF16>
__global__ __launch_bounds__(64) void decode_split_persist_kernel(const DecodeParams p) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::kStageBytes];
  const int lane = threadIdx.x;
  unsigned char* ks = smem;
  unsigned char* vs = smem + C::kBK * C::kStrideK;
  const int G = (int)gridDim.x, w = (int)blockIdx.x;
  const int hblocks = (p.group + 15) / 16;
  const int per_req = p.n_splits * p.n_kv * hblocks;  // the host bounds the unit count to int
  const int units = per_req * p.batch;
  const int lane_rank = request_rank(p, lane);

  f32x4 park[kDecodeMaxUnits][C::kDBlocks];
  float park_lse[kDecodeMaxUnits];
  int park_pos[kDecodeMaxUnits];
#pragma unroll
  for (int s = 0; s < kDecodeMaxUnits; ++s) {
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) park[s][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    park_lse[s] = -INFINITY;
    park_pos[s] = 0;
  }
  int done = 0;
  for (int k = 0; k < p.units_per_wave; ++k) {
    const int pos = k * G + ((k & 1) ? G - 1 - w : w);
    if (pos >= units) break;  // later units of this wave lie further on
    int b, c, g, h0;
    decode_unit_coords(p, lane, lane_rank, pos, per_req, hblocks, b, c, g, h0);
    const int64_t L = p.kv_len[b] > 0 ? p.kv_len[b] : 0;
    const int64_t lo = ((int64_t)c * L) / p.n_splits;
    const int64_t hi = ((int64_t)(c + 1) * L) / p.n_splits;
    float m, l;
    f32x4 oacc[C::kDBlocks];
    decode_walk<D>(p, ks, vs, lane, b, g, h0, lo, (int)(hi - lo), m, l, oacc);
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // park: slot 0 takes this unit, the others move up one (static register indices)
#pragma unroll
    for (int s = kDecodeMaxUnits - 1; s > 0; --s) {
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db) park[s][db] = park[s - 1][db];
      park_lse[s] = park_lse[s - 1];
      park_pos[s] = park_pos[s - 1];
    }
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db) park[0][db] = oacc[db] * inv;
    park_lse[0] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
    park_pos[0] = pos;
    ++done;
  }
#pragma unroll
  for (int s = 0; s < kDecodeMaxUnits; ++s) {
    if (s < done) {
      int b, c, g, h0;
      decode_unit_coords(p, lane, lane_rank, park_pos[s], per_req, hblocks, b, c, g, h0);
      decode_store<D, WS_BF16>(p, ks, lane, b, c, g, h0, park[s], park_lse[s]);
    }
  }
}

// Merge of the S split partials of each (request, head): DS workgroups per (request, head), each
// taking D / DS of the head dimension (DS > 1 for small batches: more workgroups, each with less
// to read). The partials are S rows of D values (fp32, or bf16 for the half-size workspace) and S
// fp32 LSEs, n_h rows apart. A lane loads 16 bytes of a row (4 fp32 or 8 bf16 values); D / DS /
// (values per lane) lanes cover the workgroup's slice and the 256 threads form kGroups lane
// groups that take every kGroups-th split. A lane issues the loads of up to kBatch splits (their
// LSEs and O slices) before combining any of them; batches are folded into a running max, weight
// and sum. The groups are then combined through LDS in a fixed order (deterministic), and every
// workgroup of a row derives the same weights from the same LSEs.
template <int D, int DS, bool OUT_BF16, bool WS_BF16>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeParams p) {
  constexpr int kVals = WS_BF16 ? 8 : 4;  // values per 16-byte load
  constexpr int kLanes = D / DS / kVals;
  constexpr int kGroups = 256 / kLanes;
  constexpr int kBatch = 16;
  __shared__ float red_m[kGroups];
  __shared__ float red_w[kGroups];
  __shared__ float red_o[kGroups][kLanes][kVals];
  const int r = blockIdx.x / DS;  // b * n_h + head
  const int piece = blockIdx.x % DS;
  const int grp = threadIdx.x / kLanes;
  const int cl = threadIdx.x % kLanes;  // 16-byte column within the slice
  const int cv = piece * kLanes + cl;   // and within the row
  const int64_t row0 = (int64_t)(r / p.n_h) * p.n_splits * p.n_h + r % p.n_h;  // split 0's row
  const float* lse = p.ws_lse + row0;
  const unsigned char* o = static_cast<const unsigned char*>(p.ws_o) + (row0 * D + cv * kVals) * (WS_BF16 ? 2 : 4);
  const int64_t stride_b = (int64_t)p.n_h * D * (WS_BF16 ? 2 : 4);  // bytes between splits

  float M = -INFINITY, wsum = 0.f;
  float acc[kVals];
#pragma unroll
  for (int e = 0; e < kVals; ++e) acc[e] = 0.f;
  for (int c0 = grp; c0 < p.n_splits; c0 += kGroups * kBatch) {
    float li[kBatch];
    u32x4 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = min(c0 + i * kGroups, p.n_splits - 1);  // clamped: in bounds, masked below
      li[i] = c0 + i * kGroups < p.n_splits ? lse[(int64_t)c * p.n_h] : -INFINITY;
      v[i] = *reinterpret_cast<const u32x4*>(o + c * stride_b);
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) Mb = fmaxf(Mb, li[i]);
    if (Mb == -INFINITY) continue;  // nothing seen yet
    const float a = expf(M - Mb);    // M = -inf -> 0
    wsum *= a;
#pragma unroll
    for (int e = 0; e < kVals; ++e) acc[e] *= a;
    M = Mb;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float w = expf(li[i] - M);  // -inf -> 0: the part saw no key
      if (w == 0.f) continue;           // skip its O, which may be anything
      wsum += w;
      if constexpr (WS_BF16) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, v[i]);
#pragma unroll
        for (int e = 0; e < kVals; ++e) acc[e] = fmaf(w, (float)x[e], acc[e]);
      } else {
        const f32x4 x = __builtin_bit_cast(f32x4, v[i]);
#pragma unroll
        for (int e = 0; e < kVals; ++e) acc[e] = fmaf(w, x[e], acc[e]);
      }
    }
  }
  if (cl == 0) red_m[grp] = M;
  __syncthreads();
  float Mt = red_m[0];
#pragma unroll
  for (int i = 1; i < kGroups; ++i) Mt = fmaxf(Mt, red_m[i]);
  const float a = (M == -INFINITY) ? 0.f : expf(M - Mt);
#pragma unroll
  for (int e = 0; e < kVals; ++e) red_o[grp][cl][e] = acc[e] * a;
  if (cl == 0) red_w[grp] = wsum * a;
  __syncthreads();
  if (grp != 0) return;
  wsum = 0.f;
#pragma unroll
  for (int e = 0; e < kVals; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < kGroups; ++i) {  // fixed order: deterministic
    wsum += red_w[i];
#pragma unroll
    for (int e = 0; e < kVals; ++e) acc[e] += red_o[i][cl][e];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t orow = (int64_t)r * D + cv * kVals;
  if constexpr (OUT_BF16) {
    __bf16* out = static_cast<__bf16*>(p.o_out) + orow;
#pragma unroll
    for (int e0 = 0; e0 < kVals; e0 += 4) {
      const bf16x4 o4 = {(__bf16)(acc[e0] * inv), (__bf16)(acc[e0 + 1] * inv),
                         (__bf16)(acc[e0 + 2] * inv), (__bf16)(acc[e0 + 3] * inv)};
      *reinterpret_cast<bf16x4*>(out + e0) = o4;
    }
  } else {
    float* out = static_cast<float*>(p.o_out) + orow;
#pragma unroll
    for (int e0 = 0; e0 < kVals; e0 += 4)
      *reinterpret_cast<float4*>(out + e0) =
          make_float4(acc[e0] * inv, acc[e0 + 1] * inv, acc[e0 + 2] * inv, acc[e0 + 3] * inv);
  }
  if (cv == 0 && p.lse_out) p.lse_out[r] = wsum > 0.f ? Mt + logf(wsum) : -INFINITY;  // piece 0
}

// Split kernel variants: one wave per split, four waves per split (small grids), or the
// persistent walkers of decode_split_persist_kernel (large batches).
enum DecodeSplitMode { kSplitOneWave, kSplitFourWaves, kSplitPersistent };

template <int D, bool WS_BF16>
void launch_decode_d(const DecodeParams& p, DecodeSplitMode mode, dim3 grid, dim3 mgrid, hipStream_t stream) {
  if (mode == kSplitPersistent)
    hipLaunchKernelGGL((decode_split_persist_kernel<D, WS_BF16>), grid, dim3(64), 0, stream, p);
  else if (mode == kSplitFourWaves)
    hipLaunchKernelGGL((decode_split_kernel<D, 4, WS_BF16>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, 1, WS_BF16>), grid, dim3(64), 0, stream, p);
  // Fewer (request, head) rows than CUs (e.g. one request's heads): four workgroups per row, each
  // on a quarter of D. (With more rows, one workgroup per row measured faster.)
  if (mgrid.x < 256) {
    const dim3 g4(mgrid.x * 4);
    if (p.out_bf16)
      hipLaunchKernelGGL((decode_merge_kernel<D, 4, true, WS_BF16>), g4, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_merge_kernel<D, 4, false, WS_BF16>), g4, dim3(256), 0, stream, p);
  } else {
    if (p.out_bf16)
      hipLaunchKernelGGL((decode_merge_kernel<D, 1, true, WS_BF16>), mgrid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_merge_kernel<D, 1, false, WS_BF16>), mgrid, dim3(256), 0, stream, p);
  }
}

hipError_t launch_decode(const DecodeParams& p, int d_h, hipStream_t stream) {
  // grid sizes are checked on the host (api.cpp) to fit these 32-bit dimensions
  const int hblocks = (p.group + 15) / 16;
  dim3 grid(p.n_splits * p.batch, p.n_kv * hblocks);
  const dim3 mgrid(p.batch * p.n_h);
  DecodeSplitMode mode = kSplitOneWave;
  if (p.units_per_wave > 0) {
    // the host sets units_per_wave only where the unit count fits int and one round of waves
    const int units = p.batch * p.n_splits * p.n_kv * hblocks;
    grid = dim3((units + p.units_per_wave - 1) / p.units_per_wave);
    mode = kSplitPersistent;
  } else if ((int64_t)grid.x * grid.y < 2048) {
    mode = kSplitFourWaves;  // fewer workgroups than 8 per CU: four waves share each split
  }
  if (d_h == 64) {
    if (p.ws_bf16) launch_decode_d<64, true>(p, mode, grid, mgrid, stream);
    else launch_decode_d<64, false>(p, mode, grid, mgrid, stream);
  } else {
    if (p.ws_bf16) launch_decode_d<128, true>(p, mode, grid, mgrid, stream);
    else launch_decode_d<128, false>(p, mode, grid, mgrid, stream);
  }
  return hipGetLastError();
}

// ---- the allocation-free variant: the split workspace in a file-scope device array -------------
// For callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation). Each device the library runs on holds its own copy of
// this array until the process ends. Host code never uses the array's name as an address (on the
// host it is only a stand-in): the device address is looked up once per device with
// hipGetSymbolAddress and cached.
static __device__ __align__(256) unsigned char scratch[CP_DECODE_NOALLOC_MAX_BYTES];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // on the current device
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace cpk
