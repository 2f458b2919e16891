// attn_bf16.hip -- partial attention of a Q shard over one KV shard, bf16 inputs, gfx950 MFMA.
//
// What it computes: for every query row (token, head) of the Q shard, exact attention over the
// keys of the KV shard it may see, as a partial result O = sum_j p_j V_j / sum_j p_j and
// LSE = ln sum_j exp(s_j) with s_j = scale * q.k_j ([CPMTI §3 "核心公式": each ring step is the
// partial attention of the local Q with the KV shard held; [CPEP §5.1]: per-token softmax
// attention, causal mask keeps key positions <= query position; [CPEP §8.2]: consecutive query
// heads share one KV head).
//
// How (MI355X-first design; the pages name FlashAttention-3 on H100 as prior art only):
//  - GQA packing: the G = N_H / N_KV query heads of a KV group are flattened with the tokens into
//    one row space (row = token * G + head). A workgroup of 8 waves owns 256 rows; every K/V tile
//    it stages in LDS serves all of them (for G = 16 that is 16 tokens x 16 heads).
//  - Orientation S^T = K Q^T: v_mfma_f32_32x32x16_bf16 with K as the A operand (rows = keys)
//    and Q^T as the B operand (columns = queries). In the 32x32 accumulator a lane holds 16 keys
//    of one query, so a query's row max needs only one exchange between the two half-waves.
//    Each wave owns one 32-query block whose Q^T operand stays in registers.
//  - P.V as O^T = V^T P^T: the probabilities, rounded to bf16, are already laid out as the
//    B operand; V^T comes straight from the row-major V tile with ds_read_b64_tr_b16, whose
//    16-lane transpose turns four key rows into per-lane key vectors.
//  - Software pipeline: while the VALUs run the softmax of tile n, the MFMA pipe already works
//    on QK^T of tile n+1; K/V tiles live in three LDS stages (tile n being consumed, tile n+1
//    ready for QK^T, tile n+2 arriving from registers loaded during the previous tile).
//  - Online softmax in base 2 with scale*log2(e) folded into one FMA; the running max only moves
//    when a tile raises it by more than 2^8, so the O^T accumulators are rarely rescaled; fp32
//    accumulators, LSE returned in natural log.
//  - Masks are computed from segment positions, never stored. Tiles entirely visible to every
//    row of the workgroup skip the mask; runs of other sequences and keys past the causal
//    frontier are never loaded.
//
// Pages cited: [CPEP] "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두
// 축"; [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (paper review).
#include "device_common.h"

namespace cpk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
// Native vector for 16-byte staging (arrays of HIP's uint4 struct are not promoted to registers).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int D, int WAVES>
struct Bf16Cfg {
  static constexpr int kWaves = WAVES;          // 32 query rows per wave
  static constexpr int kRows = 32 * WAVES;      // query rows per workgroup
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBN = 64;                // keys per LDS tile
  // Padded LDS rows. K rows are read 16 bytes at a time by 16 lanes on 16 different rows: a
  // stride of 4 (mod 64) dwords puts those rows on disjoint bank quads. V rows are read by the
  // transposing loads, 4 lanes x 8 bytes on each of 4 rows per half-wave: a stride of 16
  // (mod 64) dwords puts those four 64-byte runs on disjoint banks.
  static constexpr int kStrideK = D * 2 + 16;
  static constexpr int kStrideV = D * 2 + 64;
  static constexpr int kStageBytes = kBN * (kStrideK + kStrideV);
  static constexpr int kStages = 3;
  static constexpr int kChunks = D / 8;         // 16-byte chunks per key row
  static constexpr int kRowsPerPass = kThreads / kChunks;
  static constexpr int kPasses = kBN / kRowsPerPass;
  static constexpr int kKSteps = D / 16;        // MFMA k-steps over the head dimension
  static constexpr int kDBlocks = D / 32;       // 32-row blocks of O^T
};

// The running max is only moved when a tile raises it by more than this many base-2 units, so
// probabilities stay <= 2^8 (exact in fp32 and within bf16's exponent range) and the O^T
// accumulators are rescaled a handful of times per row instead of once per tile. Any stale max
// gives the same result in exact arithmetic: LSE and O are computed against the max in use.
constexpr float kRescaleThreshold = 8.0f;

// s_waitcnt immediate for "vmcnt(0)" on gfx9-family targets (expcnt and lgkmcnt left at max).
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ inline bf16x8 lds_read_b128(const unsigned char* base, int byte_off) {
  return *reinterpret_cast<const bf16x8*>(base + byte_off);
}

__device__ inline i16x4 lds_read_tr(const unsigned char* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + byte_off));
}

// Position of a K/V tile: run j of the KV shard (j == n_kv_segs means "no tile"), key offset kt
// inside the run, and the run's fields, carried along so that scalar loads of the run table
// (whose waits would also drain every outstanding LDS read) only happen at run boundaries.
struct TilePos {
  int j;
  int kt;
  int vis;  // keys of the run visible to the workgroup's last query
  int loc, pos, len;
};

template <int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(const AttnParams p) {
  using C = Bf16Cfg<D, WAVES>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::kStages * C::kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column of this lane in the 32x32 blocks
  const int half = lane >> 5;  // which 8-wide k slice (and which 4-row group of the output)
  const int g = blockIdx.y;    // KV head

  int seg, tile;
  locate_tile(p, blockIdx.x, seg, tile);
  const Seg qs = p.qs[seg];
  const int rows = qs.len * p.group;
  const int tile_row0 = tile * C::kRows;
  const int tile_row_last = min(tile_row0 + C::kRows, rows) - 1;
  // positions of the first and last query token of the workgroup (classifies whole tiles)
  const int qpos_lo = qs.pos + tile_row0 / p.group;
  const int qpos_hi = qs.pos + tile_row_last / p.group;

  const __bf16* __restrict__ Q = static_cast<const __bf16*>(p.q);
  const __bf16* __restrict__ K = static_cast<const __bf16*>(p.k);
  const __bf16* __restrict__ V = static_cast<const __bf16*>(p.v);

  // ---- this lane's query row and its Q^T operand ------------------------------------------
  const int r = tile_row0 + wave * 32 + col;
  const bool live = r < rows;
  const int rc = live ? r : rows - 1;
  const int qtok = rc / p.group;
  const int qpos = qs.pos + qtok;
  const int64_t qrow = (int64_t)(qs.loc + qtok) * p.n_h + g * p.group + rc % p.group;
  bf16x8 qreg[C::kKSteps];
  {
    const __bf16* qp = Q + qrow * D + half * (D / 2);
#pragma unroll
    for (int s = 0; s < C::kKSteps; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + s * 8);
  }
  // Retire the Q loads here: otherwise the wait analysis keeps them pending at the tile loop's
  // header and makes the QK^T of every tile also wait for the next tile's prefetch.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // ---- KV tiles: runs of the same sequence, the prefix visible to the last query ----------
  auto first_run_from = [&](int j) -> TilePos {
    for (; j < p.n_kv_segs; ++j) {
      const Seg ks = p.ks[j];
      if (ks.seq != qs.seq) continue;
      const int vis = visible_prefix(ks, qpos_hi, p.causal);
      if (vis > 0) return TilePos{j, 0, vis, ks.loc, ks.pos, ks.len};
    }
    return TilePos{p.n_kv_segs, 0, 0, 0, 0, 1};
  };
  auto next_tile = [&](TilePos t) -> TilePos {
    if (t.j >= p.n_kv_segs) return t;
    if (t.kt + C::kBN < t.vis) {
      t.kt += C::kBN;
      return t;
    }
    return first_run_from(t.j + 1);
  };

  // K/V staging: each thread moves 16-byte chunks; a wave covers whole key rows.
  const int ld_chunk = tid % C::kChunks;
  const int ld_row0 = tid / C::kChunks;
  // Addresses: the tile's first key row is a uniform 64-bit base (scalar arithmetic); a lane
  // adds a 32-bit offset (its row inside the tile, clamped to the run's last key, and its chunk).
  const uint32_t row_bytes = (uint32_t)p.n_kv * D * 2;
  const unsigned char* Kb = reinterpret_cast<const unsigned char*>(K + (int64_t)g * D);
  const unsigned char* Vb = reinterpret_cast<const unsigned char*>(V + (int64_t)g * D);
  uint32_t row_off[C::kPasses];  // byte offset of this lane's row in pass ps of a tile
#pragma unroll
  for (int ps = 0; ps < C::kPasses; ++ps) row_off[ps] = (ld_row0 + ps * C::kRowsPerPass) * row_bytes;
  // Two tiles on their way from HBM to LDS: a tile is loaded two steps before it is stored,
  // so the load latency hides behind two tiles of work.
  u32x4 kst0[C::kPasses], vst0[C::kPasses], kst1[C::kPasses], vst1[C::kPasses];
#define CP_TILE_LOAD(T, kst, vst)                                                         \
  {                                                                                       \
    const int64_t first = (int64_t)((T).loc + (T).kt) * row_bytes;                        \
    const uint32_t last_off = (uint32_t)min((T).len - 1 - (T).kt, C::kBN - 1) * row_bytes; \
    _Pragma("unroll") for (int ps = 0; ps < C::kPasses; ++ps) {                           \
      const uint32_t o = min(row_off[ps], last_off) + ld_chunk * 16;                      \
      kst[ps] = *reinterpret_cast<const u32x4*>(Kb + first + o);                          \
      vst[ps] = *reinterpret_cast<const u32x4*>(Vb + first + o);                          \
    }                                                                                     \
  }
#define CP_TILE_STORE(STAGE, kst, vst)                                            \
  {                                                                               \
    unsigned char* kt_s = smem + (STAGE) * C::kStageBytes;                        \
    unsigned char* vt_s = kt_s + C::kBN * C::kStrideK;                            \
    _Pragma("unroll") for (int ps = 0; ps < C::kPasses; ++ps) {                   \
      const int rr = ld_row0 + ps * C::kRowsPerPass;                              \
      *reinterpret_cast<u32x4*>(kt_s + rr * C::kStrideK + ld_chunk * 16) = kst[ps]; \
      *reinterpret_cast<u32x4*>(vt_s + rr * C::kStrideV + ld_chunk * 16) = vst[ps]; \
    }                                                                             \
  }

  // S^T = K Q^T of the tile in stage `st`: two 32-key halves against this wave's 32 queries.
  auto qk = [&](int st, f32x16 (&s)[2]) {
    const unsigned char* Kt = smem + st * C::kStageBytes;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
    for (int k = 0; k < C::kKSteps; ++k) {
      const int coff = (half * (D / 2) + k * 8) * 2;
      const bf16x8 a0 = lds_read_b128(Kt, col * C::kStrideK + coff);
      const bf16x8 a1 = lds_read_b128(Kt, (32 + col) * C::kStrideK + coff);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[k], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[k], s[1], 0, 0, 0);
    }
  };

  float m = -INFINITY;  // max in use, base-2 scaled units (same in both half-waves)
  float l = 0.f;        // running sum over this half-wave's keys
  f32x16 oacc[C::kDBlocks];
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;

  // V^T operand addressing for ds_read_b64_tr_b16: each 16-lane group covers 16 d-rows
  const int grp = lane >> 4;          // 0..3
  const int dsub = grp & 1;           // which 16 of the 32 d-rows
  const int j16 = lane & 15;
  const int tr_key = 4 * half + (j16 >> 2);
  const int tr_dcol = dsub * 16 + 4 * (j16 & 3);

  // ---- prologue: tiles 0 and 1 into stages 0 and 1, tiles 2 and 3 in flight, QK^T of tile 0
  TilePos cur = first_run_from(0);
  TilePos nxt = next_tile(cur);
  TilePos nn = next_tile(nxt);
  TilePos n3 = next_tile(nn);
  // Loads and stores are issued unconditionally once there is a tile (a position past the last
  // tile reads key row 0 of the shard into a free stage), so the number of loads in flight is
  // the same on every path and each store waits only for its own tile.
  int st_cur = 0;  // stage of tile cur; tile nxt is in st_cur+1, tile nn goes to st_cur+2 (mod 3)
  // One tile: s holds its scores S^T (from the previous step), s_nx receives the next tile's;
  // (kst, vst) hold tile nn and receive tile nn+2.
  auto step = [&](f32x16 (&s)[2], f32x16 (&s_nx)[2], u32x4 (&kst)[C::kPasses],
                  u32x4 (&vst)[C::kPasses]) {
    const int st_nxt = st_cur == 2 ? 0 : st_cur + 1;
    const int st_nn = st_nxt == 2 ? 0 : st_nxt + 1;
    // tile nn: registers -> LDS (its stage was last read by tile cur-1, before the last barrier)
    const TilePos n4 = next_tile(n3);
    CP_TILE_STORE(st_nn, kst, vst);
    CP_TILE_LOAD(n4, kst, vst);

    // ---- mask (only tiles not fully visible to every row of the workgroup) ----
    const int n_full = p.causal ? max(0, min(cur.len, qpos_lo - cur.pos + 1)) : cur.len;
    if (cur.kt + C::kBN > n_full) {
      // key ko of the run is visible iff ko < len and (not causal or pos + ko <= qpos):
      // ko < lim with lim = min(len, qpos - pos + 1) (or len without the causal mask)
      const int lim = p.causal ? min(cur.len, qpos - cur.pos + 1) : cur.len;
      const int base = cur.kt + 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ko = base + kb * 32 + 8 * (v >> 2) + (v & 3);
          s[kb][v] = ko < lim ? s[kb][v] : -INFINITY;
        }
    }

    // ---- online softmax (base 2, lazily moved max) ----
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = max_xor32(mx) * p.scale_log2;
    if (__any(mx > m + kRescaleThreshold)) {
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // m = -inf -> 0; mnew = m -> 1
      if (mnew != -INFINITY) {
        l *= alpha;
#pragma unroll
        for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
        m = mnew;
      }
    }
    // QK^T of the next tile goes to the MFMA pipe while this tile's exponentials run on the
    // VALUs (same basic block, so the two interleave). Issued unconditionally: after the last
    // tile the stage holds stale keys and the result is never used.
    qk(st_nxt, s_nx);

    const float msafe = m == -INFINITY ? 0.f : m;
    bf16x8 pb[4];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][v], p.scale_log2, -msafe));
        rs += e;
        // P^T operand of k-step t: keys 16t + 8(e/4) + 4*half + e%4 == entries 8(t%2) + e
        pb[2 * kb + (v >> 3)][v & 7] = (__bf16)e;
      }
    l += rs;

    // ---- O^T += V^T P^T ----
    const unsigned char* Vt = smem + st_cur * C::kStageBytes + C::kBN * C::kStrideK;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db) {
        const int off = (16 * t + tr_key) * C::kStrideV + (db * 32 + tr_dcol) * 2;
        const i16x4 lo = lds_read_tr(Vt, off);
        const i16x4 hi = lds_read_tr(Vt, off + 8 * C::kStrideV);
        const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 va = __builtin_bit_cast(bf16x8, both);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[t], oacc[db], 0, 0, 0);
      }
    }

    // every wave is done with stage st_cur, and tile nn is visible in stage st_nn
    __syncthreads();
    cur = nxt;
    nxt = nn;
    nn = n3;
    n3 = n4;
    st_cur = st_nxt;
  };
  // Two steps per trip with the score buffers and the staging registers swapping roles (no
  // register copies). A workgroup without visible keys skips the loop (uniform branch).
  f32x16 sa[2], sb[2];
  int n_tiles = 0;  // tiles of this workgroup: ceil(visible / kBN) over its runs
  for (int j = 0; j < p.n_kv_segs; ++j) {
    const Seg ks = p.ks[j];
    if (ks.seq == qs.seq) n_tiles += (visible_prefix(ks, qpos_hi, p.causal) + C::kBN - 1) / C::kBN;
  }
  if (n_tiles > 0) {
    CP_TILE_LOAD(cur, kst0, vst0);
    CP_TILE_STORE(0, kst0, vst0);
    CP_TILE_LOAD(nxt, kst1, vst1);
    CP_TILE_STORE(1, kst1, vst1);
    CP_TILE_LOAD(nn, kst0, vst0);
    CP_TILE_LOAD(n3, kst1, vst1);
    __syncthreads();
    qk(0, sa);
    // a counted loop without exits in its body keeps the two staging sets' loads in a fixed
    // order, so each store waits only for its own set
    for (int it = 0; it + 1 < n_tiles; it += 2) {
      step(sa, sb, kst0, vst0);
      step(sb, sa, kst1, vst1);
    }
    if (n_tiles & 1) step(sa, sb, kst0, vst0);
  }
#undef CP_TILE_LOAD
#undef CP_TILE_STORE

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2, optional merge into the running result
  const float lt = l + __shfl_xor(l, 32);
  if (!live) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_new = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  float wp = 0.f, wn = 1.f, lse_out = lse_new;
  float* orow = p.o + qrow * D;
  float4 prev[C::kDBlocks * 4];
  if (p.accumulate) {
    running_merge_weights(p.lse[qrow], lse_new, wp, wn, lse_out);
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq)
        prev[db * 4 + vq] = *reinterpret_cast<const float4*>(orow + db * 32 + 8 * vq + 4 * half);
  } else {
#pragma unroll
    for (int i = 0; i < C::kDBlocks * 4; ++i) prev[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float sc = wn * inv;
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      const float4 pv = prev[db * 4 + vq];
      float4 o4;
      o4.x = fmaf(wp, pv.x, oacc[db][4 * vq] * sc);
      o4.y = fmaf(wp, pv.y, oacc[db][4 * vq + 1] * sc);
      o4.z = fmaf(wp, pv.z, oacc[db][4 * vq + 2] * sc);
      o4.w = fmaf(wp, pv.w, oacc[db][4 * vq + 3] * sc);
      *reinterpret_cast<float4*>(orow + db * 32 + 8 * vq + 4 * half) = o4;
    }
  if (half == 0) p.lse[qrow] = lse_out;
}

hipError_t launch_attn_bf16(const AttnParams& p, int d_h, hipStream_t stream) {
  const dim3 grid(p.total_tiles, p.n_kv);
  constexpr int W = kTileRowsBf16 / 32;
  const dim3 block(W * 64);
  if (d_h == 64)
    hipLaunchKernelGGL((attn_bf16_kernel<64, W>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<128, W>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace cpk
