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
//    on QK^T of tile n+1. K/V tiles move HBM -> LDS with direct-to-LDS buffer loads (no VGPR
//    staging, no per-lane address math: one descriptor per tile bounds the run, rows past its
//    end arrive as zeros) into four stages of unpadded, XOR-swizzled rows; tile n+3's loads are
//    issued right after tile n's V reads, and the per-tile barrier waits only for tile n+2.
//  - The tile loop is unrolled over the four stages, so every LDS operand address is a per-lane
//    base plus an immediate offset (K tiles of all stages below 64 KB, V tiles above).
//  - One launch may carry several independent problems (e.g. the ranks of one ring step), each
//    with its own pointers and a range of the pooled segment tables.
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

template <int D, int WAVES>
struct Bf16Cfg {
  static constexpr int kWaves = WAVES;          // 32 query rows per wave
  static constexpr int kRows = 32 * WAVES;      // query rows per workgroup
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBN = 64;                // keys per LDS tile
  static constexpr int kRowBytes = D * 2;       // LDS rows are unpadded (see the swizzles)
  static constexpr int kChunks = D / 8;         // 16-byte chunks per key row
  static constexpr int kTileBytes = kBN * kRowBytes;  // one K or one V tile
  static constexpr int kStages = 4;
  // LDS holds the K tiles of all stages, then the V tiles of all stages: every operand read is a
  // per-lane base plus an immediate offset below 64 KB.
  static constexpr int kLdsBytes = 2 * kStages * kTileBytes;
  static constexpr int k_at(int st) { return st * kTileBytes; }
  static constexpr int v_at(int st) { return (kStages + st) * kTileBytes; }
  // A direct-to-LDS load writes 64 lanes x 16 bytes = 1 KB contiguously: a block of rows.
  static constexpr int kRowsPerBlock = 1024 / kRowBytes;
  static constexpr int kBlocksPerWave = kTileBytes / 1024 / kWaves;
  static constexpr int kDmaPerTile = 2 * kBlocksPerWave;  // K and V loads per wave per tile
  static constexpr int kKSteps = D / 16;        // MFMA k-steps over the head dimension
  static constexpr int kDBlocks = D / 32;       // 32-row blocks of O^T
  // Rows that share a 256-byte bank cycle (1 for D = 128, 2 for D = 64).
  static constexpr int kRowsPerBankCycle = 256 / kRowBytes;
  // Chunk c of key row r sits in slot c ^ swz(r). K rows are read 16 bytes at a time by 16
  // lanes on 16 consecutive rows: swz_k spreads those rows over the 16 bank quads. V rows are
  // read by the transposing loads, a half-wave covering 4 consecutive rows x 4 aligned chunks:
  // swz_v moves each of the 4 rows to its own group of 4 slots.
  static __device__ __host__ constexpr int swz_k(int r) { return (r / kRowsPerBankCycle) & (kChunks - 1); }
  static __device__ __host__ constexpr int swz_v(int r) {
    return ((r / kRowsPerBankCycle) & (4 / kRowsPerBankCycle - 1)) << 2;
  }
};

// The running max is only moved when a tile raises it by more than this many base-2 units, so
// probabilities stay <= 2^8 (exact in fp32 and within bf16's exponent range) and the O^T
// accumulators are rescaled a handful of times per row instead of once per tile. Any stale max
// gives the same result in exact arithmetic: LSE and O are computed against the max in use.
constexpr float kRescaleThreshold = 8.0f;

// s_waitcnt immediate for "vmcnt(0)" on gfx9-family targets (expcnt and lgkmcnt left at max).
constexpr int kWaitVmcnt0 = 0x0F70;

// Word 3 of a raw buffer descriptor on gfx9-family targets (32-bit data format, no swizzle).
constexpr int kBufferWord3 = 0x00020000;

// Hides x's value from the optimiser (no instruction). Device pass only: the constraint is an
// AMDGPU one, and a host pass that rejected it would drop the kernel's launch stub.
__device__ inline void opaque(uint32_t& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
}

// One direct-to-LDS load of 16 bytes per lane through buffer descriptor r: lane l's bytes go to
// lds + 16 l; a lane whose offset lies outside the descriptor's range writes zeros. (The body is
// device-pass only: a host pass that saw the builtin would drop the kernel's launch stub.)
__device__ inline void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           (int)voff, 0, 0, 0);
#endif
}

template <int N>
struct StageIdx {
  static constexpr int value = N;
};

__device__ inline bf16x8 lds_read_b128(const unsigned char* base, int byte_off) {
  return *reinterpret_cast<const bf16x8*>(base + byte_off);
}

__device__ inline i16x4 lds_read_tr(const unsigned char* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + byte_off));
}

// Position of a K/V tile: run j of the KV shard (j == the problem's kv_hi means "no tile"), key offset kt
// inside the run, and the run's fields, carried along so that scalar loads of the run table
// (whose waits would also drain every outstanding LDS read) only happen at run boundaries.
struct TilePos {
  int j;
  int kt;
  int vis;  // keys of the run visible to the workgroup's last query
  int loc, pos, len;
  int n_full;    // keys of the run visible to every row of the workgroup
  int64_t off;   // byte offset of the tile's first key row in the shard
};

template <int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void attn_bf16_kernel(const AttnParams p) {
  using C = Bf16Cfg<D, WAVES>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column of this lane in the 32x32 blocks
  const int half = lane >> 5;  // which 8-wide k slice (and which 4-row group of the output)
  const int g = blockIdx.y;    // KV head

  int seg, tile;
  locate_tile(p, blockIdx.x, seg, tile);
  const Seg qs = p.qs[seg];
  const int pr = p.q_prob[seg];  // problem of this tile; its KV runs are [kv_lo, kv_hi)
  const int kv_lo = p.kv_lo[pr], kv_hi = p.kv_hi[pr];
  const int rows = qs.len * p.group;
  const int tile_row0 = tile * C::kRows;
  const int tile_row_last = min(tile_row0 + C::kRows, rows) - 1;
  // positions of the first and last query token of the workgroup (classifies whole tiles)
  const int qpos_lo = qs.pos + tile_row0 / p.group;
  const int qpos_hi = qs.pos + tile_row_last / p.group;

  const __bf16* __restrict__ Q = static_cast<const __bf16*>(p.q[pr]);
  const __bf16* __restrict__ K = static_cast<const __bf16*>(p.k[pr]);
  const __bf16* __restrict__ V = static_cast<const __bf16*>(p.v[pr]);

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
  const uint32_t row_bytes = (uint32_t)p.n_kv * D * 2;
  auto first_run_from = [&](int j) -> TilePos {
    for (; j < kv_hi; ++j) {
      const Seg ks = p.ks[j];
      if (ks.seq != qs.seq) continue;
      const int vis = visible_prefix(ks, qpos_hi, p.causal);
      if (vis > 0) {
        const int n_full = p.causal ? max(0, min(ks.len, qpos_lo - ks.pos + 1)) : ks.len;
        return TilePos{j, 0, vis, ks.loc, ks.pos, ks.len, n_full, (int64_t)ks.loc * row_bytes};
      }
    }
    return TilePos{kv_hi, 0, 0, 0, 0, 1, 1, 0};
  };
  auto next_tile = [&](TilePos t) -> TilePos {
    if (t.j >= kv_hi) return t;
    if (t.kt + C::kBN < t.vis) {
      t.kt += C::kBN;
      t.off += (int64_t)C::kBN * row_bytes;
      return t;
    }
    return first_run_from(t.j + 1);
  };

  // K/V staging: HBM -> LDS with direct-to-LDS loads (no VGPRs in between). Wave w fills blocks
  // w * kBlocksPerWave + i of a tile; in a block, lane l fills row l / kChunks, slot l % kChunks,
  // which holds chunk slot ^ swz(row). A lane's offset (its row and chunk) is fixed; the tile's
  // position is in the buffer descriptor.
  const unsigned char* Kb = reinterpret_cast<const unsigned char*>(K + (int64_t)g * D);
  const unsigned char* Vb = reinterpret_cast<const unsigned char*>(V + (int64_t)g * D);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t dma_k_off[C::kBlocksPerWave], dma_v_off[C::kBlocksPerWave];
#pragma unroll
  for (int i = 0; i < C::kBlocksPerWave; ++i) {
    const int row = (wave * C::kBlocksPerWave + i) * C::kRowsPerBlock + lane / C::kChunks;
    const int slot = lane % C::kChunks;
    dma_k_off[i] = row * row_bytes + (slot ^ C::swz_k(row)) * 16;
    dma_v_off[i] = row * row_bytes + (slot ^ C::swz_v(row)) * 16;
  }
  // One buffer descriptor per tile and operand covers the tile's rows inside the run; rows past
  // the run's end fall outside it and arrive in LDS as zeros (no clamp, no per-lane address math).
#define CP_TILE_DMA(T, STAGE)                                                                 \
  {                                                                                           \
    const int64_t first = (T).off;                                                            \
    const int nrec = min((T).len - (T).kt, C::kBN) * (int)row_bytes;                          \
    const __amdgpu_buffer_rsrc_t kr =                                                         \
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kb + first), 0, nrec, kBufferWord3);        \
    const __amdgpu_buffer_rsrc_t vr =                                                         \
        __builtin_amdgcn_make_buffer_rsrc((void*)(Vb + first), 0, nrec, kBufferWord3);        \
    unsigned char* kt_s = smem + C::k_at(STAGE);                                              \
    unsigned char* vt_s = smem + C::v_at(STAGE);                                              \
    _Pragma("unroll") for (int i = 0; i < C::kBlocksPerWave; ++i) {                           \
      const int blk = (wave_u * C::kBlocksPerWave + i) * 1024;                                \
      buffer_to_lds16(kr, kt_s + blk, dma_k_off[i]);                                          \
      buffer_to_lds16(vr, vt_s + blk, dma_v_off[i]);                                          \
    }                                                                                         \
  }

  // s_waitcnt immediate for vmcnt(kDmaPerTile) (at most 15, the low vmcnt field)
  static_assert(C::kDmaPerTile < 16, "vmcnt immediate");
  constexpr int kWaitVmcntDmaLgkm0 = 0x0070 | C::kDmaPerTile;  // also lgkmcnt(0)

  // S^T = K Q^T of the tile in stage `st`: two 32-key halves against this wave's 32 queries.
  // K operand addresses: key rows col and 32 + col (same swizzle), chunk half * D/16 + k.
  uint32_t k_off[C::kKSteps];
#pragma unroll
  for (int k = 0; k < C::kKSteps; ++k)
    k_off[k] = col * C::kRowBytes + 16 * ((half * (D / 16) + k) ^ C::swz_k(col));
  // (hide the bases' known bits: stage offsets are then added and folded into the instruction's
  // offset field instead of being OR-ed in by VALU ops)
#pragma unroll
  for (int k = 0; k < C::kKSteps; ++k) opaque(k_off[k]);
  auto qk = [&](int st, f32x16 (&s)[2]) {
    const unsigned char* Kt = smem + C::k_at(st);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
    for (int k = 0; k < C::kKSteps; ++k) {
      const bf16x8 a0 = lds_read_b128(Kt, k_off[k]);
      const bf16x8 a1 = lds_read_b128(Kt, k_off[k] + 32 * C::kRowBytes);
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
  // key row 16t + tr_key (+8) has the swizzle of row tr_key; columns db*32 + tr_dcol .. +3
  uint32_t v_off[C::kDBlocks];
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db)
    v_off[db] = tr_key * C::kRowBytes + 16 * (((db * 32 + tr_dcol) / 8) ^ C::swz_v(tr_key)) +
                8 * (j16 & 1) + C::v_at(0);
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db) opaque(v_off[db]);

  // ---- prologue: tiles 0 and 1 into stages 0 and 1, tiles 2 and 3 in flight, QK^T of tile 0
  TilePos cur = first_run_from(kv_lo);
  TilePos nxt = next_tile(cur);
  TilePos nn = next_tile(nxt);
  TilePos n3 = next_tile(nn);
  // Tile loads are issued unconditionally (a position past the last tile reads key row 0 of the
  // shard, and zeros, into a free stage).
  // One tile: s holds its scores S^T (from the previous step), s_nx receives the next tile's.
  // The tile's stage is a compile-time constant (the loop is unrolled over the four stages), so
  // every LDS address is a per-lane base plus an immediate offset.
  auto step = [&](auto stage, f32x16 (&s)[2], f32x16 (&s_nx)[2]) {
    constexpr int st_cur = decltype(stage)::value;  // tiles nxt, nn, n3 are in the next stages
    constexpr int st_nxt = (st_cur + 1) & 3;

    // ---- mask (only tiles not fully visible to every row of the workgroup) ----
    if (cur.kt + C::kBN > cur.n_full) {
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
    const unsigned char* Vt = smem + (C::v_at(st_cur) - C::v_at(0));  // v_off includes v_at(0)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db) {
        const uint32_t off = v_off[db] + 16 * t * C::kRowBytes;
        const i16x4 lo = lds_read_tr(Vt, off);
        const i16x4 hi = lds_read_tr(Vt, off + 8 * C::kRowBytes);
        const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 va = __builtin_bit_cast(bf16x8, both);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[t], oacc[db], 0, 0, 0);
      }
    }

    // Tile n3: HBM -> LDS into the stage of tile cur-1 (read before the last barrier). Issued
    // after this tile's V reads, so the next tile's V reads are the first LDS reads that have
    // to wait for it; before the barrier only tile nn's loads (issued one step earlier) must
    // have landed.
    CP_TILE_DMA(n3, (st_cur + 3) & 3);
    // This wave's LDS reads are done and tile nn has landed; then the workgroup barrier. (The
    // barrier is issued as a bare instruction: the compiler's own barrier would also wait for
    // tile n3's loads, which have two more tiles of time.)
    __builtin_amdgcn_s_waitcnt(kWaitVmcntDmaLgkm0);
    asm volatile("s_barrier" ::: "memory");
    cur = nxt;
    nxt = nn;
    nn = n3;
    n3 = next_tile(n3);
  };
  // Two steps per trip with the score buffers swapping roles (no register copies). A workgroup
  // without visible keys skips the loop (uniform branch).
  f32x16 sa[2], sb[2];
  int n_tiles = 0;  // tiles of this workgroup: ceil(visible / kBN) over its runs
  for (int j = kv_lo; j < kv_hi; ++j) {
    const Seg ks = p.ks[j];
    if (ks.seq == qs.seq) n_tiles += (visible_prefix(ks, qpos_hi, p.causal) + C::kBN - 1) / C::kBN;
  }
  if (n_tiles > 0) {
    CP_TILE_DMA(cur, 0);
    CP_TILE_DMA(nxt, 1);
    CP_TILE_DMA(nn, 2);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    qk(0, sa);
    int left = n_tiles;
    for (;;) {
      step(StageIdx<0>{}, sa, sb);
      if (--left == 0) break;
      step(StageIdx<1>{}, sb, sa);
      if (--left == 0) break;
      step(StageIdx<2>{}, sa, sb);
      if (--left == 0) break;
      step(StageIdx<3>{}, sb, sa);
      if (--left == 0) break;
    }
    // The last step issued loads of a tile past the end (unused). Retire them here rather than
    // leave them to the end of the program, so no LDS write is pending once the waves finish.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
#undef CP_TILE_DMA

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2, optional merge into the running result
  const float lt = l + __shfl_xor(l, 32);
  if (!live) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_new = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  float wp = 0.f, wn = 1.f, lse_out = lse_new;
  float* orow = p.o[pr] + qrow * D;
  float4 prev[C::kDBlocks * 4];
  if (p.accumulate) {
    running_merge_weights(p.lse[pr][qrow], lse_new, wp, wn, lse_out);
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
  if (half == 0) p.lse[pr][qrow] = lse_out;
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
