// attn_bwd.hip -- backward of one ring step's partial attention, bf16 inputs, gfx950 MFMA.
//
// What it computes ([CPEP §6]: in context parallelism the backward returns every rank's K/V
// gradient contributions to the owners of those K/V chunks, a reduce-scatter, i.e. a sum per
// chunk): for the Q shard's rows and the KV shard's keys each row may see, with the row's FINAL
// output O and log-sum-exp LSE (over every shard) and the output gradient dO,
//   P  = exp(scale * q.k - LSE),   dP = dO.v,   delta = dO.O (per row),   dS = P (dP - delta)
//   dQ += scale * dS K,   dK += scale * dS^T Q,   dV += P^T dO
// accumulated into the caller's fp32 buffers. Summed over the ring steps (dQ) and over the ranks
// that visit a KV shard (dK, dV) this is the exact gradient of the whole attention.
//
// One launch per ring step (two when the dK/dV work is split), nothing needing atomics. Its first
// workgroups are dK/dV workgroups, the rest dQ workgroups (same shape: 8 waves, one per CU):
//  - dQ: a workgroup owns 256 query rows (GQA rows = token * G + head, as in the forward) and
//    walks the KV tiles they see. S^T = K Q^T and dP^T = V dO^T run on v_mfma_f32_32x32x16_bf16
//    with K and V rows from LDS and Q^T, dO^T in registers, so each lane holds 16 keys of one row:
//    P, dS and the row's LSE and delta are per-lane values. dS^T, rounded to bf16, is then
//    directly the B operand of dQ^T += K^T dS^T, whose K^T operand comes from the same K tile
//    through the transposing ds_read_b64_tr_b16.
//  - dK/dV: a workgroup owns 128 keys; waves 0-3 accumulate dV of 32 keys each and waves 4-7 dK
//    of the same keys (K, or V for dK, kept in registers as B operands), walking the blocks of 64
//    query rows that see them. A dV wave forms S = Q K^T and P and hands P (fp16) to its dK wave
//    through LDS; the dK wave forms dP = dO V^T and then dS. Each lane holds 16 rows
//    of one key, the A operand layout of dV += P^T dO and dK += dS^T Q; dO and Q come from LDS
//    through the transposing read. With a workspace, the query blocks of a key tile may be
//    divided into parts worked on by separate workgroups, whose sums bwd_dkdv_reduce_kernel
//    then adds in part order.
// Both stage their shared operands through LDS buffers (the next tile or block prefetched into
// registers and stored into a buffer no wave reads any more: two buffers for dQ, three for dK/dV,
// whose workgroups pass one barrier per 64-row block), and swizzle 16-byte chunks so that row
// reads and transposing reads of one tile are conflict-free.
//
// Pages cited: [CPEP] "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두
// 축"; [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (paper review).
#include <algorithm>

#include "attn_bwd.h"
#include "device_common.h"

namespace cpk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// s_waitcnt immediate for "vmcnt(0)" on gfx9-family targets (expcnt and lgkmcnt left at max).
constexpr int kBwdWaitVmcnt0 = 0x0F70;

// An LDS tile of rows of D bf16 values, row-major without padding; the 16-byte chunk c of row r
// sits in slot c ^ sw(r). Row reads (16 lanes, 16 consecutive rows, one chunk) and transposing
// reads (a half-wave: 4 consecutive rows x 4 consecutive chunks) then touch 16 distinct slots.
template <int D>
struct BwdTile {
  static constexpr int kChunks = D / 8;
  static constexpr int kRowBytes = D * 2;
  static __device__ constexpr int sw(int r) { return (((r & 3) << 2) | ((r >> 2) & 3)) & (kChunks - 1); }
  // byte offset of element (r, c8 * 8 + e) for e in [0, 8): chunk c8, byte 2e
  static __device__ int off(int r, int col) {
    return r * kRowBytes + (((col >> 3) ^ sw(r)) << 4) + ((col & 7) << 1);
  }
};

__device__ inline bf16x8 lds_b128(const unsigned char* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

// Transposing read of rows r0 + {0..3} + 4 * (lane / 32) and the same 8 rows further, at column
// col0 + (lane % 32) of a BwdTile: lane l gets 8 values, entry e = row r0 + 8 (e / 4) +
// 4 (l / 32) + e % 4. That is the k order of the 32x32x16 MFMA operand built from a register
// tile whose k index runs over rows 8 (v / 4) + 4 (l / 32) + v % 4 (the accumulator layout).
template <int D>
__device__ inline bf16x8 lds_tr8(const unsigned char* base, int r0, int col0, int lane) {
  using T = BwdTile<D>;
  const int r = r0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int c = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + T::off(r, c)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + T::off(r + 8, c)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Division by the GQA group size, fixed for a launch, by a multiply and a shift (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994): for 0 <= n < 2^31,
// n / d = (mulhi(m, n) + n) >> l with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (the
// sum fits in 32 bits). The row -> (token, head) split of every loaded row then costs a few
// instructions instead of a full integer division.
struct DivBy {
  uint32_t m;
  int l;
  __device__ explicit DivBy(int d) {
    l = d <= 1 ? 0 : 32 - __clz(d - 1);
    m = (uint32_t)(((((uint64_t)1 << l) - (uint64_t)d) << 32) / (uint64_t)d) + 1u;
  }
  __device__ int operator()(int n) const {
    return (int)((__umulhi(m, (uint32_t)n) + (uint32_t)n) >> l);
  }
};

// Workgroup tile -> (run, tile index in the run) over a table ordered by `order`, prefix sums in
// `prefix`; first_tile_last: the first workgroup of a run takes its last tile.
__device__ inline void bwd_locate(const int32_t* prefix, const int8_t* order, int n_segs, int block,
                                  bool first_tile_last, int& seg, int& tile) {
  int slot = 0;
  while (slot + 1 < n_segs && prefix[slot + 1] <= block) ++slot;
  seg = order[slot];
  const int n = prefix[slot + 1] - prefix[slot];
  tile = first_tile_last ? n - 1 - (block - prefix[slot]) : block - prefix[slot];
}

// ------------------------------------------------------------------------------------------ dQ
constexpr int kDqThreads = 2 * kBwdQRows;  // a wave per 32 query rows
constexpr int kDqKeys = 64;                // keys per K/V tile
// LDS of a dQ workgroup: two buffers of a K and a V tile; tile n is worked on in buffer n % 2
// while tile n + 1 is staged into the other
template <int D>
constexpr int dq_lds_bytes() { return 4 * kDqKeys * BwdTile<D>::kRowBytes; }

// The dQ workgroup `bx` of the plan (heaviest row tile first).
template <int D>
__device__ __forceinline__ void bwd_dq_tile(const BwdParams& p, int bx, unsigned char* smem) {
  using T = BwdTile<D>;
  constexpr int kBN = kDqKeys;
  constexpr int kTileBytes = kBN * T::kRowBytes;
  constexpr int kLoads = kBN * T::kChunks / kDqThreads;  // 16-byte loads per thread per operand

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int g = blockIdx.y;
  int seg, tile;
  bwd_locate(p.q_prefix, p.q_order, p.n_q_segs, bx, true, seg, tile);
  const Seg qs = p.qs[seg];
  const int rows = qs.len * p.group;
  const int row0 = tile * kBwdQRows;
  const int row_last = min(row0 + kBwdQRows, rows) - 1;
  const int qpos_lo = qs.pos + row0 / p.group;
  const int qpos_hi = qs.pos + row_last / p.group;

  const int r = row0 + wave * 32 + col;
  const bool live = r < rows;
  const int rc = live ? r : rows - 1;
  const int qtok = rc / p.group;
  const int qpos = qs.pos + qtok;
  const int64_t qrow = (int64_t)(qs.loc + qtok) * p.n_h + g * p.group + rc % p.group;
  // Q^T and dO^T operands: k-step s covers d = 8 (half * D/16 + s) + e (the K rows are read with
  // the same order of d, so every MFMA's reduction covers each d once)
  bf16x8 qreg[D / 16], doreg[D / 16];
  {
    const __bf16* qp = static_cast<const __bf16*>(p.q) + qrow * D + half * (D / 2);
    const __bf16* gp = static_cast<const __bf16*>(p.d_o) + qrow * D + half * (D / 2);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qreg[s] = *reinterpret_cast<const bf16x8*>(qp + s * 8);
      doreg[s] = *reinterpret_cast<const bf16x8*>(gp + s * 8);
    }
  }
  const float L = p.lse[qrow];
  const float lse2 = L == -INFINITY ? INFINITY : L * kLog2e;  // a row that saw no key: P = 0
  const float dlt = p.delta[qrow];

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;

  const __bf16* Kg = static_cast<const __bf16*>(p.k);
  const __bf16* Vg = static_cast<const __bf16*>(p.v);
  u32x4 kpre[kLoads], vpre[kLoads];
  // loads of tile rows [kt, kt + kBN) of run ks (rows past the run repeat its last key: masked)
  auto load_tile = [&](const Seg& ks, int kt) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = i * kDqThreads + tid;
      const int row = idx / T::kChunks, ch = idx % T::kChunks;
      const int key = min(kt + row, ks.len - 1);
      const int64_t src = ((int64_t)(ks.loc + key) * p.n_kv + g) * D + ch * 8;
      kpre[i] = *reinterpret_cast<const u32x4*>(Kg + src);
      vpre[i] = *reinterpret_cast<const u32x4*>(Vg + src);
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* Ks = smem + buf * 2 * kTileBytes;
    unsigned char* Vs = Ks + kTileBytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = i * kDqThreads + tid;
      const int row = idx / T::kChunks, ch = idx % T::kChunks;
      const int o = T::off(row, ch * 8);
      *reinterpret_cast<u32x4*>(Ks + o) = kpre[i];
      *reinterpret_cast<u32x4*>(Vs + o) = vpre[i];
    }
  };

  // the KV tiles this workgroup sees: runs of its sequence, the prefix visible to its last row
  int j = 0, kt = 0;
  auto advance = [&](int jj, int tt) {  // next (run, tile) at or after (jj, tt), or j = n_kv_segs
    for (; jj < p.n_kv_segs; ++jj, tt = 0) {
      const Seg ks = p.ks[jj];
      if (ks.seq != qs.seq) continue;
      if (tt < visible_prefix(ks, qpos_hi, p.causal)) break;
    }
    j = jj;
    kt = tt;
  };
  advance(0, 0);
  // (ja, kta): the tile in buffer `cur`; (j, kt): the tile in the prefetch registers
  int cur = 0, ja = j, kta = kt;
  if (j < p.n_kv_segs) {
    load_tile(p.ks[j], kt);
    store_tile(0);
    advance(j, kt + kBN);
    if (j < p.n_kv_segs) load_tile(p.ks[j], kt);
  }
  while (ja < p.n_kv_segs) {
    __syncthreads();  // buffer `cur` is staged; every wave is done with the other one
    const int jn = j, ktn = kt;
    if (j < p.n_kv_segs) {
      store_tile(cur ^ 1);
      advance(j, kt + kBN);
      if (j < p.n_kv_segs) load_tile(p.ks[j], kt);  // in flight during this tile's math
    }
    const Seg ks = p.ks[ja];
    const int cur_kt = kta;
    const unsigned char* Ks = smem + cur * 2 * kTileBytes;
    const unsigned char* Vs = Ks + kTileBytes;

    // S^T = K Q^T and dP^T = V dO^T: two 32-key halves
    f32x16 s[2], dpt[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = dpt[kb][v] = 0.f;
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const int o = T::off(kb * 32 + col, 8 * (half * (D / 16) + st));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(Ks, o), qreg[st], s[kb], 0, 0, 0);
        dpt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(Vs, o), doreg[st], dpt[kb], 0, 0, 0);
      }
    }
    // keys past the causal frontier of this lane's row or past the run
    const int n_full = p.causal ? max(0, min(ks.len, qpos_lo - ks.pos + 1)) : ks.len;
    const bool masked = cur_kt + kBN > n_full;
    const int lim = p.causal ? min(ks.len, qpos - ks.pos + 1) : ks.len;
    // dS^T in bf16 as the B operand of dQ^T += K^T dS^T: k-step t holds keys
    // 16 t + 8 (e / 4) + 4 half + e % 4 == entries 8 (t % 2) + e of score block t / 2
    float pr[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) pr[kb][v] = __builtin_amdgcn_exp2f(fmaf(s[kb][v], p.scale_log2, -lse2));
    if (masked) {  // uniform: one branch around the whole mask
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ko = cur_kt + kb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          pr[kb][v] = ko < lim ? pr[kb][v] : 0.f;
        }
    }
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) pb[2 * kb + (v >> 3)][v & 7] = (__bf16)(pr[kb][v] * (dpt[kb][v] - dlt));
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_tr8<D>(Ks, 16 * t, db * 32, lane), pb[t],
                                                          acc[db], 0, 0, 0);
    cur ^= 1;
    ja = jn;
    kta = ktn;
  }
  if (!live) return;
  // dQ^T accumulator: lane (row, half) holds d = db*32 + 8 (v/4) + 4 half + v % 4
  float* out = p.dq + qrow * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      float4* o4 = reinterpret_cast<float4*>(out + db * 32 + 8 * vq + 4 * half);
      float4 x = *o4;
      x.x = fmaf(p.scale, acc[db][4 * vq], x.x);
      x.y = fmaf(p.scale, acc[db][4 * vq + 1], x.y);
      x.z = fmaf(p.scale, acc[db][4 * vq + 2], x.z);
      x.w = fmaf(p.scale, acc[db][4 * vq + 3], x.w);
      *o4 = x;
    }
}

// ------------------------------------------------------------------------------------ dK, dV
// A workgroup of 8 waves owns 128 keys: waves 0-3 accumulate dV of keys 32 w .. 32 w + 31 and
// waves 4-7 dK of the same keys, so each wave holds one accumulator set and one operand set and
// the kernel fits two waves per SIMD (each SIMD then runs one dV and one dK wave). Per block of 64
// query rows, a dV wave forms S = Q K^T and P, hands P to its dK wave through LDS, and adds P^T dO;
// the dK wave forms dP = dO V^T meanwhile, then dS = P (dP - delta) and adds dS^T Q: 32 MFMAs each,
// one barrier per block. The blocks are staged in three LDS buffers.
constexpr int kDkdvRows = 64;  // query rows per block (two MFMA row blocks)
// LDS of a dK/dV workgroup: three buffers, each holding a block's Q rows, dO rows, base-2 LSEs and
// deltas (block n is worked on in buffer n % 3 while block n + 1 is staged into the next one),
// then the P handed from each dV wave to the dK wave of the same keys, in fp16, in two slots
// (block n uses slot n % 2): per slot, 32-row half and key group, 16 values per lane stored as
// [8-value chunk][lane] (consecutive lanes, consecutive 16 bytes)
template <int D>
constexpr int dkdv_buf_bytes() { return 2 * kDkdvRows * BwdTile<D>::kRowBytes + 2 * kDkdvRows * 4; }
constexpr int kDkdvPBytes = 2 * 2 * 4 * 2 * 64 * 16;  // slots x halves x key groups x chunks x lanes x 16 B
template <int D>
constexpr int dkdv_lds_bytes() { return 3 * dkdv_buf_bytes<D>() + kDkdvPBytes; }

// The dK/dV workgroup `bx` of the plan: part bx % parts of key tile bx / parts.
template <int D>
__device__ __forceinline__ void bwd_dkdv_tile(const BwdParams& p, const BwdSplit& sp, int bx,
                                              unsigned char* smem) {
  using T = BwdTile<D>;
  constexpr int kThreads = 512;
  constexpr int kBR = kDkdvRows;
  constexpr int kBlockBytes = kBR * T::kRowBytes;
  constexpr int kLoads = kBR * T::kChunks / kThreads;  // 16-byte loads per thread per operand
  constexpr int kBufBytes = dkdv_buf_bytes<D>();
  uint4* pex = reinterpret_cast<uint4*>(smem + 3 * kBufBytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the mask branch is too
  const bool dk_wave = wave >= 4;                              // else a dV wave
  const int kw = wave & 3;                                     // which 32 keys of the tile
  const int col = lane & 31, half = lane >> 5;
  const int g = blockIdx.y;
  const int tt = bx / sp.parts;  // key tile in plan order
  const int part = bx - tt * sp.parts;
  int seg, tile;
  bwd_locate(p.kv_prefix, p.kv_order, p.n_kv_segs, tt, false, seg, tile);
  const Seg ks = p.ks[seg];
  const int key_wg = tile * kBwdKeys;               // the workgroup's first key in the run
  const int key0 = key_wg + kw * 32;                // this wave's first key
  const int kcol = key0 + col;                      // this lane's key (operand column)
  const int kc = min(kcol, ks.len - 1);
  const int kpos_wg_first = ks.pos + key_wg;
  const int kpos_wave_last = ks.pos + min(key0 + 31, ks.len - 1);
  const int kpos_lane = ks.pos + kcol;
  const bool wave_keys_whole = key0 + 32 <= ks.len;
  // The B operand of this lane's key: K^T in dV waves (S = Q K^T), V^T in dK waves
  // (dP = dO V^T); k-step s covers d = 8 (half * D/16 + s) + e
  bf16x8 breg[D / 16];
  {
    const int64_t krow = ((int64_t)(ks.loc + kc) * p.n_kv + g) * D + half * (D / 2);
    const __bf16* bp = static_cast<const __bf16*>(dk_wave ? p.v : p.k) + krow;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) breg[s] = *reinterpret_cast<const bf16x8*>(bp + s * 8);
  }
  // Retire these loads here: otherwise the wait analysis keeps them pending at the block loop's
  // header and makes every block's first products wait for the next block's prefetch as well.
  __builtin_amdgcn_s_waitcnt(kBwdWaitVmcnt0);
  f32x16 acc[D / 32];  // dK (dK waves) or dV (dV waves) of the wave's 32 keys
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;

  const __bf16* Qg = static_cast<const __bf16*>(p.q);
  const __bf16* Gg = static_cast<const __bf16*>(p.d_o);
  u32x4 qpre[kLoads], gpre[kLoads];
  float lpre = 0.f;
  // loads of flattened rows [b, b + 64) of Q run qs (rows past the run repeat its last row and get
  // LSE = +inf in the base-2 scale, hence P = 0); threads 0..63 load LSEs, 64..127 deltas
  const DivBy by_group(p.group);
  auto load_block = [&](const Seg& qs, int b) {
    const int rows = qs.len * p.group;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = i * kThreads + tid;
      const int row = idx / T::kChunks, ch = idx % T::kChunks;
      const int rr = min(b + row, rows - 1);
      const int tq = by_group(rr);
      const int64_t src = ((int64_t)(qs.loc + tq) * p.n_h + g * p.group + (rr - tq * p.group)) * D + ch * 8;
      qpre[i] = *reinterpret_cast<const u32x4*>(Qg + src);
      gpre[i] = *reinterpret_cast<const u32x4*>(Gg + src);
    }
    if (tid < 2 * kBR) {
      const int row = tid & (kBR - 1);
      const int rr = b + row;
      if (rr < rows) {
        const int tq = by_group(rr);
        const int64_t qrow = (int64_t)(qs.loc + tq) * p.n_h + g * p.group + (rr - tq * p.group);
        if (tid < kBR) {
          const float L = p.lse[qrow];
          lpre = L == -INFINITY ? INFINITY : L * kLog2e;
        } else {
          lpre = p.delta[qrow];
        }
      } else {
        lpre = tid < kBR ? INFINITY : 0.f;
      }
    }
  };
  auto store_block = [&](int buf) {
    unsigned char* Qs = smem + buf * kBufBytes;
    unsigned char* Gs = Qs + kBlockBytes;
    float* Ls = reinterpret_cast<float*>(Gs + kBlockBytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = i * kThreads + tid;
      const int row = idx / T::kChunks, ch = idx % T::kChunks;
      const int o = T::off(row, ch * 8);
      *reinterpret_cast<u32x4*>(Qs + o) = qpre[i];
      *reinterpret_cast<u32x4*>(Gs + o) = gpre[i];
    }
    if (tid < 2 * kBR) Ls[tid] = lpre;  // the deltas follow the LSEs
  };

  // the query blocks that see this workgroup's keys: runs of its sequence, from the first row
  // whose token may see the first key
  int j = 0, b = 0;
  auto first_row = [&](const Seg& qs) -> int {
    if (!p.causal) return 0;
    return max(0, kpos_wg_first - qs.pos) * p.group;
  };
  auto advance = [&](int jj, int bb) {  // next (run, block start) at or after (jj, bb)
    for (; jj < p.n_q_segs; ++jj, bb = -1) {
      const Seg qs = p.qs[jj];
      if (qs.seq != ks.seq) continue;
      if (bb < 0) bb = first_row(qs);
      if (bb < qs.len * p.group) break;
    }
    j = jj;
    b = bb;
  };
  // This workgroup's share: part `part` of the tile's visible blocks, split into equal runs.
  int n_blocks = 0;
  for (int jj = 0; jj < p.n_q_segs; ++jj) {
    const Seg qs = p.qs[jj];
    if (qs.seq != ks.seq) continue;
    const int rows = qs.len * p.group, fr = first_row(qs);
    if (fr < rows) n_blocks += (rows - fr + kBR - 1) / kBR;
  }
  const int blk_lo = (int)((int64_t)n_blocks * part / sp.parts);
  int left = (int)((int64_t)n_blocks * (part + 1) / sp.parts) - blk_lo;
  advance(0, -1);
  for (int skip = blk_lo; skip > 0 && j < p.n_q_segs;) {  // move to visible block blk_lo
    const int here = (p.qs[j].len * p.group - b + kBR - 1) / kBR;  // blocks of run j from b on
    if (skip < here) {
      b += skip * kBR;
      skip = 0;
    } else {
      skip -= here;
      advance(j + 1, -1);
    }
  }
  // (ja, ba): the block in buffer `cur`; (j, b): the block in the prefetch registers. A block is
  // worked on in two phases split by one barrier. Phase 1: the next block is stored into the next
  // buffer (whose last reads, two blocks back, preceded the previous barrier); a dV wave forms
  // S = Q K^T of both halves and the masked P, and hands P over; a dK wave forms dP = dO V^T of
  // both halves. Phase 2: the dK wave forms dS = P (dP - delta) from the handed-over P; the dV wave
  // adds P^T dO and the dK wave dS^T Q. The P slot of block n is written again by block n + 2,
  // after the barrier of block n + 1.
  int cur = 0, slot = 0, ja = j, ba = b;
  if (left > 0) {
    load_block(p.qs[j], b);
    store_block(0);
    if (left > 1) {
      advance(j, b + kBR);
      load_block(p.qs[j], b);
    }
    __syncthreads();  // block 0 is staged
  }
  while (left > 0) {
    const int jn = j, bn = b;
    const int nxt = cur == 2 ? 0 : cur + 1;
    if (left > 1) {
      store_block(nxt);
      if (left > 2) {
        advance(j, b + kBR);
        load_block(p.qs[j], b);
      }
    }
    const Seg qs = p.qs[ja];
    const unsigned char* Qb = smem + cur * kBufBytes;
    const unsigned char* Gb = Qb + kBlockBytes;
    const float* Lb = reinterpret_cast<const float*>(Gb + kBlockBytes);
    // S = Q K^T (dV waves) or dP = dO V^T (dK waves) of both 32-row halves: lane (key, half)
    // holds rows 32 h + 8 (v/4) + 4 half + v % 4
    f32x16 s[2];
    // the A operands of dV += P^T dO (dV waves) or of dK += dS^T Q with dS = P (dP - delta)
    // (dK waves); for half h, k-step t holds rows 32 h + 16 t + 8 (e/4) + 4 half + e % 4
    bf16x8 pa[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[h][v] = 0.f;
      const unsigned char* As = (dk_wave ? Gb : Qb) + 32 * h * T::kRowBytes;
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const int o = T::off(col, 8 * (half * (D / 16) + st));
        s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(As, o), breg[st], s[h], 0, 0, 0);
      }
    }
    if (!dk_wave) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cur_b = ba + 32 * h;
        const float* Ls = Lb + 32 * h;
        uint4* ph = pex + ((slot * 2 + h) * 4 + kw) * 2 * 64;  // this half's P of this key group
        // the half's rows are all visible to all of this wave's keys, or the mask is needed (a
        // wave-uniform branch around the whole mask)
        const bool masked = !wave_keys_whole ||
                            (p.causal && qs.pos + cur_b / p.group < kpos_wave_last);
        f32x16 pr;
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const float4 l4 = *reinterpret_cast<const float4*>(Ls + 8 * vq + 4 * half);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pr[4 * vq + e] = __builtin_amdgcn_exp2f(fmaf(s[h][4 * vq + e], p.scale_log2, -lv[e]));
        }
        if (masked) {
          // key kcol is visible to row rr (token rr / G of the run) iff kcol < len and, with
          // the causal mask, the token's position reaches the key's: rr >= row_min. Entry v is
          // row cur_b + 4 half + c(v) with c(v) = 8 (v/4) + v % 4, visible iff c(v) >= thr.
          const int row_min = p.causal ? min(max(kpos_lane - qs.pos, 0), qs.len) * p.group : 0;
          const int thr = kcol < ks.len ? row_min - cur_b - 4 * half : INT_MAX;
#pragma unroll
          for (int v = 0; v < 16; ++v) pr[v] = 8 * (v >> 2) + (v & 3) >= thr ? pr[v] : 0.f;
        }
        ph[lane] = __builtin_bit_cast(uint4, __builtin_convertvector(
            __builtin_shufflevector(pr, pr, 0, 1, 2, 3, 4, 5, 6, 7), f16x8));
        ph[64 + lane] = __builtin_bit_cast(uint4, __builtin_convertvector(
            __builtin_shufflevector(pr, pr, 8, 9, 10, 11, 12, 13, 14, 15), f16x8));
#pragma unroll
        for (int v = 0; v < 16; ++v) pa[h][v >> 3][v & 7] = (__bf16)pr[v];
      }
    }
    __syncthreads();  // the dV waves' P of the block is in LDS; the next block is staged
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (dk_wave) {
        // the same lane of the paired dV wave holds P of the same (row, key) entries
        const float* Ds = Lb + kBR + 32 * h;
        const uint4* ph = pex + ((slot * 2 + h) * 4 + kw) * 2 * 64;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const f16x8 p8 = __builtin_bit_cast(f16x8, ph[c * 64 + lane]);
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) {
            const float4 d4 = *reinterpret_cast<const float4*>(Ds + 8 * (2 * c + q2) + 4 * half);
            const float dlv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int v = 8 * c + 4 * q2 + e;
              pa[h][v >> 3][v & 7] = (__bf16)((float)p8[4 * q2 + e] * (s[h][v] - dlv[e]));
            }
          }
        }
      }
      const unsigned char* Bs = (dk_wave ? Qb : Gb) + 32 * h * T::kRowBytes;  // Q for dK, dO for dV
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[h][t], lds_tr8<D>(Bs, 16 * t, db * 32, lane),
                                                            acc[db], 0, 0, 0);
    }
    --left;
    cur = nxt;
    slot ^= 1;
    ja = jn;
    ba = bn;
  }
  // accumulator: lane (d = db*32 + col, half) holds keys key0 + 8 (v/4) + 4 half + v % 4
  if (sp.parts == 1) {
    float* out = dk_wave ? p.dk : p.dv;
    const float sc = dk_wave ? p.scale : 1.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = key0 + 8 * (v >> 2) + 4 * half + (v & 3);
      if (key >= ks.len) continue;
      const int64_t base = ((int64_t)(ks.loc + key) * p.n_kv + g) * D + col;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) out[base + db * 32] = fmaf(sc, acc[db][v], out[base + db * 32]);
    }
  } else {
    // this part's sums into its workspace slot: [128 keys][D] unscaled dK, then the same for dV
    // (keys past the run's end hold zeros: their probabilities were masked)
    float* w = sp.ws + ((int64_t)(g * p.kv_tiles + tt) * sp.parts + part) * (2 * kBwdKeys * D) +
               (dk_wave ? 0 : kBwdKeys * D);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kl = kw * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) w[kl * D + db * 32 + col] = acc[db][v];
    }
  }
}

// One launch per ring step for both halves of the backward: workgroups [0, n_dkdv) are the
// dK/dV workgroups of the plan, the rest its dQ workgroups. The two kinds have the same shape
// (8 waves, at most 256 VGPRs, one workgroup per CU), so the CUs that finish the longer dK/dV
// workgroups take the dQ ones and neither half leaves a tail of idle CUs of its own.
template <int D>
__global__ __launch_bounds__(512, 2) void bwd_kernel(const BwdParams p, const BwdSplit sp, int n_dkdv) {
  constexpr int kLds = dq_lds_bytes<D>() > dkdv_lds_bytes<D>() ? dq_lds_bytes<D>() : dkdv_lds_bytes<D>();
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  const int bx = blockIdx.x;
  if (bx < n_dkdv)
    bwd_dkdv_tile<D>(p, sp, bx, smem);
  else
    bwd_dq_tile<D>(p, bx - n_dkdv, smem);
}

// Sum of the parts of a split dK/dV launch, in part order, added into dk (times scale) and dv.
// A thread owns 4 consecutive d of one key; a workgroup covers 256 / (D / 4) keys of one tile.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const BwdParams p, const BwdSplit sp) {
  constexpr int kVec = D / 4;
  constexpr int kKeysPerBlock = 256 / kVec;
  constexpr int kBlocksPerTile = kBwdKeys / kKeysPerBlock;
  const int tt = blockIdx.x / kBlocksPerTile;
  const int kl = (blockIdx.x - tt * kBlocksPerTile) * kKeysPerBlock + (int)threadIdx.x / kVec;
  const int d4 = (int)threadIdx.x % kVec;
  const int g = blockIdx.y;
  int seg, tile;
  bwd_locate(p.kv_prefix, p.kv_order, p.n_kv_segs, tt, false, seg, tile);
  const Seg ks = p.ks[seg];
  const int key = tile * kBwdKeys + kl;
  if (key >= ks.len) return;
  constexpr int64_t kPart4 = 2 * kBwdKeys * D / 4;  // float4s per slot
  constexpr int64_t kV4 = kBwdKeys * D / 4;         // dV's offset in a slot
  const float4* src = reinterpret_cast<const float4*>(sp.ws) +
                      (int64_t)(g * p.kv_tiles + tt) * sp.parts * kPart4 + kl * kVec + d4;
  float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
  for (int c = 0; c < sp.parts; ++c) {
    const float4 a = src[c * kPart4], b = src[c * kPart4 + kV4];
    sk.x += a.x; sk.y += a.y; sk.z += a.z; sk.w += a.w;
    sv.x += b.x; sv.y += b.y; sv.z += b.z; sv.w += b.w;
  }
  const int64_t o = ((int64_t)(ks.loc + key) * p.n_kv + g) * D + d4 * 4;
  float4* k4 = reinterpret_cast<float4*>(p.dk + o);
  float4* v4 = reinterpret_cast<float4*>(p.dv + o);
  float4 x = *k4, y = *v4;
  x.x = fmaf(p.scale, sk.x, x.x); x.y = fmaf(p.scale, sk.y, x.y);
  x.z = fmaf(p.scale, sk.z, x.z); x.w = fmaf(p.scale, sk.w, x.w);
  y.x += sv.x; y.y += sv.y; y.z += sv.z; y.w += sv.w;
  *k4 = x;
  *v4 = y;
}

// ---------------------------------------------------------------------------------- delta
// delta = dO . O per row (the row term of the softmax gradient). 16 lanes per row.
template <int D, bool DO_BF16>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const float* o, const void* d_o, int64_t rows,
                                                        float* delta) {
  constexpr int kPer = D / 16;
  const int sub = threadIdx.x & 15;
  for (int64_t r = (int64_t)blockIdx.x * 16 + threadIdx.x / 16; r < rows; r += (int64_t)gridDim.x * 16) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int64_t i = r * D + sub * kPer + e;
      const float gv = DO_BF16 ? (float)static_cast<const __bf16*>(d_o)[i] : static_cast<const float*>(d_o)[i];
      acc = fmaf(gv, o[i], acc);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
    if (sub == 0) delta[r] = acc;
  }
}

hipError_t launch_bwd(const BwdParams& p, int d_h, hipStream_t stream) {
  return launch_bwd_split(p, BwdSplit{nullptr, 1}, d_h, stream);
}

hipError_t launch_bwd_split(const BwdParams& p, const BwdSplit& sp, int d_h, hipStream_t stream) {
  static_assert(kDqThreads == 512, "dQ and dK/dV workgroups share one launch shape");
  const int n_dkdv = p.kv_tiles * sp.parts;
  if (p.q_tiles + n_dkdv > 0) {
    const dim3 grid(n_dkdv + p.q_tiles, p.n_kv);
    if (d_h == 64)
      hipLaunchKernelGGL(bwd_kernel<64>, grid, dim3(512), 0, stream, p, sp, n_dkdv);
    else
      hipLaunchKernelGGL(bwd_kernel<128>, grid, dim3(512), 0, stream, p, sp, n_dkdv);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.kv_tiles > 0) {
    if (sp.parts > 1) {
      // kBwdKeys / (256 / (d_h / 4)) workgroups per tile
      const dim3 rgrid(p.kv_tiles * (kBwdKeys * d_h / 4 / 256), p.n_kv);
      if (d_h == 64)
        hipLaunchKernelGGL(bwd_dkdv_reduce_kernel<64>, rgrid, dim3(256), 0, stream, p, sp);
      else
        hipLaunchKernelGGL(bwd_dkdv_reduce_kernel<128>, rgrid, dim3(256), 0, stream, p, sp);
    }
  }
  return hipGetLastError();
}

hipError_t launch_bwd_delta(const float* o, const void* d_o, bool do_bf16, int64_t rows, int d_h,
                            float* delta, hipStream_t stream) {
  const int64_t blocks = std::min<int64_t>((rows + 15) / 16, 65536);
  const dim3 grid((unsigned)blocks), block(256);
  if (d_h == 64) {
    if (do_bf16) hipLaunchKernelGGL((bwd_delta_kernel<64, true>), grid, block, 0, stream, o, d_o, rows, delta);
    else hipLaunchKernelGGL((bwd_delta_kernel<64, false>), grid, block, 0, stream, o, d_o, rows, delta);
  } else {
    if (do_bf16) hipLaunchKernelGGL((bwd_delta_kernel<128, true>), grid, block, 0, stream, o, d_o, rows, delta);
    else hipLaunchKernelGGL((bwd_delta_kernel<128, false>), grid, block, 0, stream, o, d_o, rows, delta);
  }
  return hipGetLastError();
}

}  // namespace cpk

// --------------------------------------------------------------------------- fp32 inputs
// The same gradients for fp32 inputs in fp32 arithmetic throughout (no reduced-precision MFMA),
// for small workloads where exactness to ~1e-5 matters more than speed.
namespace cpk {

// One thread per query row (token, head): dQ over the keys it sees.
template <int D>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(const BwdParams p) {
  int seg, tile;
  bwd_locate(p.q_prefix, p.q_order, p.n_q_segs, blockIdx.x, false, seg, tile);
  const int g = blockIdx.y;
  const Seg qs = p.qs[seg];
  const int rows = qs.len * p.group;
  const int r = tile * 64 + (int)threadIdx.x;
  if (r >= rows) return;
  const int tok = r / p.group;
  const int64_t qrow = (int64_t)(qs.loc + tok) * p.n_h + g * p.group + r % p.group;
  const int qpos = qs.pos + tok;
  const float L = p.lse[qrow];
  if (L == -INFINITY) return;  // the row saw no key
  const float dlt = p.delta[qrow];
  const float* Q = static_cast<const float*>(p.q) + qrow * D;
  const float* G = static_cast<const float*>(p.d_o) + qrow * D;
  const float* K = static_cast<const float*>(p.k);
  const float* V = static_cast<const float*>(p.v);
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  for (int j = 0; j < p.n_kv_segs; ++j) {
    const Seg ks = p.ks[j];
    if (ks.seq != qs.seq) continue;
    const int n = visible_prefix(ks, qpos, p.causal);
    for (int key = 0; key < n; ++key) {
      const float* kr = K + ((int64_t)(ks.loc + key) * p.n_kv + g) * D;
      const float* vr = V + ((int64_t)(ks.loc + key) * p.n_kv + g) * D;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(Q[d], kr[d], s);
        dp = fmaf(G[d], vr[d], dp);
      }
      const float pr = expf(s * p.scale - L);
      const float ds = pr * (dp - dlt);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, kr[d], acc[d]);
    }
  }
  float* out = p.dq + qrow * D;
#pragma unroll
  for (int d = 0; d < D; ++d) out[d] = fmaf(p.scale, acc[d], out[d]);
}

// One thread per key (and KV head): dK and dV over the rows that see it, accumulated in LDS.
template <int D>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(const BwdParams p) {
  __shared__ float acc_k[64 * D];
  __shared__ float acc_v[64 * D];
  int seg, tile;
  bwd_locate(p.kv_prefix, p.kv_order, p.n_kv_segs, blockIdx.x, false, seg, tile);
  const int g = blockIdx.y;
  const Seg ks = p.ks[seg];
  const int t = threadIdx.x;
  const int key = tile * 64 + t;
  if (key >= ks.len) return;  // no barrier below: threads are independent
  float* ak = acc_k + t * D;
  float* av = acc_v + t * D;
  for (int d = 0; d < D; ++d) ak[d] = av[d] = 0.f;
  const int kpos = ks.pos + key;
  const int64_t krow = ((int64_t)(ks.loc + key) * p.n_kv + g) * D;
  const float* kr = static_cast<const float*>(p.k) + krow;
  const float* vr = static_cast<const float*>(p.v) + krow;
  for (int i = 0; i < p.n_q_segs; ++i) {
    const Seg qs = p.qs[i];
    if (qs.seq != ks.seq) continue;
    const int tok0 = p.causal ? max(0, kpos - qs.pos) : 0;
    for (int tok = tok0; tok < qs.len; ++tok) {
      for (int h = 0; h < p.group; ++h) {
        const int64_t qrow = (int64_t)(qs.loc + tok) * p.n_h + g * p.group + h;
        const float L = p.lse[qrow];
        if (L == -INFINITY) continue;
        const float* Q = static_cast<const float*>(p.q) + qrow * D;
        const float* G = static_cast<const float*>(p.d_o) + qrow * D;
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          s = fmaf(Q[d], kr[d], s);
          dp = fmaf(G[d], vr[d], dp);
        }
        const float pr = expf(s * p.scale - L);
        const float ds = pr * (dp - p.delta[qrow]);
        for (int d = 0; d < D; ++d) {
          ak[d] = fmaf(ds, Q[d], ak[d]);
          av[d] = fmaf(pr, G[d], av[d]);
        }
      }
    }
  }
  float* dk = p.dk + krow;
  float* dv = p.dv + krow;
  for (int d = 0; d < D; ++d) {
    dk[d] = fmaf(p.scale, ak[d], dk[d]);
    dv[d] += av[d];
  }
}

hipError_t launch_bwd_f32(const BwdParams& p, int d_h, hipStream_t stream) {
  if (p.q_tiles > 0) {
    const dim3 grid(p.q_tiles, p.n_kv);
    if (d_h == 64)
      hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, grid, dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, grid, dim3(64), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.kv_tiles > 0) {
    const dim3 grid(p.kv_tiles, p.n_kv);
    if (d_h == 64)
      hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, grid, dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL(bwd_dkdv_f32_kernel<128>, grid, dim3(64), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace cpk
