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
//    one row space (row = token * G + head). A workgroup of 4 waves owns 256 rows; every K/V tile
//    it stages in LDS serves all of them (for G = 16 that is 16 tokens x 16 heads).
//  - Orientation S^T = K Q^T: v_mfma_f32_32x32x16_bf16 with K as the A operand (rows = keys)
//    and Q^T as the B operand (columns = queries). In the 32x32 accumulator a lane holds 16 keys
//    of one query, so a query's row max needs only one exchange between the two half-waves.
//  - Each wave keeps two 32-query blocks: their Q^T operands stay in registers for the whole
//    kernel and every K or V operand read from LDS feeds two MFMAs.
//  - P.V as O^T = V^T P^T: the probabilities, rounded to bf16, are already laid out as the
//    B operand; V^T comes straight from the row-major V tile with ds_read_b64_tr_b16, whose
//    16-lane transpose turns four key rows into per-lane key vectors.
//  - Online softmax in base 2 with scale*log2(e) folded into one FMA, fp32 accumulators, LSE
//    returned in natural log.
//  - Masks are computed from segment positions, never stored. Tiles entirely visible to every
//    row of the workgroup skip the mask; runs of other sequences and keys past the causal
//    frontier are never loaded.
//  - K/V tiles are double-buffered in LDS; the next tile's global loads are issued before the
//    current tile's math.
//
// Pages cited: [CPEP] "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두
// 축"; [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (paper review).
#include "device_common.h"

namespace cpk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

template <int D>
struct Bf16Cfg {
  static constexpr int kRows = kTileRowsBf16;   // query rows per workgroup
  static constexpr int kThreads = 256;
  static constexpr int kBN = 64;                // keys per LDS tile
  static constexpr int kStride = D * 2 + 16;    // padded LDS row (bytes)
  static constexpr int kTileBytes = kBN * kStride;
  static constexpr int kChunks = D / 8;         // 16-byte chunks per key row
  static constexpr int kRowsPerPass = kThreads / kChunks;
  static constexpr int kPasses = kBN / kRowsPerPass;
  static constexpr int kKSteps = D / 16;        // MFMA k-steps over the head dimension
  static constexpr int kDBlocks = D / 32;       // 32-row blocks of O^T
};

__device__ inline bf16x8 lds_read_b128(const unsigned char* base, int byte_off) {
  return *reinterpret_cast<const bf16x8*>(base + byte_off);
}

__device__ inline i16x4 lds_read_tr(const unsigned char* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + byte_off));
}

template <int D>
__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(const AttnParams p) {
  using C = Bf16Cfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * C::kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column of this lane in a 32x32 block
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

  // ---- this lane's two query rows and their Q^T operands -------------------------------
  int qpos[2];
  bool live[2];
  int64_t qrow[2];
  bf16x8 qreg[2][C::kKSteps];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int r = tile_row0 + wave * 64 + b * 32 + col;
    live[b] = r < rows;
    const int rc = live[b] ? r : rows - 1;
    const int tok = rc / p.group;
    qpos[b] = qs.pos + tok;
    qrow[b] = (int64_t)(qs.loc + tok) * p.n_h + g * p.group + rc % p.group;
    const __bf16* qp = Q + qrow[b] * D + half * (D / 2);
#pragma unroll
    for (int s = 0; s < C::kKSteps; ++s) qreg[b][s] = *reinterpret_cast<const bf16x8*>(qp + s * 8);
  }

  // ---- KV tile iteration: runs of the same sequence, prefix visible to the last query ----
  auto run_visible = [&](int j) -> int {
    const Seg ks = p.ks[j];
    if (ks.seq != qs.seq) return 0;
    return visible_prefix(ks, qpos_hi, p.causal);
  };
  int j = 0;
  while (j < p.n_kv_segs && run_visible(j) == 0) ++j;
  int kt = 0;

  const int ld_chunk = tid % C::kChunks;
  const int ld_row0 = tid / C::kChunks;
  uint4 kbuf[C::kPasses], vbuf[C::kPasses];
  auto global_load = [&](int jj, int kk) {
    const Seg ks = p.ks[jj];
#pragma unroll
    for (int ps = 0; ps < C::kPasses; ++ps) {
      int key = kk + ld_row0 + ps * C::kRowsPerPass;
      key = key < ks.len ? key : ks.len - 1;  // rows past the run are masked; stay in bounds
      const int64_t off = ((int64_t)(ks.loc + key) * p.n_kv + g) * D + ld_chunk * 8;
      kbuf[ps] = *reinterpret_cast<const uint4*>(K + off);
      vbuf[ps] = *reinterpret_cast<const uint4*>(V + off);
    }
  };
  auto lds_store = [&](int stage) {
    unsigned char* kt_s = smem + (stage * 2) * C::kTileBytes;
    unsigned char* vt_s = kt_s + C::kTileBytes;
#pragma unroll
    for (int ps = 0; ps < C::kPasses; ++ps) {
      const int r = ld_row0 + ps * C::kRowsPerPass;
      *reinterpret_cast<uint4*>(kt_s + r * C::kStride + ld_chunk * 16) = kbuf[ps];
      *reinterpret_cast<uint4*>(vt_s + r * C::kStride + ld_chunk * 16) = vbuf[ps];
    }
  };

  float m[2] = {-INFINITY, -INFINITY};  // running max, base-2 scaled units
  float l[2] = {0.f, 0.f};              // running sum (this half-wave's keys)
  f32x16 oacc[2][C::kDBlocks];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[b][db][v] = 0.f;

  if (j < p.n_kv_segs) {
    global_load(j, kt);
    lds_store(0);
  }
  __syncthreads();

  // V^T operand addressing for ds_read_b64_tr_b16 (see header): lane group of 16 -> 8 d-rows
  const int grp = lane >> 4;          // 0..3
  const int dsub = grp & 1;           // which 16 of the 32 d-rows
  const int j16 = lane & 15;
  const int tr_key = 4 * half + (j16 >> 2);
  const int tr_dcol = dsub * 16 + 4 * (j16 & 3);

  int stage = 0;
  while (j < p.n_kv_segs) {
    // next tile (uniform across the workgroup)
    int nj = j, nkt = kt + C::kBN;
    if (nkt >= run_visible(j)) {
      nj = j + 1;
      while (nj < p.n_kv_segs && run_visible(nj) == 0) ++nj;
      nkt = 0;
    }
    const bool has_next = nj < p.n_kv_segs;
    if (has_next) global_load(nj, nkt);

    const Seg ks = p.ks[j];
    const unsigned char* Kt = smem + (stage * 2) * C::kTileBytes;
    const unsigned char* Vt = Kt + C::kTileBytes;

    // ---- S^T = K Q^T for both query blocks and both 32-key halves of the tile ----
    f32x16 s[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[b][kb][v] = 0.f;
#pragma unroll
    for (int st = 0; st < C::kKSteps; ++st) {
      const int coff = (half * (D / 2) + st * 8) * 2;
      const bf16x8 a0 = lds_read_b128(Kt, col * C::kStride + coff);
      const bf16x8 a1 = lds_read_b128(Kt, (32 + col) * C::kStride + coff);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        s[b][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[b][st], s[b][0], 0, 0, 0);
        s[b][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[b][st], s[b][1], 0, 0, 0);
      }
    }

    // ---- mask (only tiles not fully visible to every row of the workgroup) ----
    const int n_full = p.causal ? max(0, min(ks.len, qpos_lo - ks.pos + 1)) : ks.len;
    if (kt + C::kBN > n_full) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int ko = kt + kb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            const bool vis = ko < ks.len && (!p.causal || ks.pos + ko <= qpos[b]);
            if (!vis) s[b][kb][v] = -INFINITY;
          }
    }

    // ---- online softmax (base 2) ----
    bf16x8 pb[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[b][kb][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[b], mx * p.scale_log2);
      const float msafe = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(m[b] - msafe);
      m[b] = mnew;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[b][kb][v], p.scale_log2, -msafe));
          s[b][kb][v] = e;
          rs += e;
        }
      l[b] = l[b] * alpha + rs;
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[b][db][v] *= alpha;
      // P^T operand of k-step t: keys 16t + 8(e/4) + 4*half + e%4 == accumulator entries 8(t%2)+e
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[b][t][e] = (__bf16)s[b][t >> 1][8 * (t & 1) + e];
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int db = 0; db < C::kDBlocks; ++db) {
        const int off = (16 * t + tr_key) * C::kStride + (db * 32 + tr_dcol) * 2;
        const i16x4 lo = lds_read_tr(Vt, off);
        const i16x4 hi = lds_read_tr(Vt, off + 8 * C::kStride);
        const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 va = __builtin_bit_cast(bf16x8, both);
#pragma unroll
        for (int b = 0; b < 2; ++b)
          oacc[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[b][t], oacc[b][db], 0, 0, 0);
      }
    }

    if (has_next) lds_store(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    j = nj;
    kt = nkt;
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2, optional merge into the running result
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float lt = l[b] + __shfl_xor(l[b], 32);
    if (!live[b]) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_new = lt > 0.f ? (m[b] + __log2f(lt)) * kLn2 : -INFINITY;
    float wp = 0.f, wn = 1.f, lse_out = lse_new;
    if (p.accumulate) running_merge_weights(p.lse[qrow[b]], lse_new, wp, wn, lse_out);
    const float sc = wn * inv;
    float* orow = p.o + qrow[b] * D;
#pragma unroll
    for (int db = 0; db < C::kDBlocks; ++db)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int d0 = db * 32 + 8 * vq + 4 * half;
        float4 o4 = make_float4(oacc[b][db][4 * vq] * sc, oacc[b][db][4 * vq + 1] * sc,
                                oacc[b][db][4 * vq + 2] * sc, oacc[b][db][4 * vq + 3] * sc);
        if (p.accumulate) {
          const float4 prev = *reinterpret_cast<const float4*>(orow + d0);
          o4.x = fmaf(wp, prev.x, o4.x);
          o4.y = fmaf(wp, prev.y, o4.y);
          o4.z = fmaf(wp, prev.z, o4.z);
          o4.w = fmaf(wp, prev.w, o4.w);
        }
        *reinterpret_cast<float4*>(orow + d0) = o4;
      }
    if (half == 0) p.lse[qrow[b]] = lse_out;
  }
}

hipError_t launch_attn_bf16(const AttnParams& p, int d_h, hipStream_t stream) {
  const dim3 grid(p.total_tiles, p.n_kv);
  const dim3 block(256);
  if (d_h == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace cpk
