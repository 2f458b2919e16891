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
// each taking a quarter of its keys, and combine their results in LDS:
//  - K and V blocks are loaded with whole-row 16-byte non-temporal accesses (the cache is read
//    once; the loads must not evict the split partials the merge reads back) and staged in LDS
//    in their row-major layout;
//  - S^T = K q^T on v_mfma_f32_16x16x32_bf16: 16 keys x 16 heads per MFMA, q^T held in
//    registers;
//  - V comes back from LDS as the V^T operand of O^T += V^T P^T via ds_read_b64_tr_b16;
//  - the next block's K and V loads are issued before the current block's math, and the first
//    block's loads are in flight together with the query's.
// Each split's partial O is normalised (a convex combination of V rows) and stored in bf16, the
// precision of the probabilities its P.V already used; its LSE stays fp32. The merge kernel then
// combines the S partials of each (request, head) with the same LSE-weighted rule as
// cp_merge_lse.
//
// Pages cited: [CPEP] "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두
// 축"; [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (paper review).
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

// W waves share one (request, split, 16-head block): wave w takes the w-th of W equal parts of
// the split's keys with LDS of its own, and the W partial results are combined in LDS before
// the split's partial is written. W = 1 for large batches (enough workgroups to fill the chip);
// W = 4 for small ones, where one wave per split would leave most of each CU idle.
template <int D, int W>
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
  // splits and the tail of the launch stays short. For batches of up to 64 requests, lane i ranks
  // request i by length (ties by index) and the workgroup picks the request of rank blockIdx/S.
  int b = blockIdx.x / p.n_splits;
  if (p.batch <= 64) {
    const int want = b;
    const int i = lane;
    const int64_t li = i < p.batch ? p.kv_len[i] : -1;
    int rank = 0;
    for (int j = 0; j < p.batch; ++j) {
      const int64_t lj = p.kv_len[j];
      rank += (lj > li) || (lj == li && j < i);
    }
    const unsigned long long hit = __ballot(i < p.batch && rank == want);
    b = __ffsll(hit) - 1;
  }
  const int hblocks = (p.group + 15) / 16;
  const int g = blockIdx.y / hblocks;
  const int h0 = (blockIdx.y % hblocks) * 16;
  const int col = lane & 15;  // head column of the 16x16 blocks
  const int grp = lane >> 4;  // 0..3: k slice of the operands, row group of the accumulator
  const int64_t L = p.kv_len[b] > 0 ? p.kv_len[b] : 0;  // a negative length reads as an empty cache
  const int64_t base = p.kv_offset[b];
  const int64_t lo = ((int64_t)c * L) / p.n_splits;
  const int64_t hi = ((int64_t)(c + 1) * L) / p.n_splits;
  // this wave's part of the split
  const int64_t wlo = lo + ((hi - lo) * wave) / W;
  const int64_t whi = lo + ((hi - lo) * (wave + 1)) / W;
  const int n = (int)(whi - wlo);

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

  float m = -INFINITY, l = 0.f;
  f32x4 oacc[C::kDBlocks];
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tr-read addressing: lane group grp reads 4 key rows, 4 lanes per row, 4 d per lane
  const int j16 = lane & 15;
  const int tr_row = 4 * grp + (j16 >> 2);
  const int tr_col = 4 * (j16 & 3);

  // The staging LDS is this wave's own: the wave's LDS accesses are ordered among themselves, so
  // the loop needs no workgroup barrier (and waves with different key counts never meet one).
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
  // The partial O of this (request, split, head block) is a [heads][D] bf16 tile, and the
  // workspace layout [batch][n_splits][n_h][D] makes its valid heads one contiguous block. A lane
  // holds 4-value pieces of one head's row; stored directly, every instruction would write 16
  // separate 8-byte pieces. The tile goes through this wave's staging LDS instead (no longer
  // read; the wave's LDS accesses are in order) and leaves as whole rows, 16 bytes per lane,
  // each instruction covering 1 KB of consecutive bytes.
  constexpr int kTStride = D * 2 + 32;  // padded rows: the scattered 8-byte writes spread over banks
  unsigned char* tile = ks;
#pragma unroll
  for (int db = 0; db < C::kDBlocks; ++db) {
    const bf16x4 o4 = {(__bf16)(oacc[db][0] * inv), (__bf16)(oacc[db][1] * inv),
                       (__bf16)(oacc[db][2] * inv), (__bf16)(oacc[db][3] * inv)};
    *reinterpret_cast<bf16x4*>(tile + col * kTStride + (db * 16 + 4 * grp) * 2) = o4;
  }
  const int n_valid = min(16, p.group - h0);  // heads of this block that exist
  const int64_t prow0 = ((int64_t)b * p.n_splits + c) * p.n_h + g * p.group + h0;
  unsigned char* wo = reinterpret_cast<unsigned char*>(static_cast<__bf16*>(p.ws_o) + prow0 * D);
  constexpr int kLanesPerRow = D * 2 / 16;
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += kRowsPerStore) {
    const int r = r0 + lane / kLanesPerRow;
    const int c16 = (lane % kLanesPerRow) * 16;
    if (r < n_valid)
      *reinterpret_cast<u32x4*>(wo + r * (D * 2) + c16) = *reinterpret_cast<const u32x4*>(tile + r * kTStride + c16);
  }
  if (grp == 0 && head_ok) p.ws_lse[prow0 + col] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
}

// Merge of the S split partials of each (request, head): one workgroup per (request, head),
// whose partials are S rows of D bf16 values (and S fp32 LSEs), n_h rows apart. D/8 lanes cover
// a row, 16 bytes each; the 256 / (D/8) lane groups take every kGroups-th split. A lane issues
// the loads of up to kBatch splits (their LSEs and O slices) before combining any of them, so
// one round of loads covers 256 splits at D = 128; batches are folded into a running max,
// weight and sum. The groups are then combined through LDS in a fixed order.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeParams p) {
  constexpr int kLanes = D / 8;
  constexpr int kGroups = 256 / kLanes;
  constexpr int kBatch = 16;
  __shared__ float red_m[kGroups];
  __shared__ float red_w[kGroups];
  __shared__ float red_o[kGroups][kLanes][8];
  const int r = blockIdx.x;  // b * n_h + head
  const int grp = threadIdx.x / kLanes;
  const int c8 = threadIdx.x % kLanes;
  const int64_t row0 = (int64_t)(r / p.n_h) * p.n_splits * p.n_h + r % p.n_h;  // split 0's row
  const float* lse = p.ws_lse + row0;
  const __bf16* o = static_cast<const __bf16*>(p.ws_o) + row0 * D + c8 * 8;
  const int64_t stride = p.n_h;  // rows between consecutive splits

  float M = -INFINITY, wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c0 = grp; c0 < p.n_splits; c0 += kGroups * kBatch) {
    float li[kBatch];
    bf16x8 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = min(c0 + i * kGroups, p.n_splits - 1);  // clamped: in bounds, masked below
      li[i] = c0 + i * kGroups < p.n_splits ? lse[c * stride] : -INFINITY;
      v[i] = *reinterpret_cast<const bf16x8*>(o + c * stride * D);
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) Mb = fmaxf(Mb, li[i]);
    if (Mb == -INFINITY) continue;  // nothing seen yet
    const float a = expf(M - Mb);    // M = -inf -> 0
    wsum *= a;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= a;
    M = Mb;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float w = expf(li[i] - M);  // -inf -> 0: the part saw no key
      if (w == 0.f) continue;           // skip its O, which may be anything
      wsum += w;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, (float)v[i][e], acc[e]);
    }
  }
  if (c8 == 0) red_m[grp] = M;
  __syncthreads();
  float Mt = red_m[0];
#pragma unroll
  for (int i = 1; i < kGroups; ++i) Mt = fmaxf(Mt, red_m[i]);
  const float a = (M == -INFINITY) ? 0.f : expf(M - Mt);
#pragma unroll
  for (int e = 0; e < 8; ++e) red_o[grp][c8][e] = acc[e] * a;
  if (c8 == 0) red_w[grp] = wsum * a;
  __syncthreads();
  if (grp != 0) return;
  wsum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < kGroups; ++i) {  // fixed order: deterministic
    wsum += red_w[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += red_o[i][c8][e];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t orow = (int64_t)r * D + c8 * 8;
  if (OUT_BF16) {
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(p.o_out) + orow) = out;
  } else {
    float* out = static_cast<float*>(p.o_out) + orow;
    *reinterpret_cast<float4*>(out) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
  if (c8 == 0 && p.lse_out) p.lse_out[r] = wsum > 0.f ? Mt + logf(wsum) : -INFINITY;
}

hipError_t launch_decode(const DecodeParams& p, int d_h, hipStream_t stream) {
  const int hblocks = (p.group + 15) / 16;
  const dim3 grid(p.n_splits * p.batch, p.n_kv * hblocks);
  const dim3 mgrid(p.batch * p.n_h);
  // Fewer workgroups than 8 per CU: four waves share each split.
  const bool wide = (int64_t)grid.x * grid.y < 2048;
  if (d_h == 64) {
    if (wide)
      hipLaunchKernelGGL((decode_split_kernel<64, 4>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_split_kernel<64, 1>), grid, dim3(64), 0, stream, p);
    if (p.out_bf16)
      hipLaunchKernelGGL((decode_merge_kernel<64, true>), mgrid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_merge_kernel<64, false>), mgrid, dim3(256), 0, stream, p);
  } else {
    if (wide)
      hipLaunchKernelGGL((decode_split_kernel<128, 4>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_split_kernel<128, 1>), grid, dim3(64), 0, stream, p);
    if (p.out_bf16)
      hipLaunchKernelGGL((decode_merge_kernel<128, true>), mgrid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_merge_kernel<128, false>), mgrid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace cpk
