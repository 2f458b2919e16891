// merge.hip -- lossless LSE-weighted merge of partial attention results.
//
// Per row (query token, head): M = max_i LSE_i, w_i = exp(LSE_i - M),
// O = sum_i w_i O_i / sum_i w_i, LSE = M + ln sum_i w_i; a row no part saw gives O = 0,
// LSE = -inf ([CPMTI §3 "核心公式": Pass-Q ends with an All2All merge of partial attention
// results; §5 "关键实现细节" item 3; the ring variants are lossless and exact, §2).
//
// HBM-bound: D/4 lanes share a row and move 16 bytes each; a lane issues the loads of eight
// parts at once, all partial-O loads and the result stores non-temporal (streamed once). Parts whose LSE is -inf (they saw no key of this row, which the load-balanced
// layout produces in every ring step) are not read.
//
// Pages cited: [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (review).
#include <algorithm>

#include "device_common.h"

namespace cpk {
// Native vector for the non-temporal accesses (the partials are read once and the merged result
// is written once: neither should displace cached data).
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  constexpr int kLanesPerRow = D / 4;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  constexpr int kGroup = 8;  // parts whose loads are issued together
  const int c4 = threadIdx.x % kLanesPerRow;
  const int n = p.n_parts;
  // grid-stride over rows: the grid is capped on the host, so any row count fits one launch
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow; row < p.rows;
       row += (int64_t)gridDim.x * kRowsPerBlock) {
    // pass 1: M = max_i LSE_i
    float M = -INFINITY;
    for (int i0 = 0; i0 < n; i0 += kGroup) {
      float li[kGroup];
#pragma unroll
      for (int k = 0; k < kGroup; ++k) li[k] = i0 + k < n ? p.lse_parts[i0 + k][row] : -INFINITY;
#pragma unroll
      for (int k = 0; k < kGroup; ++k) M = fmaxf(M, li[k]);
    }
    // pass 2: weights, then the O slices of a group's parts that saw a key, all loads in flight
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f;
    if (M != -INFINITY) {
      for (int i0 = 0; i0 < n; i0 += kGroup) {
        float w[kGroup];
#pragma unroll
        for (int k = 0; k < kGroup; ++k) {
          const float li = i0 + k < n ? p.lse_parts[i0 + k][row] : -INFINITY;
          w[k] = li == -INFINITY ? 0.f : expf(li - M);
        }
        float4 o[kGroup];
#pragma unroll
        for (int k = 0; k < kGroup; ++k)
          if (w[k] != 0.f) {
            const f32x4v t = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p.o_parts[i0 + k] + row * D + c4 * 4));
            o[k] = make_float4(t[0], t[1], t[2], t[3]);
          } else {
            o[k] = make_float4(0.f, 0.f, 0.f, 0.f);
          }
#pragma unroll
        for (int k = 0; k < kGroup; ++k) {
          wsum += w[k];
          acc.x = fmaf(w[k], o[k].x, acc.x);
          acc.y = fmaf(w[k], o[k].y, acc.y);
          acc.z = fmaf(w[k], o[k].z, acc.z);
          acc.w = fmaf(w[k], o[k].w, acc.w);
        }
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    acc.x *= inv;
    acc.y *= inv;
    acc.z *= inv;
    acc.w *= inv;
    if (OUT_BF16) {
      __bf16* out = static_cast<__bf16*>(p.o_out) + row * D + c4 * 4;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 v = {(__bf16)acc.x, (__bf16)acc.y, (__bf16)acc.z, (__bf16)acc.w};
      __builtin_nontemporal_store(v, reinterpret_cast<bf16x4*>(out));
    } else {
      const f32x4v t = {acc.x, acc.y, acc.z, acc.w};
      __builtin_nontemporal_store(t, reinterpret_cast<f32x4v*>(static_cast<float*>(p.o_out) + row * D + c4 * 4));
    }
    if (c4 == 0 && p.lse_out) p.lse_out[row] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
  }
}

// An empty running result: O = 0 and LSE = -inf for `rows` rows of d_h values (folding a partial
// into it leaves the partial unchanged). A kernel rather than a memset, so that the fill can sit
// in a captured graph.
__global__ __launch_bounds__(256) void fill_running_kernel(float4* o, int64_t n4, float* lse, int64_t rows) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows; i += (int64_t)gridDim.x * 256)
    lse[i] = -INFINITY;
}

hipError_t launch_fill_running(float* o, float* lse, int64_t rows, int d_h, hipStream_t stream) {
  const int64_t n4 = rows * d_h / 4;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_running_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0,
                     stream, reinterpret_cast<float4*>(o), n4, lse, rows);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const int rows_per_block = 256 / (p.d_h / 4);
  // at most 64K workgroups (256 per CU); larger merges loop inside the kernel
  const int64_t blocks = std::min<int64_t>((p.rows + rows_per_block - 1) / rows_per_block, 65536);
  const dim3 grid((unsigned)blocks), block(256);
  if (p.d_h == 64) {
    if (p.out_bf16)
      hipLaunchKernelGGL((merge_kernel<64, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((merge_kernel<64, false>), grid, block, 0, stream, p);
  } else {
    if (p.out_bf16)
      hipLaunchKernelGGL((merge_kernel<128, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((merge_kernel<128, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace cpk
