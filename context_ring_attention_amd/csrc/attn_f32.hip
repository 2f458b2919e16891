// attn_f32.hip -- partial attention for fp32 inputs, fp32 arithmetic throughout.
//
// One thread per query row (token, head). The row walks the keys it may see in every KV run of
// its sequence and keeps an online softmax: running max m, running sum l and the weighted sum
// of values, rescaled whenever the max grows ([CPEP §4.1]: block-wise attention with online
// softmax gives exact attention without the [T, T] score matrix). Head h reads KV head
// h / (N_H / N_KV) ([CPEP §8.2]); the causal mask keeps key positions <= the query position
// ([CPEP §5.1]). This path serves small fp32 workloads where exactness to ~1e-6 matters more
// than speed; bf16 inputs take the MFMA kernel instead.
//
// Pages cited: [CPEP] "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두
// 축"; [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (paper review).
#include "device_common.h"

namespace cpk {

template <int D>
__global__ __launch_bounds__(kTileRowsF32) void attn_f32_kernel(const AttnParams p) {
  int seg, tile;
  locate_tile(p, blockIdx.x, seg, tile);
  const int g = blockIdx.y;
  const Seg qs = p.qs[seg];
  const int pr = p.q_prob[seg];  // problem of this tile
  const int rows = qs.len * p.group;
  const int r = tile * kTileRowsF32 + (int)threadIdx.x;
  if (r >= rows) return;

  const int tok = r / p.group;
  const int head = g * p.group + r % p.group;
  const int64_t qrow = (int64_t)(qs.loc + tok) * p.n_h + head;
  const int qpos = qs.pos + tok;
  const float* __restrict__ Q = static_cast<const float*>(p.q[pr]);
  const float* __restrict__ K = static_cast<const float*>(p.k[pr]);
  const float* __restrict__ V = static_cast<const float*>(p.v[pr]);

  float qv[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const float4 x = *reinterpret_cast<const float4*>(Q + qrow * D + d);
    qv[d] = x.x * p.scale;
    qv[d + 1] = x.y * p.scale;
    qv[d + 2] = x.z * p.scale;
    qv[d + 3] = x.w * p.scale;
  }
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int j = p.kv_lo[pr]; j < p.kv_hi[pr]; ++j) {
    const Seg ks = p.ks[j];
    if (ks.seq != qs.seq) continue;
    const int n = visible_prefix(ks, qpos, p.causal);
    for (int key = 0; key < n; ++key) {
      const int64_t krow = ((int64_t)(ks.loc + key) * p.n_kv + g) * D;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const float4 kk = *reinterpret_cast<const float4*>(K + krow + d);
        s = fmaf(qv[d], kk.x, s);
        s = fmaf(qv[d + 1], kk.y, s);
        s = fmaf(qv[d + 2], kk.z, s);
        s = fmaf(qv[d + 3], kk.w, s);
      }
      if (s > m) {
        const float alpha = expf(m - s);  // m = -inf -> 0
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= alpha;
        m = s;
      }
      const float w = expf(s - m);
      l += w;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const float4 vv = *reinterpret_cast<const float4*>(V + krow + d);
        acc[d] = fmaf(w, vv.x, acc[d]);
        acc[d + 1] = fmaf(w, vv.y, acc[d + 1]);
        acc[d + 2] = fmaf(w, vv.z, acc[d + 2]);
        acc[d + 3] = fmaf(w, vv.w, acc[d + 3]);
      }
    }
  }

  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse_new = l > 0.f ? m + logf(l) : -INFINITY;
  float* orow = p.o[pr] + qrow * D;
  if (p.accumulate) {
    float wp, wn, lse_out;
    running_merge_weights(p.lse[pr][qrow], lse_new, wp, wn, lse_out);
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = wp * orow[d] + wn * (acc[d] * inv);
    p.lse[pr][qrow] = lse_out;
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
    p.lse[pr][qrow] = lse_new;
  }
}

hipError_t launch_attn_f32(const AttnParams& p, int d_h, hipStream_t stream) {
  const dim3 grid(p.total_tiles, p.n_kv);
  const dim3 block(kTileRowsF32);
  if (d_h == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace cpk
