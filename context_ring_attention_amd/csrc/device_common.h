// device_common.h -- small device helpers shared by the gfx950 attention kernels.
//
// Pages cited: [CPEP] "Context Parallelism과 Expert Parallelism: Long Context와 MoE를 쪼개는 두
// 축"; [CPMTI] "Context Parallelism for Scalable Million-Token Inference" (paper review).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "cp_internal.h"

namespace cpk {

constexpr float kLn2 = 0.69314718055994530942f;

// Workgroup tile -> (Q segment, tile index inside the segment). Slots are visited in the order
// the host chose; inside a slot the first workgroup takes the segment's last tile.
__device__ inline void locate_tile(const AttnParams& p, int block, int& seg, int& tile) {
  int slot = 0;
  while (slot + 1 < p.n_q_segs && p.tile_prefix[slot + 1] <= block) ++slot;
  seg = p.order[slot];
  const int n_tiles = p.tile_prefix[slot + 1] - p.tile_prefix[slot];
  tile = n_tiles - 1 - (block - p.tile_prefix[slot]);
}

// Keys of KV run `ks` visible to a query at position qpos of the same sequence: with the causal
// mask a query sees keys at positions <= its own ([CPEP §5.1]); they form a prefix of the run.
__device__ inline int visible_prefix(const Seg& ks, int qpos, int causal) {
  if (!causal) return ks.len;
  int n = qpos - ks.pos + 1;
  return n < 0 ? 0 : (n > ks.len ? ks.len : n);
}

// Merge of a running partial (lse_prev) with a new one (lse_new): the same LSE-weighted combine
// as the merge kernel, for two parts. Returns the weights of the two parts' outputs and the
// merged LSE; if neither part saw a key both weights are 0 and the LSE stays -inf.
__device__ inline void running_merge_weights(float lse_prev, float lse_new, float& w_prev,
                                             float& w_new, float& lse_out) {
  const float M = fmaxf(lse_prev, lse_new);
  if (M == -INFINITY) {
    w_prev = 0.f;
    w_new = 0.f;
    lse_out = -INFINITY;
    return;
  }
  const float a = expf(lse_prev - M);
  const float b = expf(lse_new - M);
  const float s = a + b;
  w_prev = a / s;
  w_new = b / s;
  lse_out = M + logf(s);
}

// max(a, b) as one v_max_f32 (the compiler's fmaxf also quiets each operand first, two more VALU
// instructions on the row max's critical path; scores are never signalling NaNs). Device pass
// only, like every AMDGPU-constraint asm here.
__device__ inline float vmax(float a, float b) {
#if defined(__HIP_DEVICE_COMPILE__)
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
#else
  return a > b ? a : b;
#endif
}

// Max of x over lanes l and l ^ 32 (the two half-waves), without going through LDS: swapping
// the upper half of one copy with the lower half of another leaves each lane holding both values.
// Each result is copied out of the returned vector before its bit cast: a bit cast of a vector
// element expression reads element 0 whatever the index (seen with this compiler), which would
// leave each lane with one half-wave's value only (harmless while scores are close, an exp2
// overflow once they spread over more than 128 base-2 units).
__device__ inline float max_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t r0 = sw[0], r1 = sw[1];
  return vmax(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

// Max of x over lanes l and l ^ 16 (odd and even 16-lane rows), without going through LDS.
__device__ inline float max_xor16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t r0 = sw[0], r1 = sw[1];
  return vmax(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

}  // namespace cpk
