// attn_bwd.h -- launchers of the backward kernels (attn_bwd.hip) beyond launch_bwd and
// launch_bwd_delta.
#pragma once

#include "cp_internal.h"

namespace cpk {

// fp32 inputs: the tile plan of their BwdParams uses 64 query rows per dQ workgroup and 64 keys
// per dK/dV workgroup.
constexpr int kBwdF32Rows = 64;
constexpr int kBwdF32Keys = 64;
hipError_t launch_bwd_f32(const BwdParams& p, int d_h, hipStream_t stream);

// bf16 inputs with the dK/dV work of every key tile split over `parts` workgroups: the blocks of
// query rows that see the tile are divided into `parts` equal runs, part c of tile t (in the
// order of the plan) writes its unscaled dK and its dV to workspace slot
// (kv_head * kv_tiles + t) * parts + c ([128 keys][d_h] fp32 each, dK first), and a reduce kernel
// adds scale * sum(dK parts) and sum(dV parts), in part order, into dk and dv. parts == 1: no
// workspace, every workgroup adds its tile's sums into dk and dv itself.
struct BwdSplit {
  float* ws;
  int32_t parts;
};
// The split aims at this many dK/dV workgroups per launch (one runs per CU at a time), so the
// plan uses at most 2 * kBwdSplitTarget workspace slots.
constexpr int kBwdSplitTarget = 1024;
constexpr int kBwdMaxParts = 16;
constexpr int kBwdMaxSlots = 2 * kBwdSplitTarget;
inline size_t bwd_slot_bytes(int d_h) { return (size_t)kBwdKeys * d_h * sizeof(float) * 2; }
hipError_t launch_bwd_split(const BwdParams& p, const BwdSplit& sp, int d_h, hipStream_t stream);

}  // namespace cpk
