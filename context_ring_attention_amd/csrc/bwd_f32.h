// bwd_f32.h -- launcher of the fp32-input backward kernels (attn_bwd.hip). The tile plan of its
// BwdParams uses 64 query rows per dQ workgroup and 64 keys per dK/dV workgroup.
#pragma once

#include "cp_internal.h"

namespace cpk {
constexpr int kBwdF32Rows = 64;
constexpr int kBwdF32Keys = 64;
hipError_t launch_bwd_f32(const BwdParams& p, int d_h, hipStream_t stream);
}  // namespace cpk
