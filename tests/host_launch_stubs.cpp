// host_launch_stubs.cpp -- stand-ins for the kernel launchers, for a host-only build of the C ABI
// (api.cpp) under AddressSanitizer. The checks that use this build exercise validation and the
// host-only entry points, which return before any launch; reaching a stub is itself an error.
#include <cstdio>
#include <cstdlib>

#include "attn_bwd.h"
#include "cp_internal.h"

namespace cpk {

static hipError_t unexpected(const char* what) {
  std::fprintf(stderr, "host-only build: %s was reached\n", what);
  std::abort();
}

hipError_t launch_attn_f32(const AttnParams&, int, hipStream_t) { return unexpected("launch_attn_f32"); }
hipError_t launch_attn_bf16(const AttnParams&, int, hipStream_t) { return unexpected("launch_attn_bf16"); }
hipError_t launch_merge(const MergeParams&, hipStream_t) { return unexpected("launch_merge"); }
hipError_t launch_fill_running(float*, float*, int64_t, int, hipStream_t) {
  return unexpected("launch_fill_running");
}
hipError_t launch_decode(const DecodeParams&, int, hipStream_t) { return unexpected("launch_decode"); }
hipError_t decode_scratch(void**) { return unexpected("decode_scratch"); }
hipError_t launch_bwd(const BwdParams&, int, hipStream_t) { return unexpected("launch_bwd"); }
hipError_t launch_bwd_f32(const BwdParams&, int, hipStream_t) { return unexpected("launch_bwd_f32"); }
hipError_t launch_bwd_split(const BwdParams&, const BwdSplit&, int, hipStream_t) {
  return unexpected("launch_bwd_split");
}
hipError_t launch_bwd_delta(const float*, const void*, bool, int64_t, int, float*, hipStream_t) {
  return unexpected("launch_bwd_delta");
}

}  // namespace cpk
