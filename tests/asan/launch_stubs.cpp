// launch_stubs.cpp -- stand-ins for the device launchers, for the host
// sanitizer build of the argument-validation layer (api.cpp, trace.cpp,
// sizes.cpp).  That build runs the C ABI's error paths, which return before
// any launch; a call that got here anyway reports hipErrorNoDevice, so a
// validation hole shows up as ATTN_ERR_HIP in the tests instead of a launch.
#include "launch.hpp"

namespace lcattn {

hipError_t launch_transpose_rows_batch(const TransposeJob*, int, unsigned, bool, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_sum_replicas(const void*, bool, uint16_t*, long long, long long, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_attn_fwd(const FwdArgs&, int, int, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_fwd_group(const FwdArgs*, int, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_fwd_group_split(const FwdArgs*, float* const*, int, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_attn_fwd_splitkv(const FwdArgs&, int, int, int, float*, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_partial_merge(const void*, bool, const float*, int, uint16_t*, float*, long long, int,
                                hipStream_t, const MergeSplits*) {
  return hipErrorNoDevice;
}
hipError_t launch_merge_into(const float*, const float*, int, const MergeSplits&, float*, float*, bool, uint16_t*,
                             long long, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_attn_bwd(const BwdArgs&, int, int, hipStream_t, bool, bool) { return hipErrorNoDevice; }
hipError_t launch_attn_bwd_group(const BwdArgs*, int, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bwd_delta(const uint16_t*, const uint16_t*, float*, long long, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t noalloc_scratch(hipStream_t, void**) { return hipErrorNoDevice; }

}  // namespace lcattn
