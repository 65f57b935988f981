// Kernel launchers for the host-only sanitizer build of libkvq: the same
// signatures as the kernel sources' launchers, each reporting that no device
// is present. Linked only into _build/asan/libkvq_asan.so, which exercises
// the host-side C ABI (validation, layout, split planning) and never runs a
// kernel.
#include "kvq_internal.h"

hipError_t kvq_static_workspace(hipStream_t, void**) { return hipErrorNoDevice; }
hipError_t kvq_launch_extend(const ExtendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t kvq_launch_amax(const uint16_t*, int64_t, const uint16_t*, int64_t, unsigned*, float, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t kvq_launch_store(const kvq_cache*, const uint16_t*, const uint16_t*, const int64_t*, int32_t, const float*,
                            const float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t kvq_launch_decode_gqa(const kvq_cache*, const GqaDecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t kvq_launch_decode_mla(const kvq_cache*, const MlaDecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t kvq_launch_combine(const CombineArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t kvq_launch_dequant_prev(const kvq_cache*, const int32_t*, int32_t, const float*, const float*, const float*,
                                   uint8_t*, uint8_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t kvq_launch_amax_channels(const uint16_t*, int64_t, const uint16_t*, int64_t, int, unsigned*, float, float*,
                                    hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t kvq_launch_amax_heads(const uint16_t*, int64_t, const uint16_t*, int64_t, int, int, unsigned*, float, float*,
                                 hipStream_t) {
  return hipErrorNoDevice;
}
