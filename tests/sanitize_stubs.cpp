// Launch functions for a host-only build of the ABI (api.hip and
// scheduler.cpp without the kernel files), used by tests/test_sanitizers.py
// to run the argument validation and the scheduler under AddressSanitizer
// and UndefinedBehaviorSanitizer on the CPU.  Nothing here is reached by the
// checks that run (they fail validation before any launch); if a call did get
// this far it would report hipErrorNotSupported.
#include <hip/hip_runtime_api.h>

#include "internal.hpp"

namespace spear {
hipError_t launch_projection(const Shape&, const LayerArgs&, const WsPtrs&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_decode(const Shape&, const LayerArgs&, const WsPtrs&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_prefill(const Shape&, const LayerArgs&, const WsPtrs&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_serq_operand(const Shape&, const LayerArgs&, const WsPtrs&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_quantize(int, int, int, bool, bool, const float*, uint32_t*, uint16_t*, uint32_t*,
                           hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_dequant(int, int, int, const uint32_t*, const uint16_t*, const uint32_t*, float*,
                          hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t static_scratch(void**, hipStream_t) { return hipErrorNotSupported; }
}  // namespace spear
