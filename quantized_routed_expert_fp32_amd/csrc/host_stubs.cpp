// Device-side entry points of the library for the host-only sanitizer
// build (build.build_host_sanitized): the packer, the layout arithmetic and
// the C ABI's validation are compiled with AddressSanitizer and
// UndefinedBehaviorSanitizer, and every enqueue is replaced by a refusal, so
// the host tests exercise all host code paths without a GPU or GPU code.
#include <hip/hip_runtime.h>

#include "moe_host.h"
#include "moe_launch.h"

namespace moe {

hipError_t launch_route(int, int, const RouteArgs&, hipStream_t, hipEvent_t*) { return hipErrorNoDevice; }
hipError_t launch_decode(int, int, const DecodeArgs&, hipStream_t, hipEvent_t*) { return hipErrorNoDevice; }
hipError_t launch_grouped(int, int, const GroupedArgs&, hipStream_t, hipEvent_t*) { return hipErrorNoDevice; }
hipError_t launch_grp_sort(const GroupedArgs&, hipStream_t, hipEvent_t*) { return hipErrorNoDevice; }
hipError_t launch_route_exact(int, int, const RouteArgs&, hipStream_t, hipEvent_t*) { return hipErrorNoDevice; }
hipError_t launch_exact_experts(int, int, const DecodeArgs&, hipStream_t, hipEvent_t*) { return hipErrorNoDevice; }

}  // namespace moe

extern "C" int moe_forward_windows_noalloc(const moe_layer*, const void*, int, const float*, int32_t*, float*,
                                           float*, float*, void*) {
  moe::set_error("moe_forward_windows_noalloc: not in the host-only sanitizer build");
  return MOE_EHIP;
}
