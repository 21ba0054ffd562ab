// Grouped (prompt-chunk) path: placeholder until the MFMA kernels land.
#include "moe_kernels.h"
#include "moe_launch.h"

namespace moe {
hipError_t launch_grouped(int, int, const GroupedArgs&, hipStream_t, hipEvent_t*) { return hipErrorNotSupported; }
}  // namespace moe
