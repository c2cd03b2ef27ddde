// bf16 MFMA grouped-attention kernels (placeholder until the MFMA path lands).
#include "internal.h"

namespace monarch {
bool flash_supported(const GroupedArgs&) { return false; }
hipError_t launch_flash(const GroupedArgs&, hipStream_t) { return hipErrorInvalidValue; }
bool small_supported(const GroupedArgs&) { return false; }
hipError_t launch_small(const GroupedArgs&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace monarch
