// bf16 MFMA tree-masked attention kernel (gfx950) -- placeholder until the
// MFMA path lands; the planner never selects it yet.
#include "ta_device.h"

namespace ta {
hipError_t launch_attn_mfma(const AttnParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ta
