#include "hipsa_internal.h"
namespace hipsa {
hipError_t launch_mask_prefill(const MaskArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_prefill(const AttnArgs &, hipStream_t) { return hipErrorNotSupported; }
}
