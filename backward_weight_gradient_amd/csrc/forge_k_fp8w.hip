// Kernels of the fused step with an E4M3 weight (AdamW, Lion, SGD-momentum).
#include "forge_device.h"

namespace forge {
FORGE_FP8W_LIST(FORGE_INSTANTIATE_FP8W)
}  // namespace forge
