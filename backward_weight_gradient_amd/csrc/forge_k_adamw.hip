// Kernels of the AdamW step for every supported state format.
#include "forge_device.h"

namespace forge {
FORGE_ADAMW_LIST(FORGE_INSTANTIATE)
}  // namespace forge
