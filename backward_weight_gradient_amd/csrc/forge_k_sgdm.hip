// Kernels of the SGD with momentum step for every supported state format.
#include "forge_device.h"

namespace forge {
FORGE_SGDM_LIST(FORGE_INSTANTIATE)
}  // namespace forge
