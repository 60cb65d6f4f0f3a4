// Kernels of the Lion step for every supported state format.
#include "forge_device.h"

namespace forge {
FORGE_LION_LIST(FORGE_INSTANTIATE)
}  // namespace forge
