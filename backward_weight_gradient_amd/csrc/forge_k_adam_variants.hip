// Kernels of the NAdam and RAdam steps for every supported state format.
#include "forge_device.h"

namespace forge {
FORGE_ADAM_VARIANT_LIST(FORGE_INSTANTIATE)
}  // namespace forge
