// Kernels of the RMSprop and AdaGrad steps (second moment only) and of plain
// SGD (no state), for every supported state format.
#include "forge_device.h"

namespace forge {
FORGE_SECOND_MOMENT_LIST(FORGE_INSTANTIATE)
}  // namespace forge
