// TTT-MLP forward scan (gfx950).  Kernel under construction.
#include "ttt_device.h"
#include "ttt_launch.h"

namespace ttt {
hipError_t launch_mlp(const MlpArgs&, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ttt
