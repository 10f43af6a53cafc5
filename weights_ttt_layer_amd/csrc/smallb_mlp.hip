// smallb_mlp.hip -- placeholder until the TTT-MLP path lands.
#include "kernels.h"
namespace ttt {
hipError_t launch_smallb_mlp(const MlpArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ttt
