// Placeholder launchers for the GeLU MLP until its kernels land; fab_plan
// rejects GeLU problems while mlp_available() is false.
#include "fab_internal.h"
namespace fab {
bool mlp_available() { return false; }
size_t mlp_fwd_workspace(int, int, int, int, int* splits) { *splits = 1; return 0; }
size_t mlp_bwd_workspace(int, int, int, int) { return 0; }
hipError_t launch_mlp_fwd_bf16(const MlpArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_mlp_bwd_bf16(const MlpArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace fab
