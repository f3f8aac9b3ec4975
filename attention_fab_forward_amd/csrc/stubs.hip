// Placeholder launchers for variants not built yet; fab_plan rejects them.
#include "fab_internal.h"
namespace fab {
hipError_t launch_attn_bwd_bf16(const AttnArgs&, int, hipStream_t) { return hipErrorNotSupported; }
bool mlp_available() { return false; }
size_t mlp_fwd_workspace(int, int, int, int, int* splits) { *splits = 1; return 0; }
size_t mlp_bwd_workspace(int, int, int, int) { return 0; }
hipError_t launch_mlp_fwd_bf16(const MlpArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_mlp_bwd_bf16(const MlpArgs&, hipStream_t) { return hipErrorNotSupported; }
}
