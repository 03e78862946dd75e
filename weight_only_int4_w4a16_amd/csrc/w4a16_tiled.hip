// w4a16_tiled.hip - batched / prefill W4A16 GEMM (M > 64), LDS-staged MFMA tiles.
#include "w4a16_device.hpp"
#include "w4a16_launch.hpp"

namespace w4a16 {

bool tiled_supported(const GemmArgs&) { return false; }
const char* tiled_name(int, int, int) { return "w4a16_tiled_unavailable"; }
hipError_t launch_tiled(const GemmArgs&) { return hipErrorNotSupported; }
size_t tiled_workspace_bytes(int, int, int) { return 0; }

}  // namespace w4a16
