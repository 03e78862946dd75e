// The batched W4A16 GEMM kernel instantiated for the MedTile workgroup tile (every activation
// type, group size and format; one strip pair per wave, so no SwiGLU epilogue).
#include "w4a16_tiled_kernel.hpp"

namespace w4a16 {
namespace tiled {
W4A16_TILED_INSTANTIATE(MedTile)
}  // namespace tiled
}  // namespace w4a16
