// The batched W4A16 GEMM kernel instantiated for the SmallTileDeep workgroup tile (every activation
// type, group size and format, with and without the SwiGLU epilogue).
#include "w4a16_tiled_kernel.hpp"

namespace w4a16 {
namespace tiled {
W4A16_TILED_INSTANTIATE(SmallTileDeep)
}  // namespace tiled
}  // namespace w4a16
