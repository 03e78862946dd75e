// Instantiations of the decode kernel for bf16 activations, asym weights.
#include "w4a16_decode_kernel.hpp"

namespace w4a16 {
template hipError_t decode_dispatch<ACT_BF16, FMT_ASYM>(const DecodeParams&, const DecodeConfig&,
                                                          hipStream_t);
}  // namespace w4a16
