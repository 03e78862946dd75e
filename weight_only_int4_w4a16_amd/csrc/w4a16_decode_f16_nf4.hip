// Instantiations of the decode kernel for f16 activations, nf4 weights.
#include "w4a16_decode_kernel.hpp"

namespace w4a16 {
template hipError_t decode_dispatch<ACT_F16, FMT_NF4>(const DecodeParams&, const DecodeConfig&,
                                                          hipStream_t);
}  // namespace w4a16
