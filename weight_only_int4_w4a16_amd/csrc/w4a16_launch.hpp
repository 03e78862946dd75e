// w4a16_launch.hpp - internal launchers behind the C ABI (not part of the public header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

enum ActKind { ACT_F16 = 0, ACT_BF16 = 1 };

struct GemmArgs {
  const void* x;
  int M, K, N;
  int act;                 // 0 = fp16, 1 = bf16
  const uint32_t* packed;
  const void* scales;      // affine: act [K/g][N]; NF4: fp16 absmax [K/g][N]
  const uint32_t* qzeros;  // affine only; NULL -> zero 8
  const uint16_t* codebook;// NF4 only
  bool nf4;
  int group_size;
  void* out;
  int out_dtype;           // 0 fp16, 1 bf16, 2 fp32
  hipStream_t stream;
};

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

hipError_t launch_pack(const uint32_t* qweight, int K, int N, uint32_t* packed, hipStream_t s);
hipError_t launch_dequant(const GemmArgs& a);  // writes W_hat [K][N] into a.out (act dtype)
hipError_t launch_skinny(const GemmArgs& a);   // M <= 64
hipError_t launch_tiled(const GemmArgs& a);    // M > 64
const char* skinny_name(int M);
const char* tiled_name(int M, int K, int N);
bool tiled_supported(const GemmArgs& a);

}  // namespace w4a16
