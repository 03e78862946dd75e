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
  bool glu;                // N columns = gate | up halves; out = SiLU(gate) * up, [M][N/2]
  const void* xscale;      // AWQ: S^-1 [K] in the activation dtype (x' = RN(x * s_inv)), or NULL
  void* workspace;         // scratch for split-K partial tiles (no state between calls)
  size_t workspace_bytes;
  hipStream_t stream;
};

// launch geometry of the decode kernel (at most 16 rows of x per launch)
struct DecodeConfig {
  int KC, NT;        // k-blocks per strip, 16-column strips
  int rows, MT;      // rows of x, 16-row MFMA tiles
  int SW;            // strips per workgroup tile (1, 2 or 4)
  int tiles;         // tiles of SW strips
  int grid;          // workgroups (persistent: fewer than tiles, each looping over tiles)
  bool persist;      // persistent workgroups, x staged once for all their tiles
  bool glu;          // SwiGLU: tiles pair a gate strip with its up strip
  int W;             // waves per workgroup; wave w streams k-blocks [w*slice, (w+1)*slice)
  int slice;
  int xstride;       // LDS row stride of x (halves)
  int xslice;        // LDS halves per wave for its slice of x
  bool x_in_lds;     // activations staged in LDS
  size_t lds_bytes;  // dynamic LDS per workgroup
  size_t workspace_bytes;
};
// extra_lds: bytes a launch stages after the activations (NF4: its level-pair table)
DecodeConfig decode_config(int M, int K, int N, int group_size, bool glu, size_t extra_lds = 0);

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Compute units of the current device (cached per device; 256 if it cannot be read).
inline int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    __atomic_store_n(&cached[dev], v, __ATOMIC_RELAXED);
  }
  return v;
}
inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

hipError_t launch_pack(const uint32_t* qweight, int K, int N, uint32_t* packed, hipStream_t s);
hipError_t launch_dequant(const GemmArgs& a);  // writes W_hat [K][N] into a.out (act dtype)
hipError_t launch_decode(const GemmArgs& a);   // M <= 16 (more rows: several launches)
hipError_t launch_tiled(const GemmArgs& a);    // M > 16
size_t tiled_workspace_bytes(int M, int K, int N);  // split-K partials (0 when K is not split)
hipError_t launch_skinny(const GemmArgs& a);   // 17..64 rows: K split across the waves
const char* skinny_name(int M, int K, int N);
size_t skinny_awq_workspace_bytes(int M, int K, int N);
size_t decode_awq_workspace_bytes(int M, int K, int N, int group_size);  // M <= 16
size_t tiled_awq_workspace_bytes(int M, int K, int N);
// W4A8: per-token INT8 quantization of x (xq [M][K], sx [M], and with perm the packed nibble
// order of each group of eight plus the row code sums xsum [M]); the GEMM with per-channel
// weight scales in a.scales [N]; its workspace (xq, sx, xsum)
hipError_t launch_quantize_act(const void* x, int M, int K, int act, bool perm, int8_t* xq,
                               float* sx, int* xsum, hipStream_t s);
hipError_t launch_w4a8(const GemmArgs& a);
size_t w4a8_workspace_bytes(int M, int K, int N);
const char* w4a8_name(int M, int K, int N);
// x'[rows][K] = RN(x * s_inv[k]) (act dtype) into out, 16-byte aligned, K % 8 == 0
hipError_t launch_awq_scale(const void* x, const void* s_inv, int rows, int K, int act, void* out,
                            hipStream_t stream);
// streaming read of bytes (a multiple of 16) from buf, folded into sink[kProbeSinkWords]
// (measurement)
constexpr int kProbeSinkWords = 256;
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
const char* decode_name(int M, int K, int N, int group_size, int act);
const char* tiled_name(int M, int K, int N, int group_size);
bool tiled_supported(const GemmArgs& a);

}  // namespace w4a16
