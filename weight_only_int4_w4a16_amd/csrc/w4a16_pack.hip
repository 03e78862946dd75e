// w4a16_pack.hip - load-time re-layout of the canonical INT4 weight and the dequantization
// test hook. "INT4 and Low-Bit Inference", section 5 (Marlin's tricks): weights are
// re-ordered once at load so run-time unpacking is branch-free and reads coalesce.
#include "w4a16_device.hpp"
#include "w4a16_launch.hpp"

namespace w4a16 {

// One thread per (strip nt, k-block kc, lane): gathers the four canonical words the lane
// will read at run time (each is already eight consecutive k of one column), permutes
// their nibbles and writes them as one 16-byte store.
__global__ __launch_bounds__(256) void pack_kernel(const uint32_t* __restrict__ qweight, int K,
                                                   int N, int KC, u4_t* __restrict__ packed,
                                                   size_t total) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int lane = (int)(t & 63);
  const size_t blk = t >> 6;
  const int kc = (int)(blk % KC);
  const int nt = (int)(blk / KC);
  const int n = nt * 16 + (lane & 15);
  u4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k0 = kc * 128 + j * 32 + (lane >> 4) * 8;
    o[j] = (k0 < K) ? permute_nibbles(qweight[(size_t)(k0 >> 3) * N + n]) : 0u;
  }
  packed[t] = o;
}

hipError_t launch_pack(const uint32_t* qweight, int K, int N, uint32_t* packed, hipStream_t s) {
  const int KC = ceil_div(K, 128);
  const size_t total = (size_t)(N / 16) * KC * 64;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, s, qweight, K, N, KC,
                     reinterpret_cast<u4_t*>(packed), total);
  return hipGetLastError();
}

// Dequantization test hook: one thread per (strip, k-block, lane), each word expanded with
// the same device routine the GEMM kernels that form W_hat use, written to W_hat[K][N].
template <int ACT, bool NF4>
__global__ __launch_bounds__(256) void dequant_kernel(const u4_t* __restrict__ packed,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint32_t* __restrict__ qzeros,
                                                      const uint16_t* __restrict__ codebook,
                                                      int K, int N, int KC, int gs,
                                                      uint16_t* __restrict__ out, size_t total) {
  __shared__ uint32_t ptab[kNf4PairEntries];  // NF4: the level-pair table of the GEMM kernels
  if (NF4) {
    nf4_pair_table_fill(ptab, codebook);
    __syncthreads();
  }
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int lane = (int)(t & 63);
  const size_t blk = t >> 6;
  const int kc = (int)(blk % KC);
  const int nt = (int)(blk / KC);
  const int n = nt * 16 + (lane & 15);
  const u4_t b = packed[t];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k0 = kc * 128 + j * 32 + (lane >> 4) * 8;
    if (k0 >= K) break;
    const int g = k0 / gs;
    const uint32_t sbits = scales[(size_t)g * N + n];
    // the 8 weights as four 32-bit words (element i in the low/high half of word i/2);
    // whole-vector bit casts only
    u4_t d;
    if (NF4) {
      if (ACT == ACT_F16) {
        d = __builtin_bit_cast(u4_t, dequant_word_nf4_f16_tab(b[j], ptab, as_h2(sbits * 0x00010001u)));
      } else {
        const float a = (float)__builtin_bit_cast(_Float16, (uint16_t)sbits);
        d = __builtin_bit_cast(u4_t, dequant_word_nf4_bf16_tab(b[j], ptab, a));
      }
    } else {
      const uint32_t z = qzeros ? (qzeros[(size_t)g * (N >> 3) + (n >> 3)] >> (4 * (n & 7))) & 0xFu
                                : 8u;
      if (ACT == ACT_F16) {
        d = __builtin_bit_cast(u4_t, dequant_word_f16(b[j], make_zero_f16(z), as_h2(sbits * 0x00010001u)));
      } else {
        const float s = __builtin_bit_cast(float, sbits << 16);
        d = __builtin_bit_cast(u4_t, dequant_word_bf16(b[j], make_zero_f32(z, s)));
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t word = d[i >> 1];
      out[(size_t)(k0 + i) * N + n] = (uint16_t)((i & 1) ? (word >> 16) : (word & 0xFFFFu));
    }
  }
}

hipError_t launch_dequant(const GemmArgs& a) {
  const int KC = ceil_div(a.K, 128);
  const size_t total = (size_t)(a.N / 16) * KC * 64;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  const u4_t* p = reinterpret_cast<const u4_t*>(a.packed);
  const uint16_t* s = static_cast<const uint16_t*>(a.scales);
  uint16_t* o = static_cast<uint16_t*>(a.out);
#define W4A16_DQ(ACTV, NF4V)                                                                  \
  hipLaunchKernelGGL((dequant_kernel<ACTV, NF4V>), dim3(blocks), dim3(256), 0, a.stream, p, s, \
                     a.qzeros, a.codebook, a.K, a.N, KC, a.group_size, o, total)
  if (a.nf4) {
    if (a.act == ACT_F16) W4A16_DQ(ACT_F16, true); else W4A16_DQ(ACT_BF16, true);
  } else {
    if (a.act == ACT_F16) W4A16_DQ(ACT_F16, false); else W4A16_DQ(ACT_BF16, false);
  }
#undef W4A16_DQ
  return hipGetLastError();
}

}  // namespace w4a16
