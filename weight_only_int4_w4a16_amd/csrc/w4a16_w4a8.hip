// w4a16_w4a8.hip - W4A8: INT4 weights with per-token INT8 activations on the integer MFMA.
//
// "INT4 LLMs: What 4-Bit Quantization Means…", weight-only section: weights in [-8, 7] are
// unpacked to INT8, an INT8 x INT8 product runs, and the result is dequantized with the input
// and per-channel scales; "INT8 vs INT4 Quantization, in depth", section "Two regimes": past
// the crossover batch the math rate decides, and the INT8 path has twice the FP16 rate.
//
//   y[m, n] = sx[m] * sw[n] * sum_k xq[m, k] * (u[k, n] - 8)
//
// with xq the per-token INT8 activations (sx = max|x| / 127, xq = rint(x / sx), both in fp32),
// u the stored offset-binary 4-bit code and sw the per-output-channel scale.
//
// Two kernels. The first quantizes x, one workgroup per row, and also writes the row's code
// sum; the second is the GEMM on v_mfma_i32_32x32x32_i8 (twice the operations per cycle of the
// 16-bit MFMA). The weight codes go into the MFMA as the unsigned integers u = 0..15, and the
// epilogue takes 8 * sum_k xq[m, k] off each exact integer sum, so a word of eight codes
// becomes two MFMA operand words with one AND and one shift-AND. Those two words hold the
// codes in the packed layout's nibble order (k = 0, 4, 1, 5, 2, 6, 3, 7 within each group of
// eight); the quantizer writes xq in the same order, so A and B agree without any byte
// shuffling, and the integer sum is unchanged by the order.
//
// Tiling follows the batched W4A16 kernel: 128 x 512 (eight waves) or 64 x 256 (four waves)
// output tiles, xq tile double-buffered in LDS, each wave owning 64 columns (two 32-column
// pairs of strips) over all the tile's rows. In the 32x32x32 operands lane l holds row / column
// l % 32 and k = 16 (l / 32) .. +16 of a 32-k step; for the B operand those 16 codes are word
// s of the packed block's chunks 32 (l / 32) + l % 16 and that + 16, which lane l loads itself.
// When the output tiles leave compute units idle, K is split into 2 or 4 slices whose exact
// int32 sums a third small kernel adds before the same epilogue (the result does not depend on
// the split).
#include <type_traits>

#include "w4a16_device.hpp"
#include "w4a16_launch.hpp"

namespace w4a16 {

namespace {

typedef int i4v_t __attribute__((ext_vector_type(4)));
typedef int i16v_t __attribute__((ext_vector_type(16)));

constexpr int kQThreads = 256;      // quantizer workgroup

// MT 32-row MFMA tiles by WAVES waves of 64 columns; each pipeline stage (one LDS buffer and
// one register set) covers KB k-blocks of 128.
template <int MT, int WAVES, int KB>
struct I8Tile {
  static constexpr int kMT = MT;
  static constexpr int kBM = 32 * MT;
  static constexpr int kWaves = WAVES;
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int kKB = KB;
  static constexpr int kARow = 128 * KB + 16;           // LDS row stride of the xq tile (bytes)
  static constexpr int kAChunks = kBM * 8 * KB / kThreads;  // 16-byte xq chunks per thread
  static constexpr size_t kLdsBytes = 2 * kBM * kARow;
};
typedef I8Tile<4, 8, 1> I8Large;
typedef I8Tile<2, 4, 1> I8Small;

template <int ACT>
__device__ inline float act_value(uint16_t b) {
  if constexpr (ACT == ACT_F16) return (float)__builtin_bit_cast(_Float16, b);
  else return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// ---- per-token quantization ----
// PERM: store each group of eight codes in the packed nibble order (positions 0..7 hold
// k = 0, 4, 1, 5, 2, 6, 3, 7) for the GEMM; otherwise in k order (the test hook).
template <int ACT, bool PERM>
__global__ __launch_bounds__(kQThreads) void quantize_rows_kernel(const uint16_t* __restrict__ x,
                                                                  int K, int8_t* __restrict__ xq,
                                                                  float* __restrict__ sx,
                                                                  int* __restrict__ xsum) {
  __shared__ float red_f[kQThreads / 64];
  __shared__ int red_i[kQThreads / 64];
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* row = x + (size_t)m * K;
  const int chunks = K / 8;

  float amax = 0.f;
  for (int c = threadIdx.x; c < chunks; c += kQThreads) {
    const u4_t v = *reinterpret_cast<const u4_t*>(row + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      amax = fmaxf(amax, fabsf(act_value<ACT>((uint16_t)(v[w] & 0xFFFFu))));
      amax = fmaxf(amax, fabsf(act_value<ACT>((uint16_t)(v[w] >> 16))));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if (lane == 0) red_f[wave] = amax;
  __syncthreads();
  amax = red_f[0];
#pragma unroll
  for (int w = 1; w < kQThreads / 64; ++w) amax = fmaxf(amax, red_f[w]);
  const float s = amax / 127.0f;  // one correctly rounded fp32 division

  int sum = 0;
  for (int c = threadIdx.x; c < chunks; c += kQThreads) {
    const u4_t v = *reinterpret_cast<const u4_t*>(row + c * 8);
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = act_value<ACT>((uint16_t)(v[e >> 1] >> (16 * (e & 1))));
      const float r = s > 0.f ? __builtin_rintf(f / s) : 0.f;  // quotient rounded once, then RNE
      q[e] = (int)fminf(fmaxf(r, -127.f), 127.f);
      sum += q[e];
    }
    uint32_t lo, hi;
    if constexpr (PERM) {
      lo = (q[0] & 0xFF) | (q[4] & 0xFF) << 8 | (q[1] & 0xFF) << 16 | (uint32_t)(q[5] & 0xFF) << 24;
      hi = (q[2] & 0xFF) | (q[6] & 0xFF) << 8 | (q[3] & 0xFF) << 16 | (uint32_t)(q[7] & 0xFF) << 24;
    } else {
      lo = (q[0] & 0xFF) | (q[1] & 0xFF) << 8 | (q[2] & 0xFF) << 16 | (uint32_t)(q[3] & 0xFF) << 24;
      hi = (q[4] & 0xFF) | (q[5] & 0xFF) << 8 | (q[6] & 0xFF) << 16 | (uint32_t)(q[7] & 0xFF) << 24;
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(xq + (size_t)m * K + c * 8);
    dst[0] = lo;
    dst[1] = hi;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane == 0) red_i[wave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < kQThreads / 64; ++w) t += red_i[w];
    sx[m] = s;
    if (xsum) xsum[m] = t;
  }
}

// workgroup -> output tile, so that tiles sharing weight columns run on the same XCD
__device__ __forceinline__ int i8_tile_of(int b, int G) {
  const int q = G >> 3, r = G & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

struct W4A8Params {
  const int8_t* xq;     // [M][K], groups of eight in packed nibble order
  const float* sx;      // [M]
  const int* xsum;      // [M] sum of the row's codes
  const u4_t* packed;
  const uint16_t* wscale;  // [N], activation type
  void* out;
  int out_dtype;
  int M, K, N, KC, NT;
  int tiles_m, tiles_n;
  int act;
  int S, kps;           // K slices (blockIdx.y) and k-blocks per slice
  int* partials;        // S > 1: [S][M][N] int32 sums of xq * u, summed by the reduce kernel
};

template <class T>
__global__ __launch_bounds__(T::kThreads) void w4a8_kernel(W4A8Params p) {
  constexpr int kMT = T::kMT, kBM = T::kBM, kWaves = T::kWaves, kThreads = T::kThreads;
  constexpr int kAChunks = T::kAChunks, kKB = T::kKB, kARow = T::kARow;
  constexpr int kCPR = 8 * kKB;  // 16-byte chunks per tile row per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_q[];  // [2][kBM * kARow]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = i8_tile_of(blockIdx.x, p.tiles_m * p.tiles_n);
  const int tm = t % p.tiles_m, tn = t / p.tiles_m;  // neighbours share weight columns
  const int K = p.K, M = p.M, KC = p.KC;
  const int m0 = tm * kBM;
  const int z = blockIdx.y;                      // K slice
  const int kc0 = z * p.kps, kc1 = min(kc0 + p.kps, KC);
  const int nt0 = tn * (kWaves * 4) + wave * 4;  // this wave's first strip
  const int h = lane >> 5;

  // a stage: the xq chunks this thread copies to LDS and, per k-block, the codes of this
  // wave's strips. Blocks past K (a last stage short of KB blocks) reload the last block's
  // codes; their activations are zero, so they add nothing.
  struct Regs {
    int kc;
    u4_t a[kAChunks];
    u4_t b[kKB][2][2];  // block, pair, chunk 32h + l%16 / 32h + 16 + l%16
  };
  auto load = [&](Regs& R, int kc) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c / kCPR, kch = c % kCPR;
      const int gm = min(m0 + row, M - 1);
      const int k = kc * 128 + kch * 16;
      // past K (a ragged last block, or a stage's missing blocks): an in-bounds chunk, zeroed
      // in store_a
      R.a[i] = *reinterpret_cast<const u4_t*>(p.xq + (size_t)gm * K + min(k, K - 16));
    }
    R.kc = kc;
#pragma unroll
    for (int d = 0; d < kKB; ++d)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int nt = min(nt0 + 2 * pr + ((lane >> 4) & 1), p.NT - 1);  // past N: never stored
        const u4_t* blk = p.packed + ((size_t)nt * KC + min(kc + d, kc1 - 1)) * 64 + 32 * h + (lane & 15);
        R.b[d][pr][0] = __builtin_nontemporal_load(blk);
        R.b[d][pr][1] = __builtin_nontemporal_load(blk + 16);
      }
  };
  auto store_a = [&](const Regs& R, int buf) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c / kCPR, kch = c % kCPR;
      const bool in_k = R.kc * 128 + kch * 16 < min(K, kc1 * 128);  // this slice's k only
      *reinterpret_cast<u4_t*>(lds_q + buf * kBM * kARow + row * kARow + kch * 16) =
          in_k ? R.a[i] : u4_t{0u, 0u, 0u, 0u};
    }
  };

  i16v_t acc[kMT][2];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][pr][i] = 0;

  // The A fragments of step s + 1 are read from LDS while step s's MFMAs run (two sets of
  // kMT fragments), so an MFMA never waits on the LDS read right before it.
  auto compute = [&](const Regs& R, int buf) {
    const uint8_t* as = lds_q + buf * kBM * kARow + (lane & 31) * kARow + h * 16;
    i4v_t af[2][kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) af[0][mt] = *reinterpret_cast<const i4v_t*>(as + mt * 32 * kARow);
#pragma unroll
    for (int s = 0; s < 4 * kKB; ++s) {  // 32-k steps of the stage
      if (s + 1 < 4 * kKB) {
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
          af[(s + 1) & 1][mt] = *reinterpret_cast<const i4v_t*>(as + mt * 32 * kARow + (s + 1) * 32);
      }
      i4v_t bq[2];
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const uint32_t w0 = R.b[s >> 2][pr][0][s & 3], w1 = R.b[s >> 2][pr][1][s & 3];
        bq[pr] = i4v_t{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu),
                       (int)(w1 & 0x0F0F0F0Fu), (int)((w1 >> 4) & 0x0F0F0F0Fu)};
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr)
          acc[mt][pr] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s & 1][mt], bq[pr], acc[mt][pr], 0, 0, 0);
    }
  };

  // two register sets and two LDS buffers: stage i+1 loads while stage i is multiplied
  const int nb = (kc1 - kc0 + kKB - 1) / kKB;
  Regs R0, R1;
  load(R0, kc0);
  store_a(R0, 0);
  __syncthreads();
  int i = 0;
  for (; i + 1 < nb; i += 2) {
    load(R1, kc0 + (i + 1) * kKB);
    __builtin_amdgcn_sched_barrier(0);
    compute(R0, 0);
    store_a(R1, 1);
    __syncthreads();
    load(R0, kc0 + min(i + 2, nb - 1) * kKB);
    __builtin_amdgcn_sched_barrier(0);
    compute(R1, 1);
    store_a(R0, 0);
    __syncthreads();
  }
  if (i < nb) compute(R0, 0);

  // ---- epilogue: lane l holds column 32 pair + l%32, rows 32 mt + 8 (i/4) + 4 (l/32) + i%4;
  // each row's scale and code sum are read once for both pairs ----
  float sw[2];
  int col[2];
  bool in_n[2];
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const int nt = nt0 + 2 * pr + ((lane >> 4) & 1);
    in_n[pr] = nt < p.NT;
    col[pr] = min(nt, p.NT - 1) * 16 + (lane & 15);
    sw[pr] = p.act == ACT_F16 ? act_value<ACT_F16>(p.wscale[col[pr]]) : act_value<ACT_BF16>(p.wscale[col[pr]]);
  }
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + mt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (m < M) {
        if (p.S > 1) {  // K split: this slice's exact integer sums
#pragma unroll
          for (int pr = 0; pr < 2; ++pr)
            if (in_n[pr]) p.partials[((size_t)z * M + m) * p.N + col[pr]] = acc[mt][pr][e];
          continue;
        }
        const int zs = 8 * p.xsum[m];
        const float sxm = p.sx[m];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr)
          if (in_n[pr]) {
            const int v = acc[mt][pr][e] - zs;  // exact: sum of xq * (u - 8)
            store_out(p.out, (size_t)m * p.N + col[pr], (float)v * sxm * sw[pr], p.out_dtype);
          }
      }
    }
}

// K split: the slices' integer sums add exactly (in any order), then the same epilogue as an
// unsplit launch, so the result does not depend on S. Four consecutive columns per thread.
__global__ __launch_bounds__(256) void w4a8_reduce_kernel(const int* __restrict__ partials, int M,
                                                          int N, int S, const int* __restrict__ xsum,
                                                          const float* __restrict__ sx,
                                                          const uint16_t* __restrict__ wscale,
                                                          int act, void* out, int out_dtype) {
  const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= (size_t)M * N) return;
  const int m = (int)(e / N), n = (int)(e - (size_t)m * N);
  i4v_t v = *reinterpret_cast<const i4v_t*>(partials + e);
  for (int zz = 1; zz < S; ++zz) v += *reinterpret_cast<const i4v_t*>(partials + (size_t)zz * M * N + e);
  const int zs = 8 * xsum[m];
  const float sxm = sx[m];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float sw = act == ACT_F16 ? act_value<ACT_F16>(wscale[n + c]) : act_value<ACT_BF16>(wscale[n + c]);
    store_out(out, e + c, (float)(v[c] - zs) * sxm * sw, out_dtype);
  }
}

int cu_count_w4a8() {
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

// Geometry: the large tile when its tiles fill the compute units, else the small one; and
// while the small tiles leave compute units idle, K cut into S = 2, then 4 slices (each at
// least 8 k-blocks).
struct W4A8Geometry {
  bool small;
  int tiles_m, tiles_n, S, kps;
};

W4A8Geometry w4a8_geometry(int M, int K, int N) {
  const int NT = N / 16, KC = ceil_div(K, 128), cus = cu_count_w4a8();
  W4A8Geometry g;
  const long large = (long)ceil_div(M, I8Large::kBM) * ceil_div(NT, I8Large::kWaves * 4);
  g.small = large < cus;
  g.tiles_m = ceil_div(M, g.small ? I8Small::kBM : I8Large::kBM);
  g.tiles_n = ceil_div(NT, (g.small ? I8Small::kWaves : I8Large::kWaves) * 4);
  g.S = 1;
  const long tiles = (long)g.tiles_m * g.tiles_n;
  while (g.S < 4 && tiles * g.S < cus && KC >= 2 * g.S * 8) g.S *= 2;
  g.kps = ceil_div(KC, g.S);
  g.S = ceil_div(KC, g.kps);
  return g;
}

struct W4A8Workspace {
  size_t xq, sx, xsum, partials, total;
};

W4A8Workspace w4a8_layout(int M, int K, int N) {
  const W4A8Geometry g = w4a8_geometry(M, K, N);
  W4A8Workspace w;
  w.xq = 0;
  w.sx = align256((size_t)M * K);
  w.xsum = w.sx + align256((size_t)M * 4);
  w.partials = w.xsum + align256((size_t)M * 4);
  w.total = w.partials + (g.S > 1 ? align256((size_t)g.S * M * N * 4) : 0);
  return w;
}

template <class T>
hipError_t launch_w4a8_tile(const W4A8Params& p, hipStream_t s) {
  hipLaunchKernelGGL(w4a8_kernel<T>, dim3(p.tiles_m * p.tiles_n, p.S), dim3(T::kThreads), T::kLdsBytes, s, p);
  return hipGetLastError();
}

}  // namespace

size_t w4a8_workspace_bytes(int M, int K, int N) { return M > 0 ? w4a8_layout(M, K, N).total : 0; }

const char* w4a8_name(int M, int K, int N) {
  const W4A8Geometry g = w4a8_geometry(M, K, N);
  if (g.small) return g.S > 1 ? "w4a8_64x256_splitk" : "w4a8_64x256";
  return g.S > 1 ? "w4a8_128x512_splitk" : "w4a8_128x512";
}

hipError_t launch_quantize_act(const void* x, int M, int K, int act, bool perm, int8_t* xq,
                               float* sx, int* xsum, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  if (act == ACT_F16) {
    if (perm) hipLaunchKernelGGL((quantize_rows_kernel<ACT_F16, true>), dim3(M), dim3(kQThreads), 0, s, xp, K, xq, sx, xsum);
    else hipLaunchKernelGGL((quantize_rows_kernel<ACT_F16, false>), dim3(M), dim3(kQThreads), 0, s, xp, K, xq, sx, xsum);
  } else {
    if (perm) hipLaunchKernelGGL((quantize_rows_kernel<ACT_BF16, true>), dim3(M), dim3(kQThreads), 0, s, xp, K, xq, sx, xsum);
    else hipLaunchKernelGGL((quantize_rows_kernel<ACT_BF16, false>), dim3(M), dim3(kQThreads), 0, s, xp, K, xq, sx, xsum);
  }
  return hipGetLastError();
}

hipError_t launch_w4a8(const GemmArgs& a) {
  const W4A8Geometry g = w4a8_geometry(a.M, a.K, a.N);
  const W4A8Workspace w = w4a8_layout(a.M, a.K, a.N);
  char* ws = static_cast<char*>(a.workspace);
  W4A8Params p;
  p.xq = reinterpret_cast<const int8_t*>(ws + w.xq);
  p.sx = reinterpret_cast<const float*>(ws + w.sx);
  p.xsum = reinterpret_cast<const int*>(ws + w.xsum);
  hipError_t e = launch_quantize_act(a.x, a.M, a.K, a.act, true, reinterpret_cast<int8_t*>(ws + w.xq),
                                     reinterpret_cast<float*>(ws + w.sx),
                                     reinterpret_cast<int*>(ws + w.xsum), a.stream);
  if (e != hipSuccess) return e;
  p.packed = reinterpret_cast<const u4_t*>(a.packed);
  p.wscale = static_cast<const uint16_t*>(a.scales);
  p.out = a.out;
  p.out_dtype = a.out_dtype;
  p.M = a.M;
  p.K = a.K;
  p.N = a.N;
  p.KC = ceil_div(a.K, 128);
  p.NT = a.N / 16;
  p.act = a.act;
  p.tiles_m = g.tiles_m;
  p.tiles_n = g.tiles_n;
  p.S = g.S;
  p.kps = g.kps;
  p.partials = g.S > 1 ? reinterpret_cast<int*>(ws + w.partials) : nullptr;
  e = g.small ? launch_w4a8_tile<I8Small>(p, a.stream) : launch_w4a8_tile<I8Large>(p, a.stream);
  if (e != hipSuccess || g.S == 1) return e;
  const size_t quads = (size_t)a.M * a.N / 4;
  hipLaunchKernelGGL(w4a8_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, a.stream,
                     p.partials, a.M, a.N, g.S, p.xsum, p.sx, p.wscale, a.act, a.out, a.out_dtype);
  return hipGetLastError();
}

}  // namespace w4a16
