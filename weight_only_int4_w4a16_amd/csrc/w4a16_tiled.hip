// w4a16_tiled.hip - W4A16 GEMM for batched and prefill shapes (M > 64), where the MFMAs and
// not the weight bytes bound the time.
//
// "INT8 vs INT4 Quantization, in depth", section "Two regimes": past the crossover batch a
// W4A16 layer is compute-bound and its dequantization work must be amortized over many
// rows; "INT4 and Low-Bit Inference", section 5 (Marlin): the unpack is fused into the
// tile loop and the 16-bit weight tile never goes to HBM.
//
// Tiling. A workgroup of four waves computes a 128 x 256 output tile. Each wave owns 64
// columns (4 strips of 16) over all 128 rows: per 32-k step it dequantizes one packed
// word per strip in registers (the packed layout hands each lane exactly its MFMA B
// operand) and reuses it for 8 row tiles, so the dequantization is spread over 128 rows.
// The activation tile (128 rows x 128 k, fp16/bf16) is staged in LDS, double-buffered,
// and shared by the four waves; the A fragment of a row tile is read once per step and
// used for four strips. Products: v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulators.
//
// Split-K. When the output tiles alone cannot fill the chip, the K range is cut into S
// contiguous slices, one workgroup each. Every slice stores its fp32 partial tile in the
// workspace and a second small kernel sums the S partials in slice order (deterministic)
// into the output.
#include "w4a16_device.hpp"
#include "w4a16_launch.hpp"

namespace w4a16 {

namespace {

constexpr int kBM = 128;            // rows per workgroup tile
constexpr int kStrips = 4;          // 16-column strips per wave
constexpr int kWaves = 4;           // waves per workgroup
constexpr int kBN = 16 * kStrips * kWaves;  // 256 columns per workgroup tile
constexpr int kMT = kBM / 16;       // MFMA row tiles per wave
constexpr int kAStride = 128 + 8;   // LDS row stride of the activation tile (halves)
constexpr int kAChunks = kBM * 16 / (64 * kWaves);  // 16-byte chunks per thread per k-block
constexpr size_t kLdsBytes = 2 * kBM * kAStride * 2;  // double-buffered activation tile

enum Fmt { FMT_ASYM = 0, FMT_SYM = 1, FMT_NF4 = 2 };

template <int ACT>
struct ActT;
template <>
struct ActT<ACT_F16> { typedef h8_t type; };
template <>
struct ActT<ACT_BF16> { typedef b8_t type; };

struct TiledParams {
  const uint16_t* x;
  int M, K, N;
  const u4_t* packed;
  const uint16_t* scales;
  const uint32_t* qzeros;
  const uint16_t* codebook;
  void* out;
  int out_dtype;
  int KC, NT, NG;      // k-blocks, strips, scale groups along K
  int tiles_m, tiles_n;
  int S, kps;          // K slices and k-blocks per slice
  float* partials;     // [S][tiles_m * 128][N] fp32 (S > 1)
};

// workgroup -> output tile, so that tiles sharing weight columns run on the same XCD
__device__ __forceinline__ int tile_of(int b, int G) {
  const int q = G >> 3, r = G & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

template <int ACT, int GPC, int FMT>
__global__ __launch_bounds__(256) void tiled_kernel(TiledParams p) {
  typedef typename ActT<ACT>::type AT;
  constexpr int SPG = 4 / GPC;
  constexpr bool ZEROS = FMT == FMT_ASYM;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_a[];  // [2][kBM * kAStride]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles = p.tiles_m * p.tiles_n;
  const int t = tile_of(blockIdx.x, tiles);
  const int tm = t % p.tiles_m, tn = t / p.tiles_m;  // neighbours share weight columns
  const int z = blockIdx.y;
  const int K = p.K, N = p.N, M = p.M, KC = p.KC;
  const int m0 = tm * kBM;
  const int kc0 = z * p.kps;
  const int kc1 = min(kc0 + p.kps, KC);
  const int nt0 = tn * (kWaves * kStrips) + wave * kStrips;  // this wave's first strip
  const int shift = 4 * (lane & 7);

  // ---- one k-block of operands: the activation tile slice this thread copies to LDS, and
  // the codes + metadata of this wave's strips (kept in registers until the MFMAs) ----
  struct Regs {
    int kc;
    u4_t a[kAChunks];
    u4_t b[kStrips];
    uint32_t s[kStrips][GPC];  // 16-bit scale zero-extended by the load itself
    uint32_t z[kStrips][GPC];
  };
  auto load = [&](Regs& R, int kc) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c >> 4, kch = c & 15;
      const int gm = min(m0 + row, M - 1);
      const int k = kc * 128 + kch * 8;
      // a ragged K ends inside the last block: load an in-bounds chunk (zeroed in store_a)
      R.a[i] = *reinterpret_cast<const u4_t*>(p.x + (size_t)gm * K + min(k, K - 8));
    }
    R.kc = kc;
#pragma unroll
    for (int st = 0; st < kStrips; ++st) {
      const int nt = min(nt0 + st, p.NT - 1);  // strips past N: loaded in bounds, never stored
      const int col = nt * 16 + (lane & 15);
      R.b[st] = __builtin_nontemporal_load(p.packed + ((size_t)nt * KC + kc) * 64 + lane);
#pragma unroll
      for (int gi = 0; gi < GPC; ++gi) {
        const int g = min(kc * GPC + gi, p.NG - 1);
        R.s[st][gi] = p.scales[(size_t)g * N + col];
        if constexpr (ZEROS) R.z[st][gi] = p.qzeros[(size_t)g * (N >> 3) + (col >> 3)];
      }
    }
  };
  auto store_a = [&](const Regs& R, int buf) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c >> 4, kch = c & 15;
      const bool in_k = R.kc * 128 + kch * 8 < K;
      *reinterpret_cast<u4_t*>(lds_a + buf * kBM * kAStride + row * kAStride + kch * 8) =
          in_k ? R.a[i] : u4_t{0u, 0u, 0u, 0u};
    }
  };

  Nf4Lut lut;
  if constexpr (FMT == FMT_NF4) lut = load_nf4_lut(p.codebook);

  f4_t acc[kMT][kStrips];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int st = 0; st < kStrips; ++st) acc[mt][st] = f4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Regs& R, int buf) {
    const uint16_t* as = lds_a + buf * kBM * kAStride;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gi = j / SPG;
      AT bf[kStrips];
#pragma unroll
      for (int st = 0; st < kStrips; ++st) {
        const uint32_t w = R.b[st][j];
        const uint32_t sraw = R.s[st][gi];
        if constexpr (FMT == FMT_NF4) {
          if constexpr (ACT == ACT_F16)
            bf[st] = dequant_word_nf4_f16(w, lut, as_h2(sraw * 0x00010001u));
          else
            bf[st] = dequant_word_nf4_bf16(w, lut, (float)__builtin_bit_cast(_Float16, (uint16_t)sraw));
        } else {
          const uint32_t zq = ZEROS ? (R.z[st][gi] >> shift) & 0xFu : 8u;
          if constexpr (ACT == ACT_F16)
            bf[st] = dequant_word_f16(w, make_zero_f16(zq), as_h2(sraw * 0x00010001u));
          else
            bf[st] = dequant_word_bf16(w, make_zero_f32(zq, __builtin_bit_cast(float, sraw << 16)));
        }
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const u4_t a = *reinterpret_cast<const u4_t*>(
            as + (mt * 16 + (lane & 15)) * kAStride + j * 32 + (lane >> 4) * 8);
#pragma unroll
        for (int st = 0; st < kStrips; ++st)
          acc[mt][st] = mfma16(__builtin_bit_cast(AT, a), bf[st], acc[mt][st]);
      }
    }
  };

  // Two register sets and two LDS buffers: block i+1 loads while block i is multiplied.
  // Loads are unconditional (past the slice they re-read its last block, never used), so
  // the in-order load counter only ever waits for the set about to be used; a scheduling
  // barrier after each batch of loads keeps the compiler from sinking them below the MFMAs.
  const int nb = kc1 - kc0;
  Regs R0, R1;
  load(R0, kc0);
  store_a(R0, 0);
  __syncthreads();
  int i = 0;
  for (; i + 1 < nb; i += 2) {
    load(R1, kc0 + i + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(R0, 0);
    store_a(R1, 1);
    __syncthreads();
    load(R0, min(kc0 + i + 2, kc1 - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(R1, 1);
    store_a(R0, 0);
    __syncthreads();
  }
  if (i < nb) compute(R0, 0);

  // ---- epilogue ----
  // lane l holds column 16*strip + l%16 and rows 16*mt + 4*(l/16) + r of each 16x16 tile
  if (p.S == 1) {
#pragma unroll
    for (int st = 0; st < kStrips; ++st) {
      const int nt = nt0 + st;
      if (nt < p.NT) {
        const int col = nt * 16 + (lane & 15);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + mt * 16 + 4 * (lane >> 4) + r;
            if (m < M) store_out(p.out, (size_t)m * N + col, acc[mt][st][r], p.out_dtype);
          }
      }
    }
    return;
  }
  // K split: store this slice's fp32 partial tile; the reduce kernel sums the slices
  const size_t slice_stride = (size_t)p.tiles_m * kBM * N;
#pragma unroll
  for (int st = 0; st < kStrips; ++st) {
    const int nt = nt0 + st;
    if (nt < p.NT) {
      const int col = nt * 16 + (lane & 15);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + mt * 16 + 4 * (lane >> 4) + r;
          p.partials[z * slice_stride + (size_t)m * N + col] = acc[mt][st][r];
        }
    }
  }
}

// y[m, n] = sum over slices s = 0..S-1, in that order, of partial[s][m][n]; four
// consecutive columns per thread (N is a multiple of 16)
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partials, int M,
                                                            int N, int S, size_t slice_stride,
                                                            void* out, int out_dtype) {
  const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t e = i4 * 4;
  if (e >= (size_t)M * N) return;
  f4_t v = *reinterpret_cast<const f4_t*>(partials + e);
  for (int zz = 1; zz < S; ++zz) v += *reinterpret_cast<const f4_t*>(partials + zz * slice_stride + e);
#pragma unroll
  for (int c = 0; c < 4; ++c) store_out(out, e + c, v[c], out_dtype);
}

int cu_count_tiled() {
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

struct TiledGeometry {
  int tiles_m, tiles_n, S, kps;
  size_t partial_bytes;
};

// K slices: double S while the workgroups (tiles x slices) still fit one per compute unit,
// keeping at least 8 k-blocks per slice.
TiledGeometry tiled_geometry(int M, int K, int N) {
  TiledGeometry g;
  const int KC = ceil_div(K, 128);
  g.tiles_m = ceil_div(M, kBM);
  g.tiles_n = ceil_div(N / 16, kWaves * kStrips);
  const int tiles = g.tiles_m * g.tiles_n;
  const int cus = cu_count_tiled();
  int S = 1;
  while (tiles * S * 2 <= cus && KC / (2 * S) >= 8) S *= 2;
  g.kps = ceil_div(KC, S);
  g.S = ceil_div(KC, g.kps);
  g.partial_bytes = g.S > 1 ? (size_t)g.S * g.tiles_m * kBM * N * 4 : 0;
  return g;
}

template <int ACT, int GPC>
hipError_t launch_fmt(const GemmArgs& a, const TiledParams& p, dim3 grid) {
  if (a.nf4)
    hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_NF4>), grid, dim3(256), kLdsBytes, a.stream, p);
  else if (a.qzeros)
    hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_ASYM>), grid, dim3(256), kLdsBytes, a.stream, p);
  else
    hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_SYM>), grid, dim3(256), kLdsBytes, a.stream, p);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_gpc(const GemmArgs& a, const TiledParams& p, dim3 grid) {
  switch (a.group_size) {
    case 128: return launch_fmt<ACT, 1>(a, p, grid);
    case 64: return launch_fmt<ACT, 2>(a, p, grid);
    default: return launch_fmt<ACT, 4>(a, p, grid);
  }
}

}  // namespace

bool tiled_supported(const GemmArgs&) { return true; }

const char* tiled_name(int M, int K, int N) {
  return tiled_geometry(M, K, N).S > 1 ? "w4a16_tiled_128x256_splitk" : "w4a16_tiled_128x256";
}

size_t tiled_workspace_bytes(int M, int K, int N) {
  const TiledGeometry g = tiled_geometry(M, K, N);
  return g.partial_bytes;
}

hipError_t launch_tiled(const GemmArgs& a) {
  const TiledGeometry g = tiled_geometry(a.M, a.K, a.N);
  TiledParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  p.M = a.M;
  p.K = a.K;
  p.N = a.N;
  p.packed = reinterpret_cast<const u4_t*>(a.packed);
  p.scales = static_cast<const uint16_t*>(a.scales);
  p.qzeros = a.qzeros;
  p.codebook = a.codebook;
  p.out = a.out;
  p.out_dtype = a.out_dtype;
  p.KC = ceil_div(a.K, 128);
  p.NT = a.N / 16;
  p.NG = a.K / a.group_size;
  p.tiles_m = g.tiles_m;
  p.tiles_n = g.tiles_n;
  p.S = g.S;
  p.kps = g.kps;
  p.partials = g.S > 1 ? static_cast<float*>(a.workspace) : nullptr;
  const dim3 grid(g.tiles_m * g.tiles_n, g.S);
  const hipError_t e = a.act == ACT_F16 ? launch_gpc<ACT_F16>(a, p, grid) : launch_gpc<ACT_BF16>(a, p, grid);
  if (e != hipSuccess || g.S == 1) return e;
  const size_t quads = (size_t)a.M * a.N / 4;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, a.stream,
                     p.partials, a.M, a.N, g.S, (size_t)g.tiles_m * kBM * a.N, a.out, a.out_dtype);
  return hipGetLastError();
}

}  // namespace w4a16
