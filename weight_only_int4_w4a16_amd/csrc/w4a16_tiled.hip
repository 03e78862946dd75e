// w4a16_tiled.hip - W4A16 GEMM for batched and prefill shapes (M > 16), where the MFMAs and
// not the weight bytes bound the time.
//
// "INT8 vs INT4 Quantization, in depth", section "Two regimes": past the crossover batch a
// W4A16 layer is compute-bound and its dequantization work must be amortized over many
// rows; "INT4 and Low-Bit Inference", section 5 (Marlin): the unpack is fused into the
// tile loop and the 16-bit weight tile never goes to HBM.
//
// Tiling. A workgroup of eight waves (two per SIMD) computes a 128 x 512 output tile (or, when
// those tiles would not cover the compute units, four waves a 64 x 256 tile). Each wave owns 64
// columns (two 32-column pairs of strips) over all 128 rows and multiplies with
// v_mfma_f32_32x32x16_{f16,bf16}, which on gfx950 delivers twice the flops per cycle of the
// 16x16x32 form. Its B operand gives lane l column l%32 of a pair and k = 8(l/32) + i of a
// 16-k step. In the packed layout those eight codes are word t/2 of the 16-byte chunk that
// lane 16*((2t + l/32) % 4) + l%16 of the strip's block owns; lane l loads those two
// chunks (32 bytes) itself, so every code is loaded once and no lanes exchange data. Each
// word is dequantized once, in registers, and reused for 4 row tiles (128 rows).
// The activation tile (128 rows x 128 k, fp16/bf16) is staged in LDS, double-buffered,
// and shared by the four waves; the A fragment of a row tile is read once per step and
// used for both pairs. Accumulation is fp32.
//
// Split-K. When the output tiles alone cannot fill the chip, the K range is cut into S
// contiguous slices, one workgroup each. Every slice stores its fp32 partial tile in the
// workspace and a second small kernel sums the S partials in slice order (deterministic)
// into the output.
#include <type_traits>

#include "w4a16_device.hpp"
#include "w4a16_launch.hpp"

namespace w4a16 {

namespace {

constexpr int kPairs = 2;           // 32-column strip pairs per wave (4 strips of 16)
constexpr int kStrips = 2 * kPairs;
constexpr int kAStride = 128 + 8;   // LDS row stride of the activation tile (halves)

// Workgroup tile: MT 32-row MFMA tiles (kBM = 32 MT rows) by WAVES waves of 64 columns.
// Large: 128 x 512, eight waves (two per SIMD). Small: 64 x 256, four waves, for GEMMs whose
// large tiles would leave compute units idle (each large tile row of M <= 256 is 28-56
// tiles at N = 14336).
template <int MT, int WAVES>
struct TileShape {
  static constexpr int kMT = MT;
  static constexpr int kBM = 32 * MT;
  static constexpr int kWaves = WAVES;
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int kAChunks = kBM * 16 / kThreads;  // 16-byte chunks per thread per block
  static constexpr size_t kLdsBytes = 2 * kBM * kAStride * 2;  // double-buffered activations
};
typedef TileShape<4, 8> LargeTile;
typedef TileShape<2, 4> SmallTile;

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
  float* partials;     // [S][tiles_m * tile rows][N] fp32 (S > 1)
  int half;            // GLU: strips per half of the fused gate+up weight (NT / 2)
  const uint16_t* xscale;  // XS: AWQ S^-1 [K] in the activation type
};

// workgroup -> output tile, so that tiles sharing weight columns run on the same XCD
__device__ __forceinline__ int tile_of(int b, int G) {
  const int q = G >> 3, r = G & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// GLU: the weight is a fused gate+up projection [K][2 Nh] (gate columns first). A wave's
// first strip pair is two gate strips, its second the matching up strips, and the output is
// h = SiLU(gate) * up, [M][Nh] (with K split, both halves go to the partials and the GLU
// reduce kernel forms h).
// XS: AWQ input scaling, x' = RN(x * s_inv[k]) as the activation tile goes to LDS.
template <int ACT, int GPC, int FMT, class T, bool GLU, bool XS>
__global__ __launch_bounds__(T::kThreads) void tiled_kernel(TiledParams p) {
  constexpr int kMT = T::kMT, kBM = T::kBM, kWaves = T::kWaves, kThreads = T::kThreads;
  constexpr int kAChunks = T::kAChunks;
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
  const int g0 = tn * (kWaves * 2) + wave * 2;                // GLU: its first gate strip
  // strip of pair pr, half h (h = lane/16 % 2), clamped in bounds for loads
  auto strip_of = [&](int pr, int h) {
    return GLU ? min(g0 + h, p.half - 1) + pr * p.half : min(nt0 + 2 * pr + h, p.NT - 1);
  };
  const int shift = 4 * (lane & 7);

  // ---- one k-block of operands: the activation tile slice this thread copies to LDS, and
  // the codes + metadata of this wave's strips (kept in registers until the MFMAs) ----
  struct Regs {
    int kc;
    u4_t a[kAChunks];
    u4_t xsc;                  // XS: s_inv for this thread's k chunk (the same in every row)
    u4_t b[kPairs][2];         // chunks 16h + c and 32 + 16h + c (h = lane/32, c = lane%16)
    uint32_t s[kPairs][GPC];   // 16-bit scale zero-extended by the load itself
    uint32_t z[kPairs][GPC];
  };
  auto load = [&](Regs& R, int kc) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c >> 4, kch = c & 15;
      const int gm = min(m0 + row, M - 1);
      const int k = kc * 128 + kch * 8;
      // a ragged K ends inside the last block: load an in-bounds chunk (zeroed in store_a)
      R.a[i] = *reinterpret_cast<const u4_t*>(p.x + (size_t)gm * K + min(k, K - 8));
    }
    static_assert(kThreads % 16 == 0, "a thread's k chunk is threadIdx.x % 16 in every row");
    if constexpr (XS)
      R.xsc = *reinterpret_cast<const u4_t*>(p.xscale + min(kc * 128 + (int)(threadIdx.x & 15) * 8, K - 8));
    R.kc = kc;
#pragma unroll
    for (int pr = 0; pr < kPairs; ++pr) {
      // strips past N: loaded in bounds, never stored
      const int nt = strip_of(pr, (lane >> 4) & 1);
      const int col = nt * 16 + (lane & 15);
      const u4_t* blk = p.packed + ((size_t)nt * KC + kc) * 64;
      const int c0 = 16 * (lane >> 5) + (lane & 15);
      R.b[pr][0] = __builtin_nontemporal_load(blk + c0);
      R.b[pr][1] = __builtin_nontemporal_load(blk + c0 + 32);
#pragma unroll
      for (int gi = 0; gi < GPC; ++gi) {
        const int g = min(kc * GPC + gi, p.NG - 1);
        R.s[pr][gi] = p.scales[(size_t)g * N + col];
        if constexpr (ZEROS) R.z[pr][gi] = p.qzeros[(size_t)g * (N >> 3) + (col >> 3)];
      }
    }
  };
  auto store_a = [&](const Regs& R, int buf) {
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c >> 4, kch = c & 15;
      const bool in_k = R.kc * 128 + kch * 8 < K;
      u4_t v = R.a[i];
      if constexpr (XS) v = scale_act8<ACT>(v, R.xsc);
      *reinterpret_cast<u4_t*>(lds_a + buf * kBM * kAStride + row * kAStride + kch * 8) =
          in_k ? v : u4_t{0u, 0u, 0u, 0u};
    }
  };

  Nf4Lut lut;
  if constexpr (FMT == FMT_NF4) lut = load_nf4_lut(p.codebook);

  f16v_t acc[kMT][kPairs];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int pr = 0; pr < kPairs; ++pr)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][pr][i] = 0.f;

  auto compute = [&](const Regs& R, int buf) {
    const uint16_t* as = lds_a + buf * kBM * kAStride;
#pragma unroll
    for (int t = 0; t < 8; ++t) {  // 16-k steps of the block
      const int gi = t / (8 / GPC);
      AT bf[kPairs];
#pragma unroll
      for (int pr = 0; pr < kPairs; ++pr) {
        const uint32_t w = R.b[pr][t & 1][t >> 1];
        const uint32_t sraw = R.s[pr][gi];
        if constexpr (FMT == FMT_NF4) {
          if constexpr (ACT == ACT_F16)
            bf[pr] = dequant_word_nf4_f16(w, lut, as_h2(sraw * 0x00010001u));
          else
            bf[pr] = dequant_word_nf4_bf16(w, lut, (float)__builtin_bit_cast(_Float16, (uint16_t)sraw));
        } else {
          const uint32_t zq = ZEROS ? (R.z[pr][gi] >> shift) & 0xFu : 8u;
          if constexpr (ACT == ACT_F16)
            bf[pr] = dequant_word_f16(w, make_zero_f16(zq), as_h2(sraw * 0x00010001u));
          else
            bf[pr] = dequant_word_bf16(w, make_zero_f32(zq, __builtin_bit_cast(float, sraw << 16)));
        }
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        // A: row 32 mt + l%32, k = 16 t + 8 (l/32) .. +8
        const u4_t a = *reinterpret_cast<const u4_t*>(
            as + (mt * 32 + (lane & 31)) * kAStride + t * 16 + (lane >> 5) * 8);
#pragma unroll
        for (int pr = 0; pr < kPairs; ++pr)
          acc[mt][pr] = mfma32(__builtin_bit_cast(AT, a), bf[pr], acc[mt][pr]);
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
  // lane l holds column 32*pair + l%32 and rows 32*mt + 8*(i/4) + 4*(l/32) + i%4, i < 16
  const size_t slice_stride = (size_t)p.tiles_m * kBM * N;
  if constexpr (GLU) {
    const int gs = g0 + ((lane >> 4) & 1);  // gate strip of this lane's columns
    if (gs < p.half) {
      const int col = gs * 16 + (lane & 15);  // column in the gate half and in h
      const int nh = N >> 1;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = m0 + mt * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          const float g = acc[mt][0][i], u = acc[mt][1][i];
          if (p.S == 1) {
            if (m < M) store_out(p.out, (size_t)m * nh + col, g / (1.0f + __expf(-g)) * u, p.out_dtype);
          } else if (m < M) {
            p.partials[z * slice_stride + (size_t)m * N + col] = g;
            p.partials[z * slice_stride + (size_t)m * N + nh + col] = u;
          }
        }
    }
    return;
  }
#pragma unroll
  for (int pr = 0; pr < kPairs; ++pr) {
    const int nt = nt0 + 2 * pr + ((lane >> 4) & 1);
    if (nt < p.NT) {
      const int col = nt * 16 + (lane & 15);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = m0 + mt * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (p.S == 1) {
            if (m < M) store_out(p.out, (size_t)m * N + col, acc[mt][pr][i], p.out_dtype);
          } else if (m < M) {
            // K split: this slice's fp32 partial tile; the reduce kernel sums the slices
            p.partials[z * slice_stride + (size_t)m * N + col] = acc[mt][pr][i];
          }
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

// h[m, n] = SiLU(g) * u with g, u the slice sums (in slice order) of partial[s][m][n] and
// partial[s][m][n + Nh], n < Nh; four consecutive columns per thread (Nh is a multiple of 16)
__global__ __launch_bounds__(256) void splitk_reduce_glu_kernel(const float* __restrict__ partials, int M,
                                                                int Nh, int S, size_t slice_stride,
                                                                void* out, int out_dtype) {
  const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t e = i4 * 4;
  if (e >= (size_t)M * Nh) return;
  const size_t m = e / Nh, n = e - m * Nh;
  const size_t pg = m * 2 * Nh + n;
  f4_t g = *reinterpret_cast<const f4_t*>(partials + pg);
  f4_t u = *reinterpret_cast<const f4_t*>(partials + pg + Nh);
  for (int zz = 1; zz < S; ++zz) {
    g += *reinterpret_cast<const f4_t*>(partials + zz * slice_stride + pg);
    u += *reinterpret_cast<const f4_t*>(partials + zz * slice_stride + pg + Nh);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) store_out(out, e + c, g[c] / (1.0f + __expf(-g[c])) * u[c], out_dtype);
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
  bool small;          // SmallTile instead of LargeTile
  int bm, bn;          // tile rows and columns
  int tiles_m, tiles_n, S, kps;
  size_t partial_bytes;
};

// A tile kind with K cut into (about) S contiguous slices of whole k-blocks.
TiledGeometry geometry_for(int M, int K, int N, bool small, int S) {
  TiledGeometry g;
  const int KC = ceil_div(K, 128);
  g.small = small;
  g.bm = small ? SmallTile::kBM : LargeTile::kBM;
  g.bn = 16 * kStrips * (small ? SmallTile::kWaves : LargeTile::kWaves);
  g.tiles_m = ceil_div(M, g.bm);
  g.tiles_n = ceil_div(N, g.bn);
  g.kps = ceil_div(KC, S);
  g.S = ceil_div(KC, g.kps);
  g.partial_bytes = g.S > 1 ? (size_t)g.S * g.tiles_m * g.bm * N * 4 : 0;
  return g;
}

// Modelled time of a geometry: on the busiest compute unit, each of its workgroups costs a
// fixed 2.5 us (pipeline fill, epilogue) plus its tile flops (padded rows included) at the
// rate one compute unit sustains with that tile; when K is split, the fp32 partial sums are
// written and read back at 5 TB/s and the reduce launch costs 2 us. Rates measured on MI355X
// (fp16, g128): large tile 4.2-5.4 TFLOP/s per compute unit (4.6 taken); small tile 2.7 with
// one workgroup per compute unit, 3.4 with two or more.
double modelled_us(const TiledGeometry& g, int M, int N, int cus) {
  const long wgs = (long)g.tiles_m * g.tiles_n * g.S;
  const long per_cu = (wgs + cus - 1) / cus;
  const double wg_flops = 2.0 * g.bm * g.bn * g.kps * 128;
  const double rate = !g.small ? 4.6e6 : per_cu > 1 ? 3.4e6 : 2.7e6;  // flop per us
  double us = per_cu * (2.5 + wg_flops / rate);
  if (g.S > 1) us += 2.0 * g.S * M * (double)N * 4 / 5e6 + 2.0;
  return us;
}

// Tile and K split: the large tile (each dequantized word feeds four 32-row tiles, not two)
// or the small one (more workgroups), each with S = 1, 2, 4, ... slices of at least two
// k-blocks and at most four workgroups per compute unit; the model's fastest wins. It
// tracks the measured choices: large wins by 12-21% at 8192x28672 M=256, 28672x8192 M=256,
// 8192x10240 M=512 and loses by 7-13% at 4096x4096 M=512 and 1024 (split-K partials
// outweigh its rate); small matrices past 16 rows split K deeply (4096x4096 at M=17: S=16).
TiledGeometry tiled_geometry(int M, int K, int N) {
  const int cus = cu_count_tiled();
  const int KC = ceil_div(K, 128);
  TiledGeometry best = geometry_for(M, K, N, true, 1);
  double best_us = modelled_us(best, M, N, cus);
  for (int small = 0; small < 2; ++small)
    for (int S = 1; S == 1 || KC / S >= 2; S *= 2) {
      const TiledGeometry g = geometry_for(M, K, N, small != 0, S);
      if (S > 1 && (long)g.tiles_m * g.tiles_n * g.S > 4L * cus) break;
      const double us = modelled_us(g, M, N, cus);
      if (us < best_us) {
        best = g;
        best_us = us;
      }
    }
  return best;
}

template <int ACT, int GPC, class T, bool GLU>
hipError_t launch_glu(const GemmArgs& a, const TiledParams& p, dim3 grid) {
  if (a.nf4)
    hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_NF4, T, GLU, false>), grid, dim3(T::kThreads), T::kLdsBytes, a.stream, p);
  else if (a.qzeros)
    hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_ASYM, T, GLU, false>), grid, dim3(T::kThreads), T::kLdsBytes, a.stream, p);
  else
    hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_SYM, T, GLU, false>), grid, dim3(T::kThreads), T::kLdsBytes, a.stream, p);
  return hipGetLastError();
}

// AWQ-scaled activations, small tile: the plain GEMM, affine formats, x scaled as it is
// staged (the large tile takes x' from a pre-pass instead: the multiply there cost 8% of the
// bf16 prefill GEMM against 1-2% for the pre-pass)
template <int ACT, int GPC, class T>
hipError_t launch_xs(const GemmArgs& a, const TiledParams& p, dim3 grid) {
  if constexpr (!std::is_same<T, SmallTile>::value) {
    return hipErrorNotSupported;
  } else {
    if (a.nf4 || a.glu) return hipErrorNotSupported;
    if (a.qzeros)
      hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_ASYM, T, false, true>), grid, dim3(T::kThreads), T::kLdsBytes, a.stream, p);
    else
      hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_SYM, T, false, true>), grid, dim3(T::kThreads), T::kLdsBytes, a.stream, p);
    return hipGetLastError();
  }
}

template <int ACT, int GPC, class T>
hipError_t launch_fmt(const GemmArgs& a, const TiledParams& p, dim3 grid) {
  if (p.xscale) return launch_xs<ACT, GPC, T>(a, p, grid);
  return a.glu ? launch_glu<ACT, GPC, T, true>(a, p, grid) : launch_glu<ACT, GPC, T, false>(a, p, grid);
}

template <int ACT, class T>
hipError_t launch_gpc(const GemmArgs& a, const TiledParams& p, dim3 grid) {
  switch (a.group_size) {
    case 128: return launch_fmt<ACT, 1, T>(a, p, grid);
    case 64: return launch_fmt<ACT, 2, T>(a, p, grid);
    default: return launch_fmt<ACT, 4, T>(a, p, grid);
  }
}

template <class T>
hipError_t launch_act(const GemmArgs& a, const TiledParams& p, dim3 grid) {
  return a.act == ACT_F16 ? launch_gpc<ACT_F16, T>(a, p, grid) : launch_gpc<ACT_BF16, T>(a, p, grid);
}

}  // namespace

bool tiled_supported(const GemmArgs&) { return true; }

const char* tiled_name(int M, int K, int N) {
  const TiledGeometry g = tiled_geometry(M, K, N);
  if (g.small) return g.S > 1 ? "w4a16_tiled_64x256_splitk" : "w4a16_tiled_64x256";
  return g.S > 1 ? "w4a16_tiled_128x512_splitk" : "w4a16_tiled_128x512";
}

// AWQ: the large tile reads x' from a pre-pass, placed after the split-K partials
size_t tiled_awq_workspace_bytes(int M, int K, int N) {
  const TiledGeometry g = tiled_geometry(M, K, N);
  return g.small ? g.partial_bytes : align256(g.partial_bytes) + align256((size_t)M * K * 2);
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
  p.half = p.NT / 2;
  p.xscale = static_cast<const uint16_t*>(a.xscale);
  if (a.xscale && !g.small) {
    void* xs = static_cast<char*>(a.workspace) + align256(g.partial_bytes);
    const hipError_t e = launch_awq_scale(a.x, a.xscale, a.M, a.K, a.act, xs, a.stream);
    if (e != hipSuccess) return e;
    p.x = static_cast<const uint16_t*>(xs);
    p.xscale = nullptr;
  }
  const dim3 grid(g.tiles_m * g.tiles_n, g.S);
  const hipError_t e = g.small ? launch_act<SmallTile>(a, p, grid) : launch_act<LargeTile>(a, p, grid);
  if (e != hipSuccess || g.S == 1) return e;
  const size_t slice_stride = (size_t)g.tiles_m * g.bm * a.N;
  if (a.glu) {
    const size_t quads = (size_t)a.M * (a.N / 2) / 4;
    hipLaunchKernelGGL(splitk_reduce_glu_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                       a.stream, p.partials, a.M, a.N / 2, g.S, slice_stride, a.out, a.out_dtype);
  } else {
    const size_t quads = (size_t)a.M * a.N / 4;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                       a.stream, p.partials, a.M, a.N, g.S, slice_stride, a.out, a.out_dtype);
  }
  return hipGetLastError();
}

}  // namespace w4a16
