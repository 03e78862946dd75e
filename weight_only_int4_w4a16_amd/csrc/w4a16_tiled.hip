// w4a16_tiled.hip - the batched W4A16 GEMM (M > 16): tile and K-split choice per call, the
// split-K reduce kernels and the launcher. The GEMM kernel itself is a template over the
// workgroup tile (w4a16_tiled_kernel.hpp), instantiated once per tile shape in
// w4a16_tiled_<tile>.hip.
#include <stdlib.h>
#include <string.h>

#include "w4a16_tiled_kernel.hpp"

namespace w4a16 {
namespace tiled {
W4A16_TILED_EXTERN(LargeTile)
W4A16_TILED_EXTERN(SmallTile)
W4A16_TILED_EXTERN(SmallTileDeep)
W4A16_TILED_EXTERN(SmallTile2)
W4A16_TILED_EXTERN(MedTile)
}  // namespace tiled

namespace {

using namespace tiled;

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

enum TileKind { TILE_LARGE = 0, TILE_SMALL = 1, TILE_MED = 2 };

struct TiledGeometry {
  int kind;            // TileKind
  int bm, bn;          // tile rows and columns
  int tiles_m, tiles_n, S, kps;
  int kg;              // k-groups per workgroup (small tile: 1 or 2)
  size_t partial_bytes;
};

// A tile kind with K cut into (about) S contiguous slices of whole k-blocks.
TiledGeometry geometry_for(int M, int K, int N, int kind, int S, int kg) {
  TiledGeometry g;
  g.kg = kg;
  const int KC = ceil_div(K, 128);
  g.kind = kind;
  g.bm = kind == TILE_LARGE ? LargeTile::kBM : kind == TILE_MED ? MedTile::kBM : SmallTile::kBM;
  g.bn = kind == TILE_LARGE ? LargeTile::kBN : kind == TILE_MED ? MedTile::kBN : SmallTile::kBN;
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
// one workgroup per compute unit, 3.4 with two or more, 4.0 with two k-groups (which the
// search offers only where every workgroup has a compute unit to itself).
double modelled_us(const TiledGeometry& g, int M, int N, int cus) {
  const long wgs = (long)g.tiles_m * g.tiles_n * g.S;
  const long per_cu = (wgs + cus - 1) / cus;
  const double wg_flops = 2.0 * g.bm * g.bn * g.kps * 128;
  const double rate = g.kind == TILE_LARGE ? 4.6e6
                      : g.kind == TILE_MED   ? 4.6e6
                      : g.kg == 2            ? 4.0e6
                      : per_cu > 1           ? 3.4e6
                                             : 2.7e6;  // flop per us
  double us = per_cu * (2.5 + wg_flops / rate);
  if (g.S > 1) us += 2.0 * g.S * M * (double)N * 4 / 5e6 + 2.0;
  return us;
}

// W4A16_FORCE_KG=1|2 pins the small tile's k-groups the same way.
int forced_kg() {
  static const int forced = [] {
    const char* v = getenv("W4A16_FORCE_KG");
    if (!v) return 0;
    if (!strcmp(v, "1")) return 1;
    if (!strcmp(v, "2")) return 2;
    return 0;
  }();
  return forced;
}

// W4A16_FORCE_TILE=large|small pins the batched kernel's tile kind (its K split is still
// chosen by the model), for benchmarking one tile against another; read once per process.
int forced_tile() {
  static const int forced = [] {
    const char* v = getenv("W4A16_FORCE_TILE");
    if (!v) return -1;
    if (!strcmp(v, "large")) return (int)TILE_LARGE;
    if (!strcmp(v, "small")) return (int)TILE_SMALL;
    if (!strcmp(v, "med")) return (int)TILE_MED;
    return -1;
  }();
  return forced;
}

// Tile and K split: the large tile (each dequantized word feeds four 32-row tiles) or the small
// one (more workgroups), each with S = 1, 2, 4, ... slices of at least two
// k-blocks and at most four workgroups per compute unit; the model's fastest wins. It
// tracks the measured choices: large wins by 12-21% at 8192x28672 M=256, 28672x8192 M=256,
// 8192x10240 M=512 and loses by 7-13% at 4096x4096 M=512 and 1024 (split-K partials
// outweigh its rate); small matrices past 16 rows split K deeply (4096x4096 at M=17: S=16).
//
// The choice depends on the shape only (never on the SwiGLU epilogue), so the workspace a
// caller sizes for a shape is the workspace the launch uses.
TiledGeometry tiled_geometry(int M, int K, int N, bool allow_forced = true) {
  const int cus = cu_count_tiled();
  const int KC = ceil_div(K, 128);
  const int f = allow_forced ? forced_tile() : -1, fkg = allow_forced ? forced_kg() : 0;
  TiledGeometry best{};
  double best_us = -1;
  for (int kind = 0; kind < 3; ++kind) {
    if (f >= 0 && kind != f) continue;
    if (kind == TILE_MED && f != TILE_MED) continue;
    for (int kg = kind == TILE_MED ? 2 : 1; kg <= (kind == TILE_LARGE ? 1 : 2); ++kg) {
      if (fkg && kind == TILE_SMALL && kg != fkg) continue;
      for (int S = 1; S == 1 || KC / S >= 2 * kg; S *= 2) {
        const TiledGeometry g = geometry_for(M, K, N, kind, S, kg);
        const long wgs = (long)g.tiles_m * g.tiles_n * g.S;
        if (S > 1 && wgs > 4L * cus) break;
        if (kg == 2 && wgs > cus) break;  // two k-groups only where one workgroup per CU is left
        if (kind == TILE_MED && S > 1) break;
        const double us = modelled_us(g, M, N, cus);
        if (best_us < 0 || us < best_us) {
          best = g;
          best_us = us;
        }
      }
    }
  }
  // a forced tile or k-group count with no valid launch for this shape: the model's choice
  if (best_us < 0 && allow_forced) return tiled_geometry(M, K, N, false);
  return best;
}

// The tile a launch runs: the model's choice, with one swap that never changes the workspace
// (both sides run with K unsplit). Where dequantization is dear (groups of 32 or 64 scale
// pairs per block, or NF4's 16-level lookup, blocks of 64) and the model picks the small tile
// with two k-groups and no K split, the medium tile, whose waves own 128 rows and feed each
// dequantized word to twice the MFMAs, takes over from 192 rows on (4096x14336 at M=256:
// g32 44.7 -> 41.4 us, NF4 54.0 -> 45.4 us; g128 41.6 -> 40.6 us, within run-to-run noise,
// and M=128/192 slower, so those keep the small tile). The medium tile holds one strip pair
// per wave, so a SwiGLU call keeps the small tile.
TiledGeometry launch_geometry(int M, int K, int N, int group_size, bool glu) {
  TiledGeometry g = tiled_geometry(M, K, N);
  const bool forced_med = g.kind == TILE_MED;
  if (glu && forced_med) return geometry_for(M, K, N, TILE_SMALL, 1, 2);
  if (!glu && group_size <= 64 && M >= 192 && g.kind == TILE_SMALL && g.kg == 2 && g.S == 1)
    return geometry_for(M, K, N, TILE_MED, 1, 2);
  return g;
}

}  // namespace

bool tiled_supported(const GemmArgs&) { return true; }

const char* tiled_name(int M, int K, int N, int group_size) {
  const TiledGeometry g = launch_geometry(M, K, N, group_size, false);
  if (g.kind == TILE_MED) return "w4a16_tiled_128x128_kg2";
  if (g.kind == TILE_SMALL && g.kg == 2)
    return g.S > 1 ? "w4a16_tiled_64x256_kg2_splitk" : "w4a16_tiled_64x256_kg2";
  if (g.kind == TILE_SMALL) return g.S > 1 ? "w4a16_tiled_64x256_splitk" : "w4a16_tiled_64x256";
  return g.S > 1 ? "w4a16_tiled_128x512_splitk" : "w4a16_tiled_128x512";
}

// AWQ: the activation tiles go from HBM to LDS untouched, so the kernel reads x' from a
// pre-pass, placed after the split-K partials
size_t tiled_awq_workspace_bytes(int M, int K, int N) {
  const TiledGeometry g = tiled_geometry(M, K, N);
  return align256(g.partial_bytes) + align256((size_t)M * K * 2);
}

size_t tiled_workspace_bytes(int M, int K, int N) {
  const TiledGeometry g = tiled_geometry(M, K, N);
  return g.partial_bytes;
}

hipError_t launch_tiled(const GemmArgs& a) {
  const TiledGeometry g = launch_geometry(a.M, a.K, a.N, a.group_size, a.glu);
  // never write past the caller's scratch: the split-K partials, then (AWQ) x'
  const size_t need = (a.xscale ? align256(g.partial_bytes) + align256((size_t)a.M * a.K * 2) : g.partial_bytes);
  if (need && (!a.workspace || a.workspace_bytes < need)) return hipErrorInvalidValue;
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
  if (a.xscale) {
    void* xs = static_cast<char*>(a.workspace) + align256(g.partial_bytes);
    const hipError_t e = launch_awq_scale(a.x, a.xscale, a.M, a.K, a.act, xs, a.stream);
    if (e != hipSuccess) return e;
    p.x = static_cast<const uint16_t*>(xs);
  }
  const dim3 grid(g.tiles_m * g.tiles_n, g.S);
  const hipError_t e = g.kind == TILE_LARGE      ? launch_act<LargeTile>(a, p, grid)
                       : g.kind == TILE_MED        ? launch_act<MedTile>(a, p, grid)
                       : g.kg == 2                 ? launch_act<SmallTile2>(a, p, grid)
                       : g.kps >= kDeepBlocks      ? launch_act<SmallTileDeep>(a, p, grid)
                                                   : launch_act<SmallTile>(a, p, grid);
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
