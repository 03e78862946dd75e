// w4a16_decode.hip - host side of the decode kernel (w4a16_decode_kernel.hpp): launch
// geometry and dispatch on activation type and weight format.
#include <stdio.h>
#include <stdlib.h>

#include "w4a16_decode_kernel.hpp"

namespace w4a16 {

// The kernels are instantiated in the w4a16_decode_<act>_<fmt>.hip units, one per activation
// type and weight format; declared here so this unit does not compile them all again.
extern template hipError_t decode_dispatch<ACT_F16, FMT_ASYM>(const DecodeParams&, const DecodeConfig&, hipStream_t);
extern template hipError_t decode_dispatch<ACT_F16, FMT_SYM>(const DecodeParams&, const DecodeConfig&, hipStream_t);
extern template hipError_t decode_dispatch<ACT_F16, FMT_NF4>(const DecodeParams&, const DecodeConfig&, hipStream_t);
extern template hipError_t decode_dispatch<ACT_BF16, FMT_ASYM>(const DecodeParams&, const DecodeConfig&, hipStream_t);
extern template hipError_t decode_dispatch<ACT_BF16, FMT_SYM>(const DecodeParams&, const DecodeConfig&, hipStream_t);
extern template hipError_t decode_dispatch<ACT_BF16, FMT_NF4>(const DecodeParams&, const DecodeConfig&, hipStream_t);

namespace {

int cu_count() {
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

constexpr size_t kXldsBytes = 128 * 1024;  // largest x staged in LDS per workgroup
constexpr size_t kMaxLds = 160 * 1024;     // LDS per compute unit on gfx950

// Launch geometry for a given tile width SW and wave count W per workgroup; `extra` LDS bytes
// follow the activations (the NF4 level-pair table).
DecodeConfig geometry(int M, int K, int N, bool x_in_lds, int SW, int W, size_t extra) {
  DecodeConfig c;
  c.KC = ceil_div(K, 128);
  c.NT = N / 16;
  c.rows = M < 16 ? M : 16;
  c.MT = ceil_div(c.rows, 16);
  c.x_in_lds = x_in_lds;
  c.SW = SW;
  c.tiles = c.NT / SW;
  c.grid = c.tiles;
  c.persist = false;
  c.glu = false;
  c.slice = ceil_div(c.KC, W);
  c.W = ceil_div(c.KC, c.slice);  // drop waves left without blocks
  c.xstride = c.slice * 128 + 8;
  c.xslice = x_in_lds ? c.rows * c.xstride : 0;
  c.lds_bytes = (size_t)c.W * SW * c.rows * 16 * 4 + (size_t)c.W * c.xslice * 2 + extra;
  c.workspace_bytes = 0;
  return c;
}

// Pick SW and W. A launch of `tiles` workgroups of W waves runs in
// ceil(tiles / (CUs * workgroups per CU)) rounds (resident waves per compute unit: 16 for
// 1024-thread instantiations, which stay within 128 registers, else 8); each round costs
// about the groups one wave streams plus a fixed latency of about two groups. The cheapest
// choice wins, wider tiles (shared activation fragments and scale lines) and then more
// waves on ties. Two-strip tiles exist for x in LDS, one 16-row tile and one scale group per
// k-block (the register-spill-free instantiations).
//
// Persistent workgroups. Every round restages all of x in LDS (rows x K x 2 bytes, against
// SW x 8 x K bytes of codes per tile), so from 8 rows on, when the best launch above needs
// more than one round, the workgroups persist instead: 512 threads (up to 256 registers,
// 8 waves per compute unit), one per resident slot (a multiple of 8), each taking every
// grid-th tile with x staged once. A tile then costs its groups plus one (the next tile's
// loads are in flight while the wave partials are summed), the launch one more. Measured:
// 4096x28672 at M=16 33.5 -> 23.0 us, 8192x57344 at M=8 77.9 -> 54.7 us, 8192x10240 at M=8
// 21.0 -> 18.2 us; at M=4 the same rule would lose (4096x28672 17.3 -> 20.4 us).
// W4A16_DECODE_GEOMETRY=SW,W limits the choice below to tiles of SW strips and W waves per
// workgroup where such a launch exists (for benchmarking geometries against each other); read
// once per process.
struct ForcedGeometry { int sw, w; };
ForcedGeometry forced_geometry() {
  static const ForcedGeometry f = [] {
    ForcedGeometry r{0, 0};
    const char* v = getenv("W4A16_DECODE_GEOMETRY");
    if (v && sscanf(v, "%d,%d", &r.sw, &r.w) != 2) r = ForcedGeometry{0, 0};
    return r;
  }();
  return f;
}

DecodeConfig choose(int M, int K, int N, int group_size, bool x_in_lds, bool glu, size_t extra,
                    bool allow_forced = true) {
  const int KC = ceil_div(K, 128), NT = N / 16;
  const ForcedGeometry fg = allow_forced ? forced_geometry() : ForcedGeometry{0, 0};
  const int rows = M < 16 ? M : 16, MT = ceil_div(rows, 16);
  const int GPC = 128 / group_size;
  const int cus = cu_count();
  const int wmax = decode_block_threads(MT, GPC, x_in_lds) / 64;
  const int waves_per_cu = wmax == 16 ? 16 : 8;
  DecodeConfig best{}, pbest{};
  long best_cost = -1, best_rounds = 0, pbest_cost = -1;
  for (int SW = 2; SW >= (glu ? 2 : 1); SW >>= 1) {  // SwiGLU tiles: a gate and an up strip
    if (NT % SW) continue;
    if (SW > 1 && !glu && !(x_in_lds && MT == 1 && GPC == 1)) continue;
    const int D = decode_group_blocks(SW, GPC, x_in_lds);  // k-blocks per pipeline group
    if (fg.sw && fg.sw != SW) continue;
    for (int W = wmax; W >= 1; W >>= 1) {
      if (W > 1 && W > KC / D) continue;  // every wave streams at least one whole group
      if (fg.w && fg.w != W) continue;
      DecodeConfig c = geometry(M, K, N, x_in_lds, SW, W, extra);
      // the same number of groups per wave with whole groups only, on fewer waves where the
      // slice would end in a partial group (14336 = 112 blocks: 14 waves of 8, not 16 of 7;
      // measured 9.6 -> 9.0 us at M=1)
      if (c.slice % D) {
        const int whole = ceil_div(c.slice, D) * D;
        c = geometry(M, K, N, x_in_lds, SW, ceil_div(KC, whole), extra);
      }
      c.glu = glu;
      if (c.lds_bytes > kMaxLds) continue;
      int wg_per_cu = waves_per_cu / W;
      const int by_lds = (int)(kMaxLds / c.lds_bytes);
      if (by_lds < wg_per_cu) wg_per_cu = by_lds;
      if (wg_per_cu < 1) wg_per_cu = 1;
      const long rounds = ceil_div(c.tiles, cus * wg_per_cu);
      const long cost = rounds * (ceil_div(c.slice, D) + 2);
      // ties: the choice that keeps more compute units busy, counting three quarters of them
      // as all, so that the wider tile (tried first) keeps a tie there (4096x6144: two-strip
      // tiles on 192 units against one-strip tiles on 256 measured 5.11 / 5.49 against 5.21 /
      // 6.48 us at M=1 / 4; with 128 two-strip tiles the one-strip tiles stay faster)
      auto busy_of = [&](int tiles) { const int b = tiles < cus ? tiles : cus; return 4 * b >= 3 * cus ? cus : b; };
      const int busy = busy_of(c.tiles);
      const int best_busy = busy_of(best.tiles);
      if (best_cost < 0 || cost < best_cost || (cost == best_cost && busy > best_busy)) {
        best = c;
        best_cost = cost;
        best_rounds = rounds;
      }
      if (x_in_lds && W <= decode_persistent_threads / 64) {
        int per_cu = 8 / W;
        if (by_lds < per_cu) per_cu = by_lds;
        if (per_cu < 1) per_cu = 1;
        const int grid = cus * per_cu / 8 * 8;
        if (grid >= 8 && grid < c.tiles) {
          const long pcost = ceil_div(c.tiles, grid) * (ceil_div(c.slice, D) + 1) + 1;
          if (pbest_cost < 0 || pcost < pbest_cost) {
            pbest = c;
            pbest.grid = grid;
            pbest.persist = true;
            pbest_cost = pcost;
          }
        }
      }
    }
  }
  if (fg.sw) {  // a forced geometry as it is, or the unforced choice if it does not exist
    return best_cost >= 0 ? best : choose(M, K, N, group_size, x_in_lds, glu, extra, false);
  }
  if (rows >= 8 && best_rounds > 1 && pbest_cost >= 0) return pbest;
  // One row of x: the waves of a tile stream four groups each where the tile allows it. The
  // model above counts launch rounds, but a wave keeps only two groups in flight, so shorter,
  // more numerous waves keep more loads outstanding, and below four groups a wave's prologue
  // (staging its slice of x) and epilogue are no longer amortized. Measured at M=1
  // (8192x57344: 16, 8, 4, 2 groups per wave 46.4, 43.1, 40.6, 51.6 us; the other benchmarked
  // shapes already stream four to eight groups per wave at their best geometry).
  if (rows == 1 && x_in_lds) {
    const int D = decode_group_blocks(best.SW, GPC, x_in_lds);
    while (best.W * 2 <= wmax && ceil_div(ceil_div(KC, best.W * 2), D) >= 4) {
      DecodeConfig c = geometry(M, K, N, x_in_lds, best.SW, best.W * 2, extra);
      c.glu = glu;
      if (c.lds_bytes > kMaxLds) break;
      best = c;
    }
  }
  return best;
}

}  // namespace

// x goes to LDS when it fits beside the reduction area; otherwise it is read per k-block
// (every instantiated configuration exists for both activation types)
DecodeConfig decode_config(int M, int K, int N, int group_size, bool glu, size_t extra_lds) {
  const int rows = M < 16 ? M : 16;
  const size_t xbytes = (size_t)rows * ceil_div(K, 128) * 128 * 2;
  if (xbytes <= kXldsBytes) {
    const DecodeConfig c = choose(M, K, N, group_size, true, glu, extra_lds);
    if (c.W > 0) return c;
  }
  return choose(M, K, N, group_size, false, glu, extra_lds);
}

namespace {

// AWQ input scaling as a pre-pass (decode launches whose x does not fit in LDS, batched
// launches on the large tile): x' = RN(x * s_inv[k]) written to the workspace, one 16-byte
// chunk (8 activations) per thread; the plain kernel then reads x'.
template <int ACT>
__global__ __launch_bounds__(256) void awq_scale_kernel(const u4_t* __restrict__ x,
                                                        const u4_t* __restrict__ s_inv, int K8,
                                                        size_t chunks, u4_t* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < chunks) out[i] = scale_act8<ACT>(x[i], s_inv[i % K8]);
}

}  // namespace

hipError_t launch_awq_scale(const void* x, const void* s_inv, int rows, int K, int act, void* out,
                            hipStream_t stream) {
  const size_t chunks = (size_t)rows * (K / 8);
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(act == ACT_F16 ? awq_scale_kernel<ACT_F16> : awq_scale_kernel<ACT_BF16>,
                     dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const u4_t*>(x), static_cast<const u4_t*>(s_inv), K / 8, chunks,
                     static_cast<u4_t*>(out));
  return hipGetLastError();
}

// Rows of x one launch takes: at most 16, one MFMA tile (larger M goes to the batched
// kernel; a caller of this launcher with more rows gets several launches).
DecodeConfig decode_launch_config(int M, int K, int N, int group_size, bool glu, size_t extra_lds = 0) {
  return decode_config(M < 16 ? M : 16, K, N, group_size, glu, extra_lds);
}

const char* decode_name(int M, int K, int N, int group_size, int act) {
  (void)act;
  const DecodeConfig c = decode_launch_config(M, K, N, group_size, false);
  if (c.persist) return c.SW == 1 ? "w4a16_decode_sw1_persist" : "w4a16_decode_sw2_persist";
  return c.SW == 1 ? "w4a16_decode_sw1" : "w4a16_decode_sw2";
}

size_t decode_awq_workspace_bytes(int M, int K, int N, int group_size) {
  const DecodeConfig c = decode_launch_config(M, K, N, group_size, false);
  return c.x_in_lds ? 0 : align256((size_t)c.rows * K * 2);
}

hipError_t launch_decode(const GemmArgs& a) {
  const size_t osz = a.out_dtype == 2 ? 4 : 2;
  for (int r0 = 0; r0 < a.M;) {
    // NF4 reads its levels from a pair table after x
    const size_t extra = a.nf4 ? (size_t)kNf4PairEntries * 4 : 0;
    const DecodeConfig c = decode_launch_config(a.M - r0, a.K, a.N, a.group_size, a.glu, extra);
    const int rows = c.rows;
    DecodeParams p;
    p.x = static_cast<const uint16_t*>(a.x) + (size_t)r0 * a.K;
    p.xscale = nullptr;
    if (a.xscale && c.x_in_lds) {
      p.xscale = static_cast<const uint16_t*>(a.xscale);
    } else if (a.xscale) {  // x' to the workspace (launches run in order on the stream)
      if (!a.workspace || a.workspace_bytes < (size_t)rows * a.K * 2) return hipErrorInvalidValue;
      const hipError_t e = launch_awq_scale(p.x, a.xscale, rows, a.K, a.act, a.workspace, a.stream);
      if (e != hipSuccess) return e;
      p.x = static_cast<const uint16_t*>(a.workspace);
    }
    p.M = rows;
    p.K = a.K;
    p.N = a.N;
    p.packed = reinterpret_cast<const u4_t*>(a.packed);
    p.scales = static_cast<const uint16_t*>(a.scales);
    p.qzeros = a.qzeros;
    p.codebook = a.codebook;
    p.out = static_cast<char*>(a.out) + (size_t)r0 * (a.glu ? a.N / 2 : a.N) * osz;
    p.out_dtype = a.out_dtype;
    p.KC = c.KC;
    p.NG = a.K / a.group_size;
    p.W = c.W;
    p.slice = c.slice;
    p.tiles = c.tiles;
    p.xstride = c.xstride;
    p.xslice = c.xslice;
    p.GPC = 128 / a.group_size;
    p.half = a.N / 32;
    hipError_t e;
    const int fmt = a.nf4 ? FMT_NF4 : a.qzeros ? FMT_ASYM : FMT_SYM;
    if (a.act == ACT_F16) {
      e = fmt == FMT_NF4 ? decode_dispatch<ACT_F16, FMT_NF4>(p, c, a.stream)
        : fmt == FMT_ASYM ? decode_dispatch<ACT_F16, FMT_ASYM>(p, c, a.stream)
                          : decode_dispatch<ACT_F16, FMT_SYM>(p, c, a.stream);
    } else {
      e = fmt == FMT_NF4 ? decode_dispatch<ACT_BF16, FMT_NF4>(p, c, a.stream)
        : fmt == FMT_ASYM ? decode_dispatch<ACT_BF16, FMT_ASYM>(p, c, a.stream)
                          : decode_dispatch<ACT_BF16, FMT_SYM>(p, c, a.stream);
    }
    if (e != hipSuccess) return e;
    r0 += rows;
  }
  return hipSuccess;
}

}  // namespace w4a16
