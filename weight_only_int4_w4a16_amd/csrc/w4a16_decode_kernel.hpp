// w4a16_decode_kernel.hpp - memory-bound W4A16 GEMM for small M (decode): up to 16 rows per launch.
//
// "INT8 vs INT4 Quantization, in depth", section "Two regimes": at small batch a linear
// layer waits on weight bytes, so this kernel's job is to stream the packed codes once at
// full HBM rate and hide unpacking, dequantization and the MFMAs under the loads.
//
// Work split. A workgroup owns a tile of SW adjacent 16-column strips over the whole K
// range; its W waves split the k-blocks of the tile into W contiguous slices, so every
// wave streams SW independent runs of 1 KiB blocks (the packed layout stores each strip's
// k-blocks contiguously). No wave ever waits for another until the very end, where the W
// partial tiles are summed through LDS in wave order (deterministic, no atomics, no global
// scratch). Workgroups are numbered so that neighbouring tiles, which share the cache lines
// of their scales and zero-points, run on the same XCD (dispatch is round-robin over the
// eight XCDs, each with its own L2).
//
// Pipeline. A wave moves its slice in groups of D k-blocks x SW strips (4 blocks, i.e.
// 4 KiB) with two register sets: group t+1 is in flight while group t is dequantized and
// multiplied, and every group's loads are issued together, so the in-order load counter
// never makes one set wait for the other. The first two groups are issued before the
// activations are written to LDS, so that copy costs no extra memory latency.
//
// Activations. When x fits, each wave copies the k-slice of x it needs into its own LDS
// region (no barrier) and reads the MFMA A fragments from there; one fragment serves all
// SW strips. Otherwise the fragments are loaded with the codes of their k-block (D = 1).
// Rows of the 16-row MFMA tile past M repeat row M-1 and are never stored (an output row
// depends on its own A row only).
#pragma once

#include <type_traits>

#include "w4a16_device.hpp"
#include "w4a16_launch.hpp"

namespace w4a16 {

enum Fmt { FMT_ASYM = 0, FMT_SYM = 1, FMT_NF4 = 2 };

template <int ACT>
struct ActT;
template <>
struct ActT<ACT_F16> { typedef h8_t type; };
template <>
struct ActT<ACT_BF16> { typedef b8_t type; };

struct DecodeParams {
  const uint16_t* x;
  int M, K, N;
  const u4_t* packed;
  const uint16_t* scales;   // act [K/gs][N], or fp16 NF4 absmax
  const uint32_t* qzeros;   // FMT_ASYM only
  const uint16_t* codebook; // FMT_NF4 only
  void* out;
  int out_dtype;
  int KC;        // k-blocks per strip
  int NG;        // scale groups along K (K / group size)
  int W;         // waves per workgroup
  int slice;     // k-blocks per wave (the last waves may get fewer or none)
  int tiles;     // workgroups (= strips / SW)
  int xstride;   // LDS row stride of x in halves (XL)
  int xslice;    // LDS halves reserved per wave for its slice of x (XL)
  int GPC;       // scale groups per 128-k block (128 / group size)
  int half;      // GLU: strips per half of the fused gate+up weight (N / 32)
  const uint16_t* xscale;  // XS: AWQ S^-1 [K] in the activation type
};

constexpr int kXRegs = 2;  // 16-byte chunks of x per lane staged in registers ahead of the weights

// Largest workgroup of an instantiation, 1024 or 512 threads. 1024 caps a lane at 128
// registers (4 waves per SIMD); instantiations that need more (two 16-row tiles, or
// activation fragments held in registers) get 512.
constexpr int decode_block_threads(int MT, int GPC, bool XL) {
  return MT == 1 && XL ? 1024 : 512;
}

// Workgroup size of the persistent instantiations: 512 threads, so a lane may hold the next
// tile's prefetched groups beside the current tile's accumulators (up to 256 registers).
constexpr int decode_persistent_threads = 512;

// k-blocks per pipeline group: four blocks (4 KiB) per group with x in LDS, halved for four
// scale groups per block, and for two with two strips per tile (their scales and zero words
// would not fit the 128 registers of a 1024-thread workgroup); one block when the
// activation fragments travel with the codes.
constexpr int decode_group_blocks(int SW, int GPC, bool XL) {
  return XL ? (GPC == 4 || (GPC == 2 && SW == 2) ? 2 : 4) / SW : 1;
}

// fp16 activations: the affine formats multiply integer-valued operands and NF4 the bare
// codebook levels, and the group scale (absmax) is applied to the fp32 partial sums; with bf16
// activations W_hat is formed in registers with its one rounding to the activation type.
constexpr bool decode_defers_scale(int ACT, int FMT) { return ACT == 0; }

// workgroup -> tile: tiles [start(x), start(x) + count(x)) run on XCD x = blockIdx % 8
__device__ __forceinline__ int tile_of(int b, int G) {
  const int q = G >> 3, r = G & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// PT (persistent tiles): the grid is smaller than the tile count and each workgroup loops
// over tiles blockIdx.x, + gridDim.x, ... with x staged once.
// GLU: the weight is a fused gate+up projection [K][2 Nh] (gate columns first); tile t pairs
// gate strip t with up strip t + Nh/16 and stores h = SiLU(gate) * up, [M][Nh].
// XS (x in LDS only): AWQ input scaling, x' = RN(x * s_inv[k]) as x is staged.
template <int ACT, int MT, int SW, int GPC, int FMT, bool XL, int LB, bool PT, bool GLU, bool XS>
__global__ __launch_bounds__(LB) void decode_kernel(DecodeParams p) {
  typedef typename ActT<ACT>::type AT;
  static_assert(!GLU || SW == 2, "a SwiGLU tile is one gate strip and one up strip");
  static_assert(!XS || XL, "x is scaled as it is staged in LDS");
  constexpr int D = decode_group_blocks(SW, GPC, XL);  // k-blocks per group
  constexpr int SPG = 4 / GPC;        // 32-k steps per scale group
  constexpr bool ZEROS = FMT == FMT_ASYM;
  constexpr bool DEFER = decode_defers_scale(ACT, FMT);
  // fp16 NF4 with x in LDS: the levels come from the workgroup's pair table in LDS, two codes
  // per read, in the word's byte order, and x is staged with each group of eight k in that
  // order, so the levels go into the MFMA without regrouping
  constexpr bool XPAIR = XL && DEFER && FMT == FMT_NF4;

  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = p.K, N = p.N, KC = p.KC, rows = p.M;
  const int kc0 = min(wave * p.slice, KC);
  const int kc1 = min(kc0 + p.slice, KC);
  const int ng = (kc1 - kc0 + D - 1) / D;  // groups of this wave
  const int shift = 4 * (lane & 7);  // nibble of the lane's column in its zero word
  // strip sw of a tile: SW adjacent strips, or (GLU) the gate strip and its up strip
  auto strip_of = [&](int tile, int sw) __attribute__((always_inline)) {
    return GLU ? tile + sw * p.half : tile * SW + sw;
  };

  float* red = reinterpret_cast<float*>(lds);                                   // [W][SW][rows][16]
  uint16_t* xs = reinterpret_cast<uint16_t*>(red + (size_t)p.W * SW * rows * 16) +
                 (size_t)wave * p.xslice;                                        // [rows][xstride]
  // NF4: the level-pair table after every wave's x (16-byte aligned: xslice is a multiple of 8)
  uint32_t* const ptab = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(red + (size_t)p.W * SW * rows * 16) +
                                                     (size_t)p.W * p.xslice);

  // ---- group loads: codes, per-group metadata and (not XL) the A fragments ----
  u4_t bA[D][SW], bB[D][SW];
  uint16_t sA[D][SW][GPC], sB[D][SW][GPC];
  uint32_t zA[D][SW][GPC], zB[D][SW][GPC];
  u4_t xA[XL ? 1 : MT][4], xB[XL ? 1 : MT][4];

  auto load_group = [&](u4_t(&b)[D][SW], uint16_t(&s)[D][SW][GPC], uint32_t(&z)[D][SW][GPC],
                        u4_t(&xf)[XL ? 1 : MT][4], int tile, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kc = min(kc0 + t * D + d, kc1 - 1);  // past the slice: reload its last block
#pragma unroll
      for (int sw = 0; sw < SW; ++sw) {
        const int nt = strip_of(tile, sw);
        const int col = nt * 16 + (lane & 15);  // this lane's column
        b[d][sw] = __builtin_nontemporal_load(p.packed + ((size_t)nt * KC + kc) * 64 + lane);
#pragma unroll
        for (int gi = 0; gi < GPC; ++gi) {
          const int g = min(kc * GPC + gi, p.NG - 1);  // groups past K are never used
          s[d][sw][gi] = p.scales[(size_t)g * N + col];
          if constexpr (ZEROS) z[d][sw][gi] = p.qzeros[(size_t)g * (N >> 3) + (col >> 3)];
        }
      }
      if constexpr (!XL) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = min(mt * 16 + (lane & 15), rows - 1);
          const uint16_t* xr = p.x + (size_t)m * K + (size_t)kc * 128 + (lane >> 4) * 8;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kj = kc * 128 + j * 32 < K ? j * 32 : 0;  // ragged tail: unused, in bounds
            xf[mt][j] = *reinterpret_cast<const u4_t*>(xr + kj);
          }
        }
      }
    }
  };

  f4_t acc[SW][MT];
  f4_t part[SW][DEFER ? MT : 1];  // DEFER: the current scale group's sum of x (q - z)
#pragma unroll
  for (int sw = 0; sw < SW; ++sw)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[sw][mt] = f4_t{0.f, 0.f, 0.f, 0.f};

  if constexpr (FMT == FMT_NF4) {
    nf4_pair_table_fill(ptab, p.codebook);
    __syncthreads();  // the table is complete before any wave reads it
  }

  // GUARD: the group may run past the wave's slice or end inside a ragged last k-block;
  // full groups take the branch-free copy
  auto compute_group = [&](const u4_t(&b)[D][SW], const uint16_t(&s)[D][SW][GPC],
                           const uint32_t(&z)[D][SW][GPC], const u4_t(&xf)[XL ? 1 : MT][4],
                           int t, auto guard) __attribute__((always_inline)) {
    constexpr bool GUARD = decltype(guard)::value;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kc = kc0 + t * D + d;
      if (!GUARD || kc < kc1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!GUARD || kc * 128 + j * 32 < K) {
            AT a[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              u4_t v;
              if constexpr (XL) {
                const int m = min(mt * 16 + (lane & 15), rows - 1);
                v = *reinterpret_cast<const u4_t*>(xs + (size_t)m * p.xstride +
                                                   (kc - kc0) * 128 + j * 32 + (lane >> 4) * 8);
              } else {
                v = xf[mt][j];
              }
              a[mt] = __builtin_bit_cast(AT, v);
            }
            const int gi = j / SPG;
            if constexpr (!DEFER) {
#pragma unroll
              for (int sw = 0; sw < SW; ++sw) {
                const uint32_t w = b[d][sw][j];
                const uint32_t sraw = s[d][sw][gi];
                AT bf;
                if constexpr (FMT == FMT_NF4) {
                  if constexpr (ACT == ACT_F16)
                    bf = dequant_word_nf4_f16_tab(w, ptab, as_h2(sraw * 0x00010001u));
                  else
                    bf = dequant_word_nf4_bf16_tab(w, ptab, (float)__builtin_bit_cast(_Float16, (uint16_t)sraw));
                } else {
                  const uint32_t zq = ZEROS ? (z[d][sw][gi] >> shift) & 0xFu : 8u;
                  if constexpr (ACT == ACT_F16)
                    bf = dequant_word_f16(w, make_zero_f16(zq), as_h2(sraw * 0x00010001u));
                  else
                    bf = dequant_word_bf16(w, make_zero_f32(zq, __builtin_bit_cast(float, sraw << 16)));
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[sw][mt] = mfma16(a[mt], bf, acc[sw][mt]);
              }
            } else {
              // integer-valued operands (affine) or the bare codebook levels (NF4) into the
              // group's partial sum, scaled once when the group's last 32-k step is done
              const bool first = j % SPG == 0, last = j % SPG == SPG - 1;
#pragma unroll
              for (int sw = 0; sw < SW; ++sw) {
                const uint32_t w = b[d][sw][j];
                if constexpr (FMT == FMT_NF4) {
                  AT bq;
                  if constexpr (XPAIR) bq = nf4_levels_f16_pairs(w, ptab);
                  else bq = __builtin_bit_cast(h8_t, nf4_levels_k_order(w, ptab));
#pragma unroll
                  for (int mt = 0; mt < MT; ++mt)
                    part[sw][mt] = mfma16(a[mt], bq, first ? f4_t{0.f, 0.f, 0.f, 0.f} : part[sw][mt]);
                } else {
                  const uint32_t zq = ZEROS ? (z[d][sw][gi] >> shift) & 0xFu : 8u;
                  AT bq, bz;
                  if constexpr (ACT == ACT_F16) {
                    bq = unpack_biased_f16(w);
                    bz = neg_bias_f16(zq);
                  } else {
                    bq = unpack_biased_bf16(w);
                    bz = neg_bias_bf16(zq);
                  }
#pragma unroll
                  for (int mt = 0; mt < MT; ++mt) {
                    part[sw][mt] = mfma16(a[mt], bq, first ? f4_t{0.f, 0.f, 0.f, 0.f} : part[sw][mt]);
                    part[sw][mt] = mfma16(a[mt], bz, part[sw][mt]);
                  }
                }
                if (last) {
                  const uint32_t sraw = s[d][sw][gi];
                  const float sf = ACT == ACT_F16
                                       ? (float)__builtin_bit_cast(_Float16, (uint16_t)sraw)
                                       : __builtin_bit_cast(float, sraw << 16);
#pragma unroll
                  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                      acc[sw][mt][r] = __builtin_fmaf(sf, part[sw][mt][r], acc[sw][mt][r]);
                }
              }
            }
          }
        }
      }
    }
  };
  // a group is full when all its k-blocks lie in the slice and hold four 32-k steps
  const int kfull = K >> 7;  // k-blocks without a ragged tail
  const int kend = kc1 < kfull ? kc1 : kfull;
  auto compute = [&](const u4_t(&b)[D][SW], const uint16_t(&s)[D][SW][GPC],
                     const uint32_t(&z)[D][SW][GPC], const u4_t(&xf)[XL ? 1 : MT][4], int t) __attribute__((always_inline)) {
    if (kc0 + (t + 1) * D <= kend) compute_group(b, s, z, xf, t, std::false_type{});
    else compute_group(b, s, z, xf, t, std::true_type{});
  };

  // Activations: this wave's slice of x, up to kXRegs 16-byte chunks per lane staged in
  // registers; loaded before the first weight groups and written to LDS after them, so the
  // write waits for the x loads only (the load counter retires in order) while the weight
  // groups are still in flight.
  const int kbeg = kc0 * 128;
  const int cpr = (min(kc1 * 128, K) - kbeg) >> 3;  // 16-byte chunks per row of the slice
  const int nchunks = XL ? rows * cpr : 0;
  u4_t xr[kXRegs];
  u4_t xsr[kXRegs];  // XS: the matching chunks of s_inv
  int xoff[kXRegs];
  auto x_load = [&]() __attribute__((always_inline)) {
    if constexpr (XL) {
#pragma unroll
      for (int i = 0; i < kXRegs; ++i) {
        // past the end: a copy of the last chunk, stored again to the same place (harmless,
        // and keeps the store unconditional so the load is not sunk behind the weights)
        const int c = min(lane + 64 * i, nchunks - 1);
        const int m = c / cpr, cc = c - (c / cpr) * cpr;
        xoff[i] = m * p.xstride + cc * 8;
        xr[i] = *reinterpret_cast<const u4_t*>(p.x + (size_t)m * K + kbeg + cc * 8);
        if constexpr (XS) xsr[i] = *reinterpret_cast<const u4_t*>(p.xscale + kbeg + cc * 8);
      }
    }
  };
  auto x_store = [&]() __attribute__((always_inline)) {
    if constexpr (XL) {
#pragma unroll
      for (int i = 0; i < kXRegs; ++i) {
        u4_t v = xr[i];
        if constexpr (XS) v = scale_act8<ACT>(v, xsr[i]);
        if constexpr (XPAIR) v = act8_to_pair_order(v);
        *reinterpret_cast<u4_t*>(xs + xoff[i]) = v;
      }
      // chunks beyond the register-staged ones (slices of several rows)
      for (int c = lane + 64 * kXRegs; c < nchunks; c += 64) {
        const int m = c / cpr, cc = c - (c / cpr) * cpr;
        u4_t v = *reinterpret_cast<const u4_t*>(p.x + (size_t)m * K + kbeg + cc * 8);
        if constexpr (XS) v = scale_act8<ACT>(v, *reinterpret_cast<const u4_t*>(p.xscale + kbeg + cc * 8));
        if constexpr (XPAIR) v = act8_to_pair_order(v);
        *reinterpret_cast<u4_t*>(xs + (size_t)m * p.xstride + cc * 8) = v;
      }
    }
  };

  // ---- sum the W partial tiles of a tile in wave order and store it ----
  auto reduce_store = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int sw = 0; sw < SW; ++sw)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mt * 16 + 4 * (lane >> 4) + r;
          if (m < rows) red[(((size_t)wave * SW + sw) * rows + m) * 16 + (lane & 15)] = acc[sw][mt][r];
          if constexpr (PT) acc[sw][mt][r] = 0.f;
        }
    __syncthreads();
    const int per_wave = SW * rows * 16;
    if constexpr (GLU) {
      // h = SiLU(g) * u = g / (1 + exp(-g)) * u, into the [M][N/2] output
      for (int e = threadIdx.x; e < rows * 16; e += blockDim.x) {
        float g = 0.f, u = 0.f;
        for (int w = 0; w < p.W; ++w) {
          g += red[(size_t)w * per_wave + e];
          u += red[(size_t)w * per_wave + rows * 16 + e];
        }
        const int m = e >> 4, c = e & 15;
        store_out(p.out, (size_t)m * (N >> 1) + (size_t)tile * 16 + c, g / (1.0f + __expf(-g)) * u,
                  p.out_dtype);
      }
    } else {
      for (int e = threadIdx.x; e < per_wave; e += blockDim.x) {
        float v = 0.f;
        for (int w = 0; w < p.W; ++w) v += red[(size_t)w * per_wave + e];
        const int sw = e / (rows * 16);
        const int rem = e - sw * rows * 16;
        const int m = rem >> 4, c = rem & 15;
        store_out(p.out, (size_t)m * N + (size_t)(tile * SW + sw) * 16 + c, v, p.out_dtype);
      }
    }
    if constexpr (PT) __syncthreads();  // the next tile's partials overwrite red
  };

  // Every path below issues its loads unconditionally, so the compiler's wait before each
  // group covers exactly the loads issued before that group's (a load issued on only some
  // paths into a join would make it wait for everything).
  if constexpr (!PT) {
    const int tile = tile_of(blockIdx.x, p.tiles);
    if (ng == 1) {
      x_load();
      load_group(bA, sA, zA, xA, tile, 0);
      x_store();
      compute(bA, sA, zA, xA, 0);
    } else if (ng > 1) {
      x_load();
      load_group(bA, sA, zA, xA, tile, 0);
      load_group(bB, sB, zB, xB, tile, 1);
      x_store();
      int t = 0;
      for (; t + 3 < ng; t += 2) {  // groups t+2 and t+3 exist
        compute(bA, sA, zA, xA, t);
        load_group(bA, sA, zA, xA, tile, t + 2);
        compute(bB, sB, zB, xB, t + 1);
        load_group(bB, sB, zB, xB, tile, t + 3);
      }
      if (t + 2 < ng) {  // three groups left
        compute(bA, sA, zA, xA, t);
        load_group(bA, sA, zA, xA, tile, t + 2);
        compute(bB, sB, zB, xB, t + 1);
        compute(bA, sA, zA, xA, t + 2);
      } else {  // two groups left
        compute(bA, sA, zA, xA, t);
        compute(bB, sB, zB, xB, t + 1);
      }
    }
    reduce_store(tile);
  } else {
    // The workgroup's tiles: blockIdx.x, then every gridDim.x-th (a multiple of 8, so the
    // same XCD). The next tile's first two groups load while the current tile's last
    // groups are multiplied and its partials summed; waves with a single group run a loop
    // of their own, and the last tile's tail, which prefetches nothing, is a separate copy
    // after which the loop exits.
    auto tile_loop = [&](auto single) __attribute__((always_inline)) {
      constexpr bool ONE = decltype(single)::value;
      int bi = blockIdx.x;
      int tile = tile_of(bi, p.tiles);
      x_load();
      load_group(bA, sA, zA, xA, tile, 0);
      if constexpr (!ONE) load_group(bB, sB, zB, xB, tile, 1);
      x_store();
      auto body = [&]() __attribute__((always_inline)) -> int {  // all but the last 2-3 groups
        int t = 0;
        for (; t + 3 < ng; t += 2) {
          compute(bA, sA, zA, xA, t);
          load_group(bA, sA, zA, xA, tile, t + 2);
          compute(bB, sB, zB, xB, t + 1);
          load_group(bB, sB, zB, xB, tile, t + 3);
        }
        return t;
      };
      for (;;) {
        const int bn = bi + (int)gridDim.x;
        if (bn < p.tiles) {
          const int tn = tile_of(bn, p.tiles);
          if constexpr (ONE) {
            compute(bA, sA, zA, xA, 0);
            load_group(bA, sA, zA, xA, tn, 0);
          } else {
            const int t = body();
            if (t + 2 < ng) {
              compute(bA, sA, zA, xA, t);
              load_group(bA, sA, zA, xA, tile, t + 2);
              compute(bB, sB, zB, xB, t + 1);
              compute(bA, sA, zA, xA, t + 2);
              load_group(bA, sA, zA, xA, tn, 0);
              load_group(bB, sB, zB, xB, tn, 1);
            } else {
              compute(bA, sA, zA, xA, t);
              load_group(bA, sA, zA, xA, tn, 0);
              compute(bB, sB, zB, xB, t + 1);
              load_group(bB, sB, zB, xB, tn, 1);
            }
          }
          reduce_store(tile);
          bi = bn;
          tile = tn;
        } else {
          if constexpr (ONE) {
            compute(bA, sA, zA, xA, 0);
          } else {
            const int t = body();
            if (t + 2 < ng) {
              compute(bA, sA, zA, xA, t);
              load_group(bA, sA, zA, xA, tile, t + 2);
              compute(bB, sB, zB, xB, t + 1);
              compute(bA, sA, zA, xA, t + 2);
            } else {
              compute(bA, sA, zA, xA, t);
              compute(bB, sB, zB, xB, t + 1);
            }
          }
          reduce_store(tile);
          break;
        }
      }
    };
    if (ng == 1) tile_loop(std::true_type{});
    else tile_loop(std::false_type{});
  }
}

// Launch the instantiation matching the configuration (defined once per activation type and
// weight format, in the w4a16_decode_<act>_<fmt>.hip units).
template <int ACT, int FMT>
hipError_t decode_dispatch(const DecodeParams& p, const DecodeConfig& c, hipStream_t s);


template <int ACT, int MT, int SW, int GPC, int FMT, bool XL, bool PT, bool GLU, bool XS = false>
hipError_t decode_launch(const DecodeParams& p, const DecodeConfig& c, hipStream_t s) {
  constexpr int LB = PT ? decode_persistent_threads : decode_block_threads(MT, GPC, XL);
  hipLaunchKernelGGL((decode_kernel<ACT, MT, SW, GPC, FMT, XL, LB, PT, GLU, XS>), dim3(c.grid),
                     dim3(64 * c.W), c.lds_bytes, s, p);
  return hipGetLastError();
}

// The instantiated set (all free of register spills on gfx950): tiles of two strips with x
// in LDS, one 16-row tile and one scale group per k-block; every other case one strip.
// AWQ-scaled x (p.xscale set): the plain GEMM shapes with x in LDS, affine formats.
template <int ACT, int FMT, int MT, bool XL, bool PT>
hipError_t decode_dispatch_gpc(const DecodeParams& p, const DecodeConfig& c, hipStream_t s) {
  if (p.xscale) {
    if constexpr (XL && FMT != FMT_NF4) {
      if (c.glu) return hipErrorNotSupported;
      if (c.SW == 2) {
        if constexpr (MT == 1) {
          if (p.GPC == 1) return decode_launch<ACT, 1, 2, 1, FMT, true, PT, false, true>(p, c, s);
        }
        return hipErrorNotSupported;
      }
      if (c.SW != 1) return hipErrorNotSupported;
      switch (p.GPC) {
        case 1: return decode_launch<ACT, MT, 1, 1, FMT, XL, PT, false, true>(p, c, s);
        case 2: return decode_launch<ACT, MT, 1, 2, FMT, XL, PT, false, true>(p, c, s);
        default: return decode_launch<ACT, MT, 1, 4, FMT, XL, PT, false, true>(p, c, s);
      }
    }
    return hipErrorNotSupported;
  }
  if (c.glu) {  // gate/up strip pairs, every group size
    if (c.SW != 2) return hipErrorNotSupported;
    switch (p.GPC) {
      case 1: return decode_launch<ACT, MT, 2, 1, FMT, XL, PT, true>(p, c, s);
      case 2: return decode_launch<ACT, MT, 2, 2, FMT, XL, PT, true>(p, c, s);
      default: return decode_launch<ACT, MT, 2, 4, FMT, XL, PT, true>(p, c, s);
    }
  }
  if constexpr (MT == 1 && XL) {
    if (c.SW == 2) {
      if (p.GPC == 1) return decode_launch<ACT, 1, 2, 1, FMT, true, PT, false>(p, c, s);
      return hipErrorNotSupported;
    }
  }
  if (c.SW != 1) return hipErrorNotSupported;
  switch (p.GPC) {
    case 1: return decode_launch<ACT, MT, 1, 1, FMT, XL, PT, false>(p, c, s);
    case 2: return decode_launch<ACT, MT, 1, 2, FMT, XL, PT, false>(p, c, s);
    default: return decode_launch<ACT, MT, 1, 4, FMT, XL, PT, false>(p, c, s);
  }
}

template <int ACT, int FMT>
hipError_t decode_dispatch(const DecodeParams& p, const DecodeConfig& c, hipStream_t s) {
  if (c.MT == 1 && c.persist) return c.x_in_lds ? decode_dispatch_gpc<ACT, FMT, 1, true, true>(p, c, s)
                                                 : hipErrorNotSupported;  // x in LDS only
  if (c.MT == 1) return c.x_in_lds ? decode_dispatch_gpc<ACT, FMT, 1, true, false>(p, c, s)
                                   : decode_dispatch_gpc<ACT, FMT, 1, false, false>(p, c, s);
  return hipErrorNotSupported;  // launches take at most 16 rows
}

}  // namespace w4a16
