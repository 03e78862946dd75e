// w4a16_tiled_kernel.hpp - the batched W4A16 GEMM kernel (M > 16) and its launchers, as
// templates over the workgroup tile. Each tile shape is instantiated in a translation unit of
// its own (w4a16_tiled_<tile>.hip); w4a16_tiled.hip picks the tile and K split per call.
//
// W4A16 GEMM for batched and prefill shapes (M > 16), where the MFMAs and
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
// k-groups. A small-tile workgroup that has its compute unit to itself runs two sets of four
// waves (two waves per SIMD) that take the two halves of its K range, each with its own ring
// of activation tiles. The second set's fp32 tiles pass through LDS to the first, which adds
// them (in a fixed order) and stores. A second wave per SIMD issues its dequantization while
// the other's MFMAs run (4096x14336 at M=256: 46.2 -> 42.8 us; M=192: 50.5 -> 40.0 us).
//
// Split-K. When the output tiles alone cannot fill the chip, the K range is cut into S
// contiguous slices, one workgroup each. Every slice stores its fp32 partial tile in the
// workspace and a second small kernel sums the S partials in slice order (deterministic)
// into the output.
//
// Loads. Every load is a buffer instruction: the wave-uniform part of the address (block,
// scale group) is a scalar offset, the per-lane part a VGPR fixed for the whole K loop, so
// the loop spends no vector instructions on addresses. A two-stage tile issues block i+1's
// loads over the first four steps of block i's multiply (codes first): a burst right after
// the barrier stalls the issuing waves while the compute unit's address units take it in
// (about 16 cycles per 1 KiB load), with the MFMAs idle. Measured (4096x14336, fp16):
// M=256 44.2 -> 41.4 us.
#pragma once

#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "w4a16_device.hpp"
#include "w4a16_launch.hpp"

namespace w4a16 {
namespace tiled {

// Workgroup tile: MT 32-row MFMA tiles (kBM = 32 MT rows) by WAVES waves of NP 32-column
// strip pairs. Large: 128 x 512, eight waves (two per SIMD) of two pairs. Small: 64 x 256, four
// waves of two pairs, for GEMMs whose large tiles would leave compute units idle (each large
// tile row of M <= 256 is 28-56 tiles at N = 14336).
template <int MT, int WAVES, int NP, int STAGES, int KG = 1>
struct TileShape {
  static constexpr int kStages = STAGES;  // blocks in flight: LDS slots and code register sets
  static constexpr int kMT = MT;
  static constexpr int kBM = 32 * MT;
  static constexpr int kNP = NP;
  static constexpr int kBN = 32 * NP * WAVES;
  static constexpr int kWaves = WAVES;    // waves of one k-group (each owns 64 NP/2 columns)
  static constexpr int kKG = KG;          // k-groups: wave sets that split the tile's K range
  static constexpr int kThreads = 64 * WAVES * KG;
  static constexpr int kADma = kBM / 4 / WAVES;  // 1 KiB direct-to-LDS loads per wave per block
  // next step's A fragments read while this step's MFMAs run, where registers allow it (not
  // in the large tile: 128 accumulators and two waves per SIMD)
  static constexpr bool kPrefetchA = MT <= 2;
  // two stages: the next block's loads are issued over the first four steps of this block's
  // multiply instead of in one burst after the barrier (a burst stalls the issuing waves while
  // the compute unit's address units take it in: about 16 cycles per 1 KiB load)
  static constexpr bool kSpread = STAGES == 2;
  static constexpr size_t kSlotBytes = (size_t)kBM * 256;       // one activation tile
  static constexpr size_t kRingBytes = kStages * kSlotBytes;    // a k-group's ring of tiles
  // the rings, which the later k-groups' fp32 tiles reuse at the end
  static constexpr size_t kRedBytes = (size_t)(KG - 1) * WAVES * MT * NP * 16 * 64 * 4;
  static constexpr size_t kLdsBytes = KG * kRingBytes > kRedBytes ? KG * kRingBytes : kRedBytes;
  static_assert(kADma * WAVES * 4 == kBM, "the tile's rows split evenly over the waves");
};
// Stages: a small tile's block takes about one HBM round trip to multiply, so a workgroup that
// streams many blocks loads three blocks ahead (4096x14336 at M=192/256, 32 blocks per
// workgroup: 47.2 -> 43.7, 48.2 -> 45.4 us against one block ahead); with K split into short
// slices (8 blocks) the deeper prologue costs more than it hides (5-10%), so those keep one
// block ahead. The large tile's 128 accumulators leave registers for one block ahead, which
// its four-times-longer blocks cover. Two k-groups keep one block ahead each: their waves may
// hold at most 256 registers, which three register sets exceed for most formats, and the
// second wave per SIMD covers the latency (three blocks ahead measured no faster).
typedef TileShape<4, 8, 2, 2> LargeTile;
typedef TileShape<2, 4, 2, 2> SmallTile;
typedef TileShape<2, 4, 2, 4> SmallTileDeep;
typedef TileShape<2, 4, 2, 2, 2> SmallTile2;
typedef TileShape<4, 4, 1, 2, 2> MedTile;
constexpr int kDeepBlocks = 16;  // k-blocks per workgroup from which the small tile goes deep

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
};

// workgroup -> output tile, so that tiles sharing weight columns run on the same XCD
__device__ __forceinline__ int tile_of(int b, int G) {
  const int q = G >> 3, r = G & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// s_waitcnt with only the vector-memory counter bounded: vmcnt <= n, the LDS and export
// counters left alone (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8). The
// counter holds at most 63 (a wave stalls at issue beyond that), so larger n wait for 63: a
// stricter, still correct condition.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0, "a count of outstanding instructions");
  constexpr int c = n < 63 ? n : 63;
  __builtin_amdgcn_s_waitcnt((c & 0xF) | ((c >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// GLU: the weight is a fused gate+up projection [K][2 Nh] (gate columns first). A wave's
// first strip pair is two gate strips, its second the matching up strips, and the output is
// h = SiLU(gate) * up, [M][Nh] (with K split, both halves go to the partials and the GLU
// reduce kernel forms h).
//
// Pipeline. The activation tile of a k-block (kBM rows x 128 k) goes from HBM straight to LDS
// (global_load_lds_dwordx4: no registers, no LDS stores, no masking instructions) into one of
// two slots, and the codes, scales and zero-points of the block into one of two register
// sets, one block ahead of the MFMAs. Row r of a slot holds its sixteen 16-byte k-chunks at
// positions c ^ (r % 16), so the A-fragment reads of sixteen consecutive rows fall in sixteen
// different bank groups. Each wave waits for its own copies of the block (vmcnt: only that
// block's code and metadata loads were issued after them) and a barrier makes every wave's
// copies visible; the same barrier frees the other slot, into which the next block loads.
template <int ACT, int GPC, int FMT, class T, bool GLU>
__global__ __launch_bounds__(T::kThreads) void tiled_kernel(TiledParams p) {
  constexpr int kMT = T::kMT, kBM = T::kBM, kWaves = T::kWaves, kADma = T::kADma;
  constexpr int kPairs = T::kNP, kStrips = 2 * T::kNP, kStages = T::kStages, kKG = T::kKG;
  static_assert(kKG == 1 || kKG == 2, "k-groups differ by at most one block");
  static_assert(!GLU || kPairs == 2, "a SwiGLU wave holds a gate pair and an up pair");
  typedef typename ActT<ACT>::type AT;
  constexpr bool ZEROS = FMT == FMT_ASYM;
  // vector-memory instructions one wave issues per block after its activation copies: two
  // code chunks per pair, and per pair and scale group a scale (and a zero word); and in all
  constexpr int kLoadsAfterCopies = kPairs * 2 + kPairs * GPC * (ZEROS ? 2 : 1);
  constexpr int kLoadsPerBlock = kADma + kLoadsAfterCopies;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // [kKG][kStages][kBM][128]

  const int lane = threadIdx.x & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = wave_id / kWaves;              // this wave's k-group
  const int wave = wave_id - kg * kWaves;       // and its column role within the group
  uint16_t* const lds_a = lds + (size_t)kg * kStages * kBM * 128;  // the group's ring
  // k-groups keep their own block pace: each synchronizes its four waves through a counter in
  // LDS instead of the workgroup barrier, so the wave of one group that shares a SIMD with a
  // wave of the other is not held at every block while the other finishes
  __shared__ uint32_t kg_count[kKG];
  if constexpr (kKG > 1) {
    if (threadIdx.x < kKG) kg_count[threadIdx.x] = 0;
    __syncthreads();
  }
  const int tiles = p.tiles_m * p.tiles_n;
  const int t = tile_of(blockIdx.x, tiles);
  const int tm = t % p.tiles_m, tn = t / p.tiles_m;  // neighbours share weight columns
  const int z = blockIdx.y;
  const int K = p.K, N = p.N, M = p.M, KC = p.KC;
  const int m0 = tm * kBM;
  // the workgroup's K slice [kc0, kc1), and this k-group's part of it [kb0, kb0 + nbg): the
  // groups take ceil(n / kKG) contiguous blocks each, the last possibly one fewer (or none)
  const int kc0 = z * p.kps;
  const int kc1 = min(kc0 + p.kps, KC);
  const int nbh = (kc1 - kc0 + kKG - 1) / kKG;
  const int kb0 = kc0 + kg * nbh;
  const int nbg = max(min(kb0 + nbh, kc1) - kb0, 0);
  const int klast = nbg > 0 ? kb0 + nbg - 1 : kc1 - 1;  // loads past the part re-read this block
  const int nt0 = tn * (kWaves * kStrips) + wave * kStrips;  // this wave's first strip
  const int g0 = tn * (kWaves * 2) + wave * 2;                // GLU: its first gate strip
  // strip of pair pr, half h (h = lane/16 % 2), clamped in bounds for loads
  auto strip_of = [&](int pr, int h) {
    return GLU ? min(g0 + h, p.half - 1) + pr * p.half : min(nt0 + 2 * pr + h, p.NT - 1);
  };
  const int shift = 4 * (lane & 7);

  // This lane's part of the activation copies: instruction j of the wave covers tile rows
  // 4 (wave kADma + j) .. +3, lane l row + l/16 and slot position l%16, which holds k-chunk
  // (l%16) ^ (row % 16) of that row (rows past M repeat row M-1 and are never stored; chunks
  // past a ragged K, in the last block only, read out of range and land as zeros, so they
  // add nothing to the sums). Offsets are bytes from the tile's first row.
  const int tile_rows = min(kBM, M - m0);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(p.x + (size_t)m0 * K, (uint32_t)tile_rows * K * 2);
  uint32_t aoff[kADma];
#pragma unroll
  for (int j = 0; j < kADma; ++j) {
    const int row = 4 * (wave * kADma + j) + (lane >> 4);
    const int chunk = (lane & 15) ^ (row & 15);
    aoff[j] = (uint32_t)(min(row, tile_rows - 1) * K + chunk * 8) * 2;
  }
  // RAGGED (K not a multiple of 128) is decided once per launch, outside the K loop: a
  // branch around the copies inside the loop would make the compiler lose count of the loads
  // in flight and wait for the next block's copies before multiplying this one.
  auto copy_a = [&](int kc, int slot, auto ragged) __attribute__((always_inline)) {
    uint16_t* const dst = lds_a + (size_t)slot * kBM * 128 + (size_t)wave * kADma * 512;
#pragma unroll
    for (int j = 0; j < kADma; ++j) {
      uint32_t voff = aoff[j];
      if constexpr (decltype(ragged)::value) {
        const int chunk = (lane & 15) ^ ((4 * (wave * kADma + j) + (lane >> 4)) & 15);
        voff = kc * 128 + chunk * 8 < K ? voff : kOutOfRange;
      }
      buffer_copy16_to_lds(xrs, voff, kc * 256, dst + j * 512);
    }
  };

  struct Regs {
    u4_t b[kPairs][2];         // chunks 16h + c and 32 + 16h + c (h = lane/32, c = lane%16)
    uint32_t s[kPairs][GPC];   // 16-bit scale zero-extended by the load itself
    uint32_t z[kPairs][GPC];
  };
  // The codes: from the block of the wave's first strip (clamped like every strip), this
  // lane's chunk of its strip; strips past N are loaded in bounds and never stored. The scales
  // and zero-points: this lane's column within the group's row.
  const int nbase = GLU ? min(g0, p.half - 1) : min(nt0, p.NT - 1);
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(p.packed + (size_t)nbase * KC * 64, 0xFFFFFFFFu);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(p.scales, (uint32_t)p.NG * N * 2);
  const __amdgpu_buffer_rsrc_t zrs = make_rsrc(ZEROS ? (const void*)p.qzeros : (const void*)p.scales, (uint32_t)p.NG * (N >> 3) * 4);
  uint32_t boff[kPairs], soff[kPairs], zoff[kPairs];
#pragma unroll
  for (int pr = 0; pr < kPairs; ++pr) {
    const int nt = strip_of(pr, (lane >> 4) & 1);
    const int col = nt * 16 + (lane & 15);
    boff[pr] = (uint32_t)(nt - nbase) * (uint32_t)KC * 1024u + (uint32_t)(16 * (lane >> 5) + (lane & 15)) * 16u;
    soff[pr] = (uint32_t)col * 2u;
    zoff[pr] = (uint32_t)(col >> 3) * 4u;
  }
  constexpr int kNT = 2;  // aux bits: non-temporal (the codes are read once)
  auto load_b = [&](Regs& R, int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int pr = 0; pr < kPairs; ++pr) {
      R.b[pr][0] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(brs, boff[pr], kc * 1024, kNT));
      R.b[pr][1] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(brs, boff[pr] + 512, kc * 1024, kNT));
    }
#pragma unroll
    for (int gi = 0; gi < GPC; ++gi) {
      const int g = min(kc * GPC + gi, p.NG - 1);
#pragma unroll
      for (int pr = 0; pr < kPairs; ++pr) {
        R.s[pr][gi] = __builtin_amdgcn_raw_buffer_load_b16(srs, soff[pr], g * N * 2, 0);
        if constexpr (ZEROS) R.z[pr][gi] = __builtin_amdgcn_raw_buffer_load_b32(zrs, zoff[pr], g * (N >> 3) * 4, 0);
      }
    }
  };
  // one block's loads, in a fixed order (activation copies first)
  auto load = [&](Regs& R, int kc, int slot, auto ragged) __attribute__((always_inline)) {
    copy_a(kc, slot, ragged);
    load_b(R, kc);
    __builtin_amdgcn_sched_barrier(0);
  };

  // NF4: the level-pair table after the rings (the launch adds its 1 KiB to the LDS size),
  // complete before any wave reads it
  const uint32_t* const ptab = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lds) + T::kLdsBytes);
  if constexpr (FMT == FMT_NF4) {
    nf4_pair_table_fill(reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(lds) + T::kLdsBytes), p.codebook);
    __syncthreads();
  }

  f16v_t acc[kMT][kPairs];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int pr = 0; pr < kPairs; ++pr)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][pr][i] = 0.f;

  // One 16-k step's operands: the B fragments of both pairs, dequantized in registers, and
  // the A fragments of the kMT row tiles, read from a slot.
  auto dequant_step = [&](const Regs& R, int t, AT (&bf)[kPairs]) __attribute__((always_inline)) {
    const int gi = t / (8 / GPC);
#pragma unroll
    for (int pr = 0; pr < kPairs; ++pr) {
      const uint32_t w = R.b[pr][t & 1][t >> 1];
      const uint32_t sraw = R.s[pr][gi];
      if constexpr (FMT == FMT_NF4) {
        if constexpr (ACT == ACT_F16)
          bf[pr] = dequant_word_nf4_f16_tab(w, ptab, as_h2(sraw * 0x00010001u));
        else
          bf[pr] = dequant_word_nf4_bf16_tab(w, ptab, (float)__builtin_bit_cast(_Float16, (uint16_t)sraw));
      } else {
        const uint32_t zq = ZEROS ? (R.z[pr][gi] >> shift) & 0xFu : 8u;
        if constexpr (ACT == ACT_F16)
          bf[pr] = dequant_word_f16(w, make_zero_f16(zq), as_h2(sraw * 0x00010001u));
        else
          bf[pr] = dequant_word_bf16(w, make_zero_f32(zq, __builtin_bit_cast(float, sraw << 16)));
      }
    }
  };
  auto read_a = [&](int slot, int t, u4_t (&a)[kMT]) __attribute__((always_inline)) {
    const uint16_t* as = lds_a + (size_t)slot * kBM * 128;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {  // row 32 mt + l%32, k-chunk 2 t + l/32 of the block
      const int row = mt * 32 + (lane & 31);
      const int c = (2 * t + (lane >> 5)) ^ (row & 15);
      a[mt] = *reinterpret_cast<const u4_t*>(as + row * 128 + c * 8);
    }
  };

  // Software pipeline over the 8 steps of a block: step t+1's A fragments are read (small
  // tile; the large tile's 128 accumulators leave no room for a second set, so there each is
  // read right before its MFMAs) and its B fragments dequantized while step t's MFMAs run.
  constexpr bool PREFETCH_A = T::kPrefetchA;
  auto compute = [&](const Regs& R, int slot, auto&& issue) __attribute__((always_inline)) {
    u4_t a[kMT];
    AT bf[kPairs];
    read_a(slot, 0, a);
    dequant_step(R, 0, bf);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      u4_t an[kMT];
      AT bn[kPairs];
      if constexpr (T::kSpread) __builtin_amdgcn_sched_barrier(0);
      issue(t);
      if constexpr (T::kSpread) __builtin_amdgcn_sched_barrier(0);
      if (t < 7) {
        if constexpr (PREFETCH_A) read_a(slot, t + 1, an);
        dequant_step(R, t + 1, bn);
      }
      if constexpr (!PREFETCH_A) {
        if (t > 0) read_a(slot, t, a);
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int pr = 0; pr < kPairs; ++pr)
          acc[mt][pr] = mfma32(__builtin_bit_cast(AT, a[mt]), bf[pr], acc[mt][pr]);
      if (t < 7) {
        if constexpr (PREFETCH_A) {
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt) a[mt] = an[mt];
        }
#pragma unroll
        for (int pr = 0; pr < kPairs; ++pr) bf[pr] = bn[pr];
      }
    }
  };

  // Block i is multiplied from slot i % kStages and register set i % kStages while blocks
  // i+1 .. i+kStages-1 load. Loads are unconditional (past the slice they re-read its last
  // block, never used), so every wave issues the same vector-memory instructions per block
  // and the wait count is exact: after block i's copies come its own code loads and the
  // kStages-2 later blocks' loads.
  // Every wave of the workgroup runs nbh block steps (one barrier each); a k-group with one
  // block fewer loads its last block again in its final step and skips the multiply.
  const int nb_min = max(kc1 - kc0 - (kKG - 1) * nbh, 0);  // blocks of the last group
  auto k_loop = [&](auto ragged) __attribute__((always_inline)) {
    Regs R[kStages];
    if constexpr (T::kSpread) {
      // Block i: wait for its codes and copies (issued during block i-1), a barrier, then the
      // multiply, during whose steps 0..3 the codes (step 0) and copies of block i+1 go out.
      constexpr int kDmaPerStep = (kADma + 3) / 4;
      load(R[0], min(kb0, klast), 0, ragged);
      auto issue_next = [&](Regs& Rn, int kc, int slot, int t) __attribute__((always_inline)) {
        if (t == 0) load_b(Rn, kc);
        if (t < 4) {
          uint16_t* const dst = lds_a + (size_t)slot * kBM * 128 + (size_t)wave * kADma * 512;
#pragma unroll
          for (int j = t * kDmaPerStep; j < (t + 1) * kDmaPerStep && j < kADma; ++j) {
            uint32_t voff = aoff[j];
            if constexpr (decltype(ragged)::value) {
              const int chunk = (lane & 15) ^ ((4 * (wave * kADma + j) + (lane >> 4)) & 15);
              voff = kc * 128 + chunk * 8 < K ? voff : kOutOfRange;
            }
            buffer_copy16_to_lds(xrs, voff, kc * 256, dst + j * 512);
          }
        }
      };
      auto step_block = [&](const Regs& Rb, Regs& Rn, int i, int slot, bool live) __attribute__((always_inline)) {
        wait_vmcnt<0>();                          // block i's codes and copies landed
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // no LDS access moves across the barrier
        // every wave's copies of block i are in LDS, and every wave is done with block i-1's
        // slot: the workgroup barrier, or with k-groups this group's count reaching 4 (i + 1)
        // (LDS operations of a wave complete in order, so its count comes after its reads of
        // block i-1, and after its copies of block i by the wait above). The wait is bounded,
        // so a wave always ends.
        if constexpr (kKG == 1) {
          __builtin_amdgcn_s_barrier();
        } else {
          if (lane == 0) __hip_atomic_fetch_add(&kg_count[kg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          const uint32_t target = (uint32_t)kWaves * (uint32_t)(i + 1);
          for (int spin = 0; spin < (1 << 22); ++spin) {
            if (__hip_atomic_load(&kg_count[kg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
            __builtin_amdgcn_s_sleep(1);
          }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
        const int kn = min(kb0 + i + 1, klast);
        if (live) {
          compute(Rb, slot, [&](int t) __attribute__((always_inline)) { issue_next(Rn, kn, slot ^ 1, t); });
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) issue_next(Rn, kn, slot ^ 1, t);
        }
      };
      int i = 0;
      for (; i + 2 <= nb_min; i += 2) {
        step_block(R[0], R[1], i, 0, true);
        step_block(R[1], R[0], i + 1, 1, true);
      }
      // at most two steps remain (one, and the one more of a longer k-group); the step count
      // is the workgroup's, so every wave meets the same barriers
      if (i < nbh) step_block(R[0], R[1], i, 0, i < nbg);
      if (i + 1 < nbh) step_block(R[1], R[0], i + 1, 1, i + 1 < nbg);
    } else {
#pragma unroll
      for (int st = 0; st + 1 < kStages; ++st) load(R[st], min(kb0 + st, klast), st, ragged);
      auto step_block = [&](const Regs& Rb, Regs& Rfree, int i, int slot, bool live) __attribute__((always_inline)) {
        wait_vmcnt<kLoadsAfterCopies + (kStages - 2) * kLoadsPerBlock>();  // block i's copies landed
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // no LDS access moves across the barrier
        __builtin_amdgcn_s_barrier();             // every wave's copies of block i are in LDS, and
                                                  // every wave is done with block i-1's slot
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
        load(Rfree, min(kb0 + i + kStages - 1, klast), (slot + kStages - 1) % kStages, ragged);
        if (live) compute(Rb, slot, [](int) {});
      };
      int i = 0;
      for (; i + kStages <= nb_min; i += kStages) {
#pragma unroll
        for (int u = 0; u < kStages; ++u) step_block(R[u], R[(u + kStages - 1) % kStages], i + u, u, true);
      }
      // at most kStages steps remain (kStages - 1, and the one more of a longer k-group); the
      // step count is the workgroup's, so every wave meets the same barriers
#pragma unroll
      for (int u = 0; u < kStages; ++u)
        if (i + u < nbh) step_block(R[u], R[(u + kStages - 1) % kStages], i + u, u, i + u < nbg);
    }
  };
  if (K % 128 == 0)
    k_loop(std::false_type{});
  else
    k_loop(std::true_type{});
  // the loads still in flight (re-reads past the slice) retire before the wave ends

  // k-groups: the later groups' fp32 tiles go through LDS (over the rings, once every
  // wave's copies have landed and every wave is done with its slots) and group 0 adds them
  // in group order
  if constexpr (kKG > 1) {
    constexpr int kTile = kMT * kPairs * 16 * 64;  // floats per wave
    float* red = reinterpret_cast<float*>(lds);
    wait_vmcnt<0>();
    __syncthreads();
    if (kg > 0) {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int pr = 0; pr < kPairs; ++pr)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            red[(size_t)((kg - 1) * kWaves + wave) * kTile + ((mt * kPairs + pr) * 16 + e) * 64 + lane] =
                acc[mt][pr][e];
    }
    __syncthreads();
    if (GLU && kg > 0) return;
    if (kg == 0) {
#pragma unroll
      for (int g = 1; g < kKG; ++g)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
          for (int pr = 0; pr < kPairs; ++pr)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              acc[mt][pr][e] += red[(size_t)((g - 1) * kWaves + wave) * kTile + ((mt * kPairs + pr) * 16 + e) * 64 + lane];
    }
  }

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
  } else {
    // The tile goes out in slices of 32 rows through LDS (over the rings): each lane writes its
    // values of the slice, converted to the output type, at their row and column; then every
    // thread stores whole 16-byte runs of rows. Written straight from the MFMA layout, a
    // lane's values lie in one column, so the stores were 2 or 4 bytes each (measured: the
    // output of 4096x14336 at M=256 took 6.5 us that way). K split: the slice's fp32 partials.
    constexpr int kBN = T::kBN;
    static_assert(32 * kBN * 4 <= T::kLdsBytes, "a 32-row slice of fp32 values fits in the rings");
    const bool split = p.S > 1;
    const int esz = split || p.out_dtype == 2 ? 4 : 2;  // bytes per stored element
    char* const dst = split ? reinterpret_cast<char*>(p.partials + z * slice_stride) : static_cast<char*>(p.out);
    char* const stage = reinterpret_cast<char*>(lds);
    const int row_bytes = kBN * esz;
    const int chunks_per_row = row_bytes / 16;
    const int col0 = tn * kBN;
    wait_vmcnt<0>();  // no copy (a re-read past the slice) is still landing in the rings
    __syncthreads();  // every wave is done with the rings (and the k-groups' partial sums)
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (kg == 0) {
#pragma unroll
        for (int pr = 0; pr < kPairs; ++pr) {
          const int c = wave * kStrips * 16 + pr * 32 + (lane & 31);  // column in the tile
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);  // row in the slice
            const float v = acc[mt][pr][i];
            char* const e = stage + r * row_bytes + c * esz;
            if (esz == 4)
              *reinterpret_cast<float*>(e) = v;
            else if (p.out_dtype == 0)
              *reinterpret_cast<_Float16*>(e) = (_Float16)v;
            else
              *reinterpret_cast<__bf16*>(e) = (__bf16)v;
          }
        }
      }
      __syncthreads();
      for (int q = threadIdx.x; q < 32 * chunks_per_row; q += T::kThreads) {
        const int rr = q / chunks_per_row, cc = q - rr * chunks_per_row;
        const int m = m0 + mt * 32 + rr;
        const int col = col0 + cc * (16 / esz);  // N is a multiple of 16: a run is all in or out
        if (m < M && col < N)
          *reinterpret_cast<u4_t*>(dst + ((size_t)m * N + col) * esz) =
              *reinterpret_cast<const u4_t*>(stage + rr * row_bytes + cc * 16);
      }
      __syncthreads();
    }
  }
}

template <int ACT, int GPC, class T, bool GLU>
hipError_t launch_glu(const GemmArgs& a, const TiledParams& p, dim3 grid) {
  if (a.nf4)
    hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_NF4, T, GLU>), grid, dim3(T::kThreads),
                       T::kLdsBytes + kNf4PairEntries * 4, a.stream, p);
  else if (a.qzeros)
    hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_ASYM, T, GLU>), grid, dim3(T::kThreads), T::kLdsBytes, a.stream, p);
  else
    hipLaunchKernelGGL((tiled_kernel<ACT, GPC, FMT_SYM, T, GLU>), grid, dim3(T::kThreads), T::kLdsBytes, a.stream, p);
  return hipGetLastError();
}

template <int ACT, int GPC, class T>
hipError_t launch_fmt(const GemmArgs& a, const TiledParams& p, dim3 grid) {
  if constexpr (T::kNP == 2) {
    if (a.glu) return launch_glu<ACT, GPC, T, true>(a, p, grid);
  } else {
    if (a.glu) return hipErrorNotSupported;  // the launcher never sends a SwiGLU call here
  }
  return launch_glu<ACT, GPC, T, false>(a, p, grid);
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


// one instantiation per tile shape, each in its own translation unit
#define W4A16_TILED_EXTERN(T) \
  extern template hipError_t launch_act<T>(const GemmArgs&, const TiledParams&, dim3);
#define W4A16_TILED_INSTANTIATE(T) \
  template hipError_t launch_act<T>(const GemmArgs&, const TiledParams&, dim3);

}  // namespace tiled
}  // namespace w4a16
