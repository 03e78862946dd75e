// w4a16_skinny.hip - W4A16 GEMM for mid-size batches (17 to 64 rows): the weight bytes still
// bound the time, but each weight now feeds enough rows that the activation reads and the
// MFMAs matter too.
//
// "INT8 vs INT4 Quantization, in depth", section "Two regimes": below the crossover batch a
// layer waits on its weight bytes, so the codes must stream at full rate while every row of x
// is multiplied on-chip; "4.3 Weight-only INT4", section 4 (Marlin): the speedup holds near
// its ceiling at batch 16-32 only if the kernel keeps enough loads in flight.
//
// Work split. A workgroup owns two pairs of 16-column strips (64 columns) and up to 32 MT rows
// over the whole K range; its eight waves take eight contiguous k-block slices of K. No wave
// waits for another until the end, where the eight partial tiles are summed through LDS in
// wave order (deterministic, no global partials, no second launch).
//
// Two load streams per wave, each sized for where it comes from.
// - Codes (HBM): whole 16-byte chunks, two per lane per pair and block, into two register
//   sets: the next block (4 KiB per wave) is in flight while one is multiplied. Deeper
//   prefetch loses here: with three blocks ahead every wave has asked for most of its slice
//   at once, the chip's requests arrive in no useful order, and a wave's first block waits
//   behind all of them (4096x14336 at M=32: 15.6 us with three blocks ahead, 16.5 with two,
//   12.8 with one). One block ahead is still about 7 MiB in flight across the chip.
// - Activations (L2: every workgroup reads all of x): half blocks (32 MT rows x 64 k) copied
//   from global memory straight into a per-wave pair of LDS slots (global_load_lds_dwordx4,
//   eight rows of 128 bytes per instruction, so every request is a whole cache line). Row r of a slot
//   holds its eight 16-byte chunks at positions c ^ (r/2 % 8), so the fragment reads of
//   sixteen consecutive rows fall in sixteen different bank groups. Only the wave that fills
//   a slot reads it, so its own load counter orders the two and no barrier is needed.
//
// Operands. v_mfma_f32_32x32x16_{f16,bf16}: lane l multiplies row l%32 of a row tile with
// column l%32 of a strip pair, k = 16t + 8(l/32) .. +8 at step t of a 128-k block. The codes of
// those k are word t/2 of the packed chunk lane 16((2t + l/32) % 4) + l%16 owns (as in the
// batched kernel). Each word is dequantized once per workgroup and used for MT row tiles.
#include <stdlib.h>

#include <type_traits>

#include "w4a16_device.hpp"
#include "w4a16_launch.hpp"

namespace w4a16 {

namespace {

enum Fmt { FMT_ASYM = 0, FMT_SYM = 1, FMT_NF4 = 2 };

template <int ACT>
struct ActT;
template <>
struct ActT<ACT_F16> { typedef h8_t type; };
template <>
struct ActT<ACT_BF16> { typedef b8_t type; };

struct SkinnyParams {
  const uint16_t* x;
  int M, K, N;
  const u4_t* packed;
  const uint16_t* scales;
  const uint32_t* qzeros;
  const uint16_t* codebook;
  void* out;
  int out_dtype;
  int KC, NT, NG;   // k-blocks, 16-column strips, scale groups along K
  int slice;        // k-blocks per wave
  int half;         // GLU: strips per half of the fused gate+up weight (NT / 2)
};

// waves per workgroup: eight for one or two row tiles; four for four (128 rows: a wave's
// accumulators fill the AGPRs of a SIMD, and four waves' activation slots fill the LDS)
constexpr int skinny_waves(int MT) { return MT == 4 ? 4 : 8; }
constexpr int kSkinnyPairs = 2;
constexpr int kCodeSets = 2;  // code register sets: the block multiplied and the next in flight
// activation slots (half blocks) per wave: the half multiplied and the next one in flight
constexpr int skinny_slots(int MT) { (void)MT; return 2; }
constexpr int skinny_slot_halves(int MT) { return 32 * MT * 64; }
constexpr int skinny_ring_halves(int MT) { return skinny_slots(MT) * skinny_slot_halves(MT); }
// the waves' activation slots, then the NF4 level-pair table (1 KiB, filled for NF4 only)
constexpr size_t skinny_lds_bytes(int MT) {
  return (size_t)skinny_waves(MT) * skinny_ring_halves(MT) * 2 + kNf4PairEntries * 4;
}

// s_waitcnt with only the vector-memory counter bounded (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int n>
__device__ __forceinline__ void skinny_wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt holds 0..63");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// GLU: pair 0 holds two gate strips and pair 1 the matching up strips; the output is
// h = SiLU(gate) * up, [M][N/2].
template <int ACT, int GPC, int FMT, int MT, bool GLU>
__global__ __launch_bounds__(64 * skinny_waves(MT)) void skinny_kernel(SkinnyParams p) {
  typedef typename ActT<ACT>::type AT;
  constexpr int W = skinny_waves(MT), NP = kSkinnyPairs, RB = kCodeSets, RA = skinny_slots(MT);
  constexpr bool ZEROS = FMT == FMT_ASYM;
  constexpr int SLOT = skinny_slot_halves(MT);
  constexpr int RING = skinny_ring_halves(MT);
  constexpr int KX = 4 * MT;                            // copy instructions per slot
  constexpr int KB = NP * 2 + NP * GPC * (ZEROS ? 2 : 1);  // load instructions per code block
  constexpr int TILE = MT * NP * 1024;                  // fp32 partial sums per wave
  static_assert(TILE * 4 <= RING * 2, "a wave's partial tile fits in its ring");
  static_assert(RA % 2 == 0 && (2 * RB) % RA == 0, "the unrolled step count covers both rings");
  constexpr int U = 2 * RB;                             // half blocks per unrolled pass
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // [W][RA][32 MT][64]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = p.K, N = p.N, M = p.M, KC = p.KC;
  const int tn = blockIdx.x;
  const int m0 = blockIdx.y * 32 * MT;
  const int kc0 = min(wave * p.slice, KC);
  const int kc1 = min(kc0 + p.slice, KC);
  const int nb = kc1 - kc0;
  const int nh = 2 * nb;  // half blocks of this wave
  uint16_t* const ring = lds + (size_t)wave * RING;
  const int h16 = (lane >> 4) & 1;  // which strip of a pair this lane's column is in
  // strip of pair pr for this lane, clamped in bounds for loads (never stored past N)
  auto strip_of = [&](int pr) __attribute__((always_inline)) {
    return GLU ? min(2 * tn + h16, p.half - 1) + pr * p.half : min(tn * 2 * NP + 2 * pr + h16, p.NT - 1);
  };
  const int shift = 4 * (lane & 7);
  const int c0 = 16 * (lane >> 5) + (lane & 15);  // first packed chunk of this lane
  int col[NP];
#pragma unroll
  for (int pr = 0; pr < NP; ++pr) col[pr] = strip_of(pr) * 16 + (lane & 15);

  // activation copies: instruction j of a slot covers its rows 8j .. 8j+7, lane l row
  // 8j + l/8 and position l%8, which holds 16-byte chunk (l%8) ^ (row/2 % 8) of the row's half
  // block (rows past M repeat row M-1 and are never stored). Offsets are bytes from the tile's
  // first row and the slice's first k; each half block adds 128 bytes (a scalar offset).
  // RAGGED (K not a multiple of 128) is decided once per launch, outside the K loop: a branch
  // around the copies inside the loop would make the compiler lose count of the loads in
  // flight and wait for every one of them before multiplying.
  const int tile_rows = min(32 * MT, M - m0);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(p.x + (size_t)m0 * K, (uint32_t)tile_rows * K * 2);
  uint32_t xoff[KX];
#pragma unroll
  for (int j = 0; j < KX; ++j) {
    const int row = 8 * j + (lane >> 3);
    xoff[j] = (uint32_t)(min(row, tile_rows - 1) * K + kc0 * 128 + ((lane & 7) ^ ((row >> 1) & 7)) * 8) * 2;
  }
  auto load_x = [&](int h, int slot, auto ragged) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < KX; ++j) {
      uint32_t voff = xoff[j];
      if constexpr (decltype(ragged)::value) {  // chunks past K read out of range: zeros
        const int row = 8 * j + (lane >> 3);
        const int k = kc0 * 128 + 64 * h + ((lane & 7) ^ ((row >> 1) & 7)) * 8;
        voff = k < K ? voff : kOutOfRange;
      }
      buffer_copy16_to_lds(xrs, voff, 128 * h, ring + slot * SLOT + j * 512);
    }
  };

  struct Codes {
    u4_t b[NP][2];          // chunks c0 and c0 + 32 of the lane's strip
    uint32_t s[NP][GPC];    // scale (NF4: absmax), zero-extended by the load
    uint32_t z[NP][GPC];
  };
  // per-lane byte offsets from the first strip of the workgroup (codes), from the group's row
  // (scales, zero-points); each load adds a wave-uniform offset
  const int nbase = GLU ? min(2 * tn, p.half - 1) : min(tn * 2 * NP, p.NT - 1);  // lowest strip
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(p.packed + (size_t)nbase * KC * 64, 0xFFFFFFFFu);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(p.scales, (uint32_t)p.NG * N * 2);
  const __amdgpu_buffer_rsrc_t zrs = make_rsrc(ZEROS ? (const void*)p.qzeros : (const void*)p.scales, (uint32_t)p.NG * (N >> 3) * 4);
  uint32_t boff[NP], soff[NP], zoff[NP];
#pragma unroll
  for (int pr = 0; pr < NP; ++pr) {
    boff[pr] = (uint32_t)(strip_of(pr) - nbase) * (uint32_t)KC * 1024u + (uint32_t)c0 * 16u;
    soff[pr] = (uint32_t)col[pr] * 2u;
    zoff[pr] = (uint32_t)(col[pr] >> 3) * 4u;
  }
  constexpr int kNT = 2;  // aux bits: non-temporal (the codes are read once)
  auto load_b = [&](Codes& R, int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      R.b[pr][0] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(brs, boff[pr], kc * 1024, kNT));
      R.b[pr][1] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(brs, boff[pr] + 512, kc * 1024, kNT));
#pragma unroll
      for (int gi = 0; gi < GPC; ++gi) {
        const int g = min(kc * GPC + gi, p.NG - 1);  // groups past K are never used
        R.s[pr][gi] = __builtin_amdgcn_raw_buffer_load_b16(srs, soff[pr], g * N * 2, 0);
        if constexpr (ZEROS) R.z[pr][gi] = __builtin_amdgcn_raw_buffer_load_b32(zrs, zoff[pr], g * (N >> 3) * 4, 0);
      }
    }
  };

  // NF4: the level-pair table after every wave's slots, complete before any wave reads it
  uint32_t* const ptab = reinterpret_cast<uint32_t*>(lds + (size_t)W * RING);
  if constexpr (FMT == FMT_NF4) {
    nf4_pair_table_fill(ptab, p.codebook);
    __syncthreads();
  }

  f16v_t acc[MT][NP];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int pr = 0; pr < NP; ++pr)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][pr][i] = 0.f;

  // half hf of a block: its four 16-k steps, codes from R, activations from one slot (the
  // chunks past a ragged K are zeros, so their products vanish)
  auto compute_half = [&](const Codes& R, int hf, int slot) __attribute__((always_inline)) {
    const uint16_t* xs = ring + slot * SLOT;
    // the half's activation fragments first (one LDS wait for all four steps): step t, row
    // tile mt is row 32 mt + l%32, chunk 2t + l/32
    u4_t af[4][MT];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 32 + (lane & 31);
        const int c = 2 * t + (lane >> 5);
        af[t][mt] = *reinterpret_cast<const u4_t*>(xs + row * 64 + ((c ^ ((row >> 1) & 7)) * 8));
      }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int st = 4 * hf + t;  // step of the block: word st/2 of chunk st%2
      const int gi = GPC >= 2 ? st / (8 / GPC) : 0;
      AT bf[NP];
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        const uint32_t w = R.b[pr][st & 1][st >> 1];
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
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int pr = 0; pr < NP; ++pr)
          acc[mt][pr] = mfma32(__builtin_bit_cast(AT, af[t][mt]), bf[pr], acc[mt][pr]);
    }
  };

  // Step h (half block h of the slice) issues the copies of half h + RA - 1 and, on even h,
  // the codes of block h/2 + RB - 1, then multiplies half h (slot h % RA, code set h/2 % RB).
  // Loads past the slice re-read its last half or block (never used), and the steps run in
  // whole passes of U (those past the slice multiply nothing), so every step issues the same
  // instructions with no branch around them and the in-order load counter counts exactly:
  // after half h's copies come RA - 1 steps' copies and RA/2 code blocks. The prologue
  // interleaves its copies and code blocks so that the count holds from the first step.
  auto k_loop = [&](auto ragged) __attribute__((always_inline)) {
    Codes R[RB];
    static_assert(RB == 2 && RA == 2, "the prologue order below");
    auto pro_b = [&](int j) __attribute__((always_inline)) {
      load_b(R[j], kc0 + min(j, nb - 1));
      __builtin_amdgcn_sched_barrier(0);
    };
    auto pro_x = [&](int q) __attribute__((always_inline)) {
      load_x(min(q, nh - 1), q, ragged);
      __builtin_amdgcn_sched_barrier(0);
    };
    pro_b(0);
    pro_x(0);
    const int passes = (nh + U - 1) / U;
    for (int ps = 0; ps < passes; ++ps) {
      const int h0 = ps * U;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int h = h0 + u;
        load_x(min(h + RA - 1, nh - 1), (u + RA - 1) % RA, ragged);
        __builtin_amdgcn_sched_barrier(0);  // the count below assumes copies, then codes
        if (u % 2 == 0) load_b(R[(u / 2 + RB - 1) % RB], kc0 + min(h / 2 + RB - 1, nb - 1));
        __builtin_amdgcn_sched_barrier(0);
        skinny_wait_vmcnt<(RA - 1) * KX + (RA / 2) * KB>();
        __builtin_amdgcn_sched_barrier(0);
        if (h < nh) compute_half(R[(u / 2) % RB], u % 2, u % RA);
      }
    }
  };
  if (nh > 0) {
    if (K % 128 == 0)
      k_loop(std::false_type{});
    else
      k_loop(std::true_type{});
  }

  // ---- the W partial tiles, summed through LDS in wave order ----
  // Each wave writes its tile over its own ring, once its copies there have landed.
  // lane l holds column l%32 of pair pr and rows 32 mt + 8 (i/4) + 4 (l/32) + i%4, i < 16
  constexpr int RED = RING / 2;  // floats per wave region
  float* red = reinterpret_cast<float*>(lds);
  skinny_wait_vmcnt<0>();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int pr = 0; pr < NP; ++pr)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        red[(size_t)wave * RED + ((mt * NP + pr) * 16 + i) * 64 + lane] = acc[mt][pr][i];
  __syncthreads();
  constexpr int OUT_TILES = GLU ? MT : MT * NP;  // GLU: gate tiles (pr = 0) only
  for (int e = threadIdx.x; e < OUT_TILES * 1024; e += 64 * W) {
    const int l = e & 63, i = (e >> 6) & 15, tile = e >> 10;
    const int mt = GLU ? tile : tile / NP, pr = GLU ? 0 : tile % NP;
    const int m = m0 + mt * 32 + 8 * (i >> 2) + 4 * (l >> 5) + (i & 3);
    const int hl = (l >> 4) & 1;
    const int e0 = ((mt * NP + pr) * 16 + i) * 64 + l;
    float v = 0.f, u = 0.f;
    for (int w = 0; w < W; ++w) {
      v += red[(size_t)w * RED + e0];
      if constexpr (GLU) u += red[(size_t)w * RED + e0 + 16 * 64];
    }
    if (m >= M) continue;
    if constexpr (GLU) {
      const int gs = 2 * tn + hl;  // gate strip of this column
      if (gs < p.half)
        store_out(p.out, (size_t)m * (N >> 1) + gs * 16 + (l & 15), v / (1.0f + __expf(-v)) * u,
                  p.out_dtype);
    } else {
      const int nt = tn * 2 * NP + 2 * pr + hl;
      if (nt < p.NT) store_out(p.out, (size_t)m * N + nt * 16 + (l & 15), v, p.out_dtype);
    }
  }
}

struct SkinnyGeometry {
  int MT;
  int tiles_n, tiles_m, slice;
  size_t lds_bytes;
};

// W4A16_SKINNY_MT=1|2|4 pins the row tiles per workgroup (for benchmarking one against
// another); read once per process.
int forced_skinny_mt() {
  static const int forced = [] {
    const char* v = getenv("W4A16_SKINNY_MT");
    if (!v) return 0;
    const int mt = atoi(v);
    return mt == 1 || mt == 2 || mt == 4 ? mt : 0;
  }();
  return forced;
}

SkinnyGeometry skinny_geometry(int M, int K, int N, bool glu) {
  SkinnyGeometry g;
  const int KC = ceil_div(K, 128);
  g.tiles_n = glu ? (N / 2) / 32 + ((N / 2) % 32 ? 1 : 0) : ceil_div(N, 32 * kSkinnyPairs);
  // 64-row tiles up to 64 rows, and beyond where they fit one launch round; else 128-row tiles
  g.MT = M <= 32 ? 1 : (M <= 64 || (long)g.tiles_n * ceil_div(M, 64) <= device_cu_count()) ? 2 : 4;
  if (forced_skinny_mt()) g.MT = forced_skinny_mt();
  g.tiles_m = ceil_div(M, 32 * g.MT);
  g.slice = ceil_div(KC, skinny_waves(g.MT));
  g.lds_bytes = skinny_lds_bytes(g.MT);
  return g;
}

template <int ACT, int GPC, int FMT, int MT, bool GLU>
hipError_t launch_cfg(const SkinnyParams& p, const SkinnyGeometry& g, hipStream_t s) {
  hipLaunchKernelGGL((skinny_kernel<ACT, GPC, FMT, MT, GLU>), dim3(g.tiles_n, g.tiles_m),
                     dim3(64 * skinny_waves(MT)), g.lds_bytes, s, p);
  return hipGetLastError();
}

template <int ACT, int GPC, int FMT>
hipError_t launch_mt(const GemmArgs& a, const SkinnyParams& p, const SkinnyGeometry& g) {
  if (g.MT == 1)
    return a.glu ? launch_cfg<ACT, GPC, FMT, 1, true>(p, g, a.stream) : launch_cfg<ACT, GPC, FMT, 1, false>(p, g, a.stream);
  if (g.MT == 2)
    return a.glu ? launch_cfg<ACT, GPC, FMT, 2, true>(p, g, a.stream) : launch_cfg<ACT, GPC, FMT, 2, false>(p, g, a.stream);
  return a.glu ? launch_cfg<ACT, GPC, FMT, 4, true>(p, g, a.stream) : launch_cfg<ACT, GPC, FMT, 4, false>(p, g, a.stream);
}

template <int ACT, int GPC>
hipError_t launch_fmt(const GemmArgs& a, const SkinnyParams& p, const SkinnyGeometry& g) {
  if (a.nf4) return launch_mt<ACT, GPC, FMT_NF4>(a, p, g);
  if (a.qzeros) return launch_mt<ACT, GPC, FMT_ASYM>(a, p, g);
  return launch_mt<ACT, GPC, FMT_SYM>(a, p, g);
}

template <int ACT>
hipError_t launch_gpc(const GemmArgs& a, const SkinnyParams& p, const SkinnyGeometry& g) {
  switch (a.group_size) {
    case 128: return launch_fmt<ACT, 1>(a, p, g);
    case 64: return launch_fmt<ACT, 2>(a, p, g);
    default: return launch_fmt<ACT, 4>(a, p, g);
  }
}

}  // namespace

const char* skinny_name(int M, int K, int N) {
  const SkinnyGeometry g = skinny_geometry(M, K, N, false);
  return g.MT == 1 ? "w4a16_skinny_32x64" : g.MT == 2 ? "w4a16_skinny_64x64" : "w4a16_skinny_128x64";
}

// AWQ-scaled activations are not scaled in this kernel: the caller passes x' from the
// pre-pass (M K 2 bytes of workspace)
size_t skinny_awq_workspace_bytes(int M, int K, int N) {
  (void)N;
  return align256((size_t)M * K * 2);
}

hipError_t launch_skinny(const GemmArgs& a) {
  const SkinnyGeometry g = skinny_geometry(a.M, a.K, a.N, a.glu);
  SkinnyParams p;
  p.x = static_cast<const uint16_t*>(a.x);
  if (a.xscale) {
    if (!a.workspace || a.workspace_bytes < (size_t)a.M * a.K * 2) return hipErrorInvalidValue;
    const hipError_t e = launch_awq_scale(a.x, a.xscale, a.M, a.K, a.act, a.workspace, a.stream);
    if (e != hipSuccess) return e;
    p.x = static_cast<const uint16_t*>(a.workspace);
  }
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
  p.slice = g.slice;
  p.half = p.NT / 2;
  return a.act == ACT_F16 ? launch_gpc<ACT_F16>(a, p, g) : launch_gpc<ACT_BF16>(a, p, g);
}

}  // namespace w4a16
