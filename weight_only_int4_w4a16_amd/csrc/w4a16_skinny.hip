// w4a16_skinny.hip - W4A16 GEMM for mid-size batches (17 to 64 rows): the weight bytes still
// bound the time, but each weight now feeds enough rows that the MFMAs and the activation
// reads matter too.
//
// "INT8 vs INT4 Quantization, in depth", section "Two regimes": below the crossover batch a
// layer waits on its weight bytes, so the codes must stream at full rate while every row of x
// is multiplied on-chip; "4.3 Weight-only INT4", section 4 (Marlin): the speedup holds near
// its ceiling at batch 16-32 only if the kernel keeps enough loads in flight.
//
// Work split. A workgroup owns NP pairs of 16-column strips (32 NP columns) and up to 32 MT
// rows over the whole K range; its W waves take W contiguous k-block slices of K, each wave
// streaming the codes of all NP pairs and the activation fragments of all MT row tiles for its
// slice. No wave waits for another until the end, where the W partial tiles are summed through
// LDS in wave order (deterministic, no global partials, no second launch). A column tile is
// thus read by one workgroup with W independent load streams, which keeps about W x 20 KB in
// flight per compute unit.
//
// Operands. v_mfma_f32_32x32x16_{f16,bf16}: lane l multiplies row l%32 of a row tile with
// column l%32 of a strip pair, k = 16t + 8(l/32) .. +8 at step t of a 128-k block. The codes of
// those k are word t/2 of the packed chunk lane 16((2t + l/32) % 4) + l%16 owns (two 16-byte
// chunks per lane per pair and block, as in the batched kernel). The activation fragment is
// 16 contiguous bytes of one row of x, loaded straight from global memory (L2): a wave's
// slice of x is its own, so staging it in LDS would save nothing. Each word is dequantized
// once per workgroup and used for MT row tiles.
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

// GLU: NP = 2, pair 0 holds two gate strips and pair 1 the matching up strips; the output is
// h = SiLU(gate) * up, [M][N/2].
template <int ACT, int GPC, int FMT, int MT, int NP, int W, bool GLU>
__global__ __launch_bounds__(64 * W) void skinny_kernel(SkinnyParams p) {
  typedef typename ActT<ACT>::type AT;
  static_assert(!GLU || NP == 2, "a SwiGLU tile is one gate pair and one up pair");
  constexpr bool ZEROS = FMT == FMT_ASYM;
  constexpr int TILE = MT * NP * 1024;  // fp32 partial sums per wave
  extern __shared__ __attribute__((aligned(16))) float red[];  // [W][MT][NP][16][64]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = p.K, N = p.N, M = p.M, KC = p.KC;
  const int tn = blockIdx.x;
  const int m0 = blockIdx.y * 32 * MT;
  const int kc0 = min(wave * p.slice, KC);
  const int kc1 = min(kc0 + p.slice, KC);
  const int nb = kc1 - kc0;
  const int h16 = (lane >> 4) & 1;  // which strip of a pair this lane's column is in
  // strip of pair pr for this lane, clamped in bounds for loads (never stored past N)
  auto strip_of = [&](int pr) __attribute__((always_inline)) {
    return GLU ? min(2 * tn + h16, p.half - 1) + pr * p.half : min(tn * 2 * NP + 2 * pr + h16, p.NT - 1);
  };
  const int shift = 4 * (lane & 7);
  const int c0 = 16 * (lane >> 5) + (lane & 15);  // first packed chunk of this lane

  // A pipeline stage is half a k-block (64 k, four MFMA steps): the A fragments of its steps,
  // words 2 hf and 2 hf + 1 of the lane's two packed chunks (8 bytes each), and the scale
  // groups it spans
  constexpr int GPH = GPC >= 2 ? GPC / 2 : 1;  // scale groups per half block
  typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
  struct Regs {
    u4_t a[MT][4];          // activation fragments, row tile mt, step t of the half
    u2_t b[NP][2];          // words (2 hf, 2 hf + 1) of chunks c0 and c0 + 32
    uint32_t s[NP][GPH];    // 16-bit scale (NF4: absmax), zero-extended by the load
    uint32_t z[NP][GPH];
  };
  int col[NP];
#pragma unroll
  for (int pr = 0; pr < NP; ++pr) col[pr] = strip_of(pr) * 16 + (lane & 15);
  int xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xrow[mt] = min(m0 + mt * 32 + (lane & 31), M - 1);

  // stage s of this wave: k-block kc0 + s / 2, half s % 2
  auto load = [&](Regs& R, int st) __attribute__((always_inline)) {
    const int kc = kc0 + (st >> 1), hf = st & 1;
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      const u2_t* blk = reinterpret_cast<const u2_t*>(p.packed + ((size_t)(col[pr] >> 4) * KC + kc) * 64);
      R.b[pr][0] = blk[2 * c0 + hf];
      R.b[pr][1] = blk[2 * (c0 + 32) + hf];
#pragma unroll
      for (int gl = 0; gl < GPH; ++gl) {
        const int gi = GPC >= 2 ? hf * GPH + gl : 0;
        const int g = min(kc * GPC + gi, p.NG - 1);  // groups past K are never used
        R.s[pr][gl] = p.scales[(size_t)g * N + col[pr]];
        if constexpr (ZEROS) R.z[pr][gl] = p.qzeros[(size_t)g * (N >> 3) + (col[pr] >> 3)];
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint16_t* xr = p.x + (size_t)xrow[mt] * K + (lane >> 5) * 8;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // a ragged K ends inside the last block: read an in-bounds chunk, zeroed in compute
        const int k = min(kc * 128 + 64 * hf + 16 * t, K - 16);
        R.a[mt][t] = *reinterpret_cast<const u4_t*>(xr + k);
      }
    }
  };

  Nf4Lut lut;
  if constexpr (FMT == FMT_NF4) lut = load_nf4_lut(p.codebook);

  f16v_t acc[MT][NP];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int pr = 0; pr < NP; ++pr)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][pr][i] = 0.f;

  auto compute = [&](const Regs& R, int st) __attribute__((always_inline)) {
    const int kc = kc0 + (st >> 1), hf = st & 1;
    const int kvalid = K - kc * 128 - 64 * hf;  // k of this half below K (a multiple of 32)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // step 4 hf + t: word (4 hf + t) / 2 of chunk c0 (even steps) or c0 + 32 (odd)
      const int gl = GPC >= 2 ? t / (8 / GPC) : 0;
      AT bf[NP];
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        const uint32_t w = R.b[pr][t & 1][t >> 1];
        const uint32_t sraw = R.s[pr][gl];
        if constexpr (FMT == FMT_NF4) {
          if constexpr (ACT == ACT_F16)
            bf[pr] = dequant_word_nf4_f16(w, lut, as_h2(sraw * 0x00010001u));
          else
            bf[pr] = dequant_word_nf4_bf16(w, lut, (float)__builtin_bit_cast(_Float16, (uint16_t)sraw));
        } else {
          const uint32_t zq = ZEROS ? (R.z[pr][gl] >> shift) & 0xFu : 8u;
          if constexpr (ACT == ACT_F16)
            bf[pr] = dequant_word_f16(w, make_zero_f16(zq), as_h2(sraw * 0x00010001u));
          else
            bf[pr] = dequant_word_bf16(w, make_zero_f32(zq, __builtin_bit_cast(float, sraw << 16)));
        }
      }
      const bool in_k = 16 * t < kvalid;  // the step's 16 k are all in, or all out
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u4_t a = in_k ? R.a[mt][t] : u4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int pr = 0; pr < NP; ++pr)
          acc[mt][pr] = mfma32(__builtin_bit_cast(AT, a), bf[pr], acc[mt][pr]);
      }
    }
  };

  // ST register sets of half blocks: stages s+1 .. s+ST-1 load while stage s is multiplied
  // (measured: four sets at 32 rows cost 5-20% against two, from the lower occupancy). Loads
  // are unconditional (past the slice they re-read its last half, never
  // used), so the in-order load counter only ever waits for the set about to be used; a
  // scheduling barrier after each batch of loads keeps the compiler from sinking them below the
  // MFMAs.
  constexpr int ST = 2;
  const int ns = 2 * nb;  // stages of this wave (even)
  if (ns > 0) {
    Regs R[ST];
#pragma unroll
    for (int u = 0; u + 1 < ST; ++u) load(R[u], min(u, ns - 1));
    int st = 0;
    for (; st + ST - 1 < ns; st += ST) {
#pragma unroll
      for (int u = 0; u < ST; ++u) {
        load(R[(u + ST - 1) % ST], min(st + u + ST - 1, ns - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(R[u], st + u);
      }
    }
#pragma unroll
    for (int u = 0; u + 1 < ST; ++u) {
      if (st + u < ns) {
        load(R[(u + ST - 1) % ST], min(st + u + ST - 1, ns - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(R[u], st + u);
      }
    }
  }

  // ---- the W partial tiles, summed through LDS in wave order ----
  // lane l holds column l%32 of pair pr and rows 32 mt + 8 (i/4) + 4 (l/32) + i%4, i < 16
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int pr = 0; pr < NP; ++pr)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        red[(size_t)wave * TILE + ((mt * NP + pr) * 16 + i) * 64 + lane] = acc[mt][pr][i];
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
      v += red[(size_t)w * TILE + e0];
      if constexpr (GLU) u += red[(size_t)w * TILE + e0 + 16 * 64];
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
  int MT, NP, W;
  int tiles_n, tiles_m, slice;
  size_t lds_bytes;
};

SkinnyGeometry skinny_geometry(int M, int K, int N, bool glu) {
  SkinnyGeometry g;
  g.MT = M <= 32 ? 1 : 2;
  g.NP = 2;
  g.W = 8;
  const int KC = ceil_div(K, 128);
  g.tiles_n = glu ? (N / 2) / 32 + ((N / 2) % 32 ? 1 : 0) : ceil_div(N, 32 * g.NP);
  g.tiles_m = ceil_div(M, 32 * g.MT);
  g.slice = ceil_div(KC, g.W);
  g.lds_bytes = (size_t)g.W * g.MT * g.NP * 1024 * 4;
  return g;
}

template <int ACT, int GPC, int FMT, int MT, bool GLU>
hipError_t launch_cfg(const SkinnyParams& p, const SkinnyGeometry& g, hipStream_t s) {
  constexpr int NP = 2, W = 8;
  hipLaunchKernelGGL((skinny_kernel<ACT, GPC, FMT, MT, NP, W, GLU>), dim3(g.tiles_n, g.tiles_m),
                     dim3(64 * W), g.lds_bytes, s, p);
  return hipGetLastError();
}

template <int ACT, int GPC, int FMT>
hipError_t launch_mt(const GemmArgs& a, const SkinnyParams& p, const SkinnyGeometry& g) {
  if (g.MT == 1)
    return a.glu ? launch_cfg<ACT, GPC, FMT, 1, true>(p, g, a.stream) : launch_cfg<ACT, GPC, FMT, 1, false>(p, g, a.stream);
  return a.glu ? launch_cfg<ACT, GPC, FMT, 2, true>(p, g, a.stream) : launch_cfg<ACT, GPC, FMT, 2, false>(p, g, a.stream);
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
  return g.MT == 1 ? "w4a16_skinny_32x64" : "w4a16_skinny_64x64";
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
