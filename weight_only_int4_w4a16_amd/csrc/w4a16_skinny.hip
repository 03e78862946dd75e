// w4a16_skinny.hip - memory-bound W4A16 GEMM for small M (decode): M <= 64 per launch.
//
// "INT8 vs INT4 Quantization, in depth", section "Two regimes": at small batch the step
// waits on weight bytes, so the kernel's job is to stream the packed codes once at full
// HBM rate and hide the unpack/dequant arithmetic under the loads.
//
// Work split: one workgroup per 16-column strip (N/16 workgroups), W waves per workgroup
// dividing the strip's K-blocks (128 k each) into contiguous ranges. Per K-block a lane
// issues one 16-byte load of packed codes (a wave reads 1 KiB contiguously), expands each
// of its four words into the B operand of one v_mfma_f32_16x16x32 step, and multiplies it
// by up to MT 16-row tiles of x (lanes of rows >= M repeat row M-1; never stored). The next block's codes and
// metadata are in flight while the current one is computed. Wave partials are reduced in
// LDS in a fixed order (deterministic, no atomics) and converted once on store.
#include "w4a16_device.hpp"
#include "w4a16_launch.hpp"

namespace w4a16 {

namespace {

constexpr int kMaxWaves = 16;

template <int GPC, bool ZEROS>
struct Meta {
  uint32_t s[GPC];  // raw 16-bit scale (or NF4 absmax) of this lane's column
  uint32_t z[GPC];  // packed zero word holding this lane's column (ZEROS only)
};

template <int GPC, bool ZEROS>
__device__ inline Meta<GPC, ZEROS> load_meta(const uint16_t* __restrict__ scales,
                                             const uint32_t* __restrict__ qzeros, int c, int K,
                                             int N, int col) {
  constexpr int GS = 128 / GPC;
  Meta<GPC, ZEROS> m;
#pragma unroll
  for (int gi = 0; gi < GPC; ++gi) {
    const int k = c * 128 + gi * GS;
    const int g = (k < K ? k : K - 1) / GS;  // clamp: tail groups past K are never used
    m.s[gi] = scales[(size_t)g * N + col];
    if (ZEROS) m.z[gi] = qzeros[(size_t)g * (N >> 3) + (col >> 3)];
    else m.z[gi] = 0;
  }
  return m;
}

template <int ACT>
struct ActT;
template <>
struct ActT<ACT_F16> { typedef h8_t type; };
template <>
struct ActT<ACT_BF16> { typedef b8_t type; };

template <int ACT, int MT, int GPC, bool ZEROS, bool NF4>
__global__ __launch_bounds__(1024) void skinny_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const u4_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
    const uint16_t* __restrict__ codebook, void* __restrict__ out, int out_dtype, int KC) {
  typedef typename ActT<ACT>::type AT;
  constexpr int SPG = 4 / GPC;  // 32-k steps per group

  __shared__ float red[kMaxWaves * 256];

  const int nt = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int W = blockDim.x >> 6;
  const int c0 = (int)(((long)KC * wave) / W);
  const int c1 = (int)(((long)KC * (wave + 1)) / W);
  const int col = nt * 16 + (lane & 15);
  const int kq = (lane >> 4) * 8;
  const int mrow = lane & 15;
  const int shift = 4 * (col & 7);

  Nf4Lut lut;
  if (NF4) lut = load_nf4_lut(codebook);

  f4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f4_t{0.f, 0.f, 0.f, 0.f};

  const u4_t* pk = packed + (size_t)nt * KC * 64 + lane;

  u4_t bn = u4_t{0u, 0u, 0u, 0u};
  Meta<GPC, ZEROS> mn;
  if (c0 < c1) {
    bn = __builtin_nontemporal_load(pk + (size_t)c0 * 64);
    mn = load_meta<GPC, ZEROS>(scales, qzeros, c0, K, N, col);
  }
  for (int c = c0; c < c1; ++c) {
    const u4_t b = bn;
    const Meta<GPC, ZEROS> md = mn;
    if (c + 1 < c1) {
      bn = __builtin_nontemporal_load(pk + (size_t)(c + 1) * 64);
      mn = load_meta<GPC, ZEROS>(scales, qzeros, c + 1, K, N, col);
    }
    // 32-k steps of this block inside K (uniform; only the last block of a ragged K is short)
    const int nj = (K - c * 128) >= 128 ? 4 : (K - c * 128) / 32;
    // activation fragments: row mt*16 + l%16, k = 128 c + 32 j + 8 (l/16) + i. Output row
    // m of an MFMA depends on A row m only, so lanes for rows >= M re-read row M-1 and
    // their results are never stored.
    u4_t av[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(mt * 16 + mrow, M - 1);
      const uint16_t* xr = x + (size_t)m * K + c * 128 + kq;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < nj) av[mt][j] = *reinterpret_cast<const u4_t*>(xr + j * 32);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= nj) break;
      const int gi = j / SPG;
      AT bf;
      if (NF4) {
        if constexpr (ACT == ACT_F16) {
          bf = dequant_word_nf4_f16(b[j], lut, as_h2(md.s[gi] * 0x00010001u));
        } else {
          const float a = (float)__builtin_bit_cast(_Float16, (uint16_t)md.s[gi]);
          bf = dequant_word_nf4_bf16(b[j], lut, a);
        }
      } else {
        const uint32_t z = ZEROS ? (md.z[gi] >> shift) & 0xFu : 8u;
        if constexpr (ACT == ACT_F16) {
          bf = dequant_word_f16(b[j], make_zero_f16(z), as_h2(md.s[gi] * 0x00010001u));
        } else {
          bf = dequant_word_bf16(b[j], make_zero_f32(z, __builtin_bit_cast(float, md.s[gi] << 16)));
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = mfma16(__builtin_bit_cast(AT, av[mt][j]), bf, acc[mt]);
    }
  }

  // deterministic reduction over the W waves of the strip
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt * 16 >= M) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave * 256 + (4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc[mt][r];
    __syncthreads();
    for (int t = threadIdx.x; t < 256; t += blockDim.x) {  // blockDim may be < 256
      float s = 0.f;
      for (int w = 0; w < W; ++w) s += red[w * 256 + t];
      const int m = mt * 16 + (t >> 4);
      if (m < M) store_out(out, (size_t)m * N + nt * 16 + (t & 15), s, out_dtype);
    }
    __syncthreads();
  }
}

int pick_waves(int KC) {
  int W = KC / 2;
  if (W < 1) W = 1;
  if (W > kMaxWaves) W = kMaxWaves;
  return W;
}

template <int ACT, int MT, int GPC, bool ZEROS, bool NF4>
void launch_one(const GemmArgs& a, const uint16_t* x, int M, void* out) {
  const int KC = ceil_div(a.K, 128);
  const int W = pick_waves(KC);
  hipLaunchKernelGGL((skinny_kernel<ACT, MT, GPC, ZEROS, NF4>), dim3(a.N / 16), dim3(64 * W), 0,
                     a.stream, x, M, a.K, a.N, reinterpret_cast<const u4_t*>(a.packed),
                     static_cast<const uint16_t*>(a.scales), a.qzeros, a.codebook, out,
                     a.out_dtype, KC);
}

template <int ACT, int MT, int GPC>
void dispatch_fmt(const GemmArgs& a, const uint16_t* x, int M, void* out) {
  if (a.nf4) launch_one<ACT, MT, GPC, false, true>(a, x, M, out);
  else if (a.qzeros) launch_one<ACT, MT, GPC, true, false>(a, x, M, out);
  else launch_one<ACT, MT, GPC, false, false>(a, x, M, out);
}

template <int ACT, int MT>
void dispatch_gpc(const GemmArgs& a, const uint16_t* x, int M, void* out) {
  switch (a.group_size) {
    case 128: dispatch_fmt<ACT, MT, 1>(a, x, M, out); break;
    case 64: dispatch_fmt<ACT, MT, 2>(a, x, M, out); break;
    default: dispatch_fmt<ACT, MT, 4>(a, x, M, out); break;
  }
}

template <int ACT>
void dispatch_mt(const GemmArgs& a, const uint16_t* x, int M, void* out) {
  if (M <= 16) dispatch_gpc<ACT, 1>(a, x, M, out);
  else if (M <= 32) dispatch_gpc<ACT, 2>(a, x, M, out);
  else dispatch_gpc<ACT, 4>(a, x, M, out);
}

}  // namespace

const char* skinny_name(int M) {
  if (M <= 16) return "w4a16_skinny_mfma16_mt1";
  if (M <= 32) return "w4a16_skinny_mfma16_mt2";
  return "w4a16_skinny_mfma16_mt4";
}

hipError_t launch_skinny(const GemmArgs& a) {
  const size_t osz = a.out_dtype == 2 ? 4 : 2;
  for (int r0 = 0; r0 < a.M; r0 += 64) {
    const int M = a.M - r0 < 64 ? a.M - r0 : 64;
    const uint16_t* x = static_cast<const uint16_t*>(a.x) + (size_t)r0 * a.K;
    void* out = static_cast<char*>(a.out) + (size_t)r0 * a.N * osz;
    if (a.act == ACT_F16) dispatch_mt<ACT_F16>(a, x, M, out);
    else dispatch_mt<ACT_BF16>(a, x, M, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace w4a16
