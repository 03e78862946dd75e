// w4a16_decode.hip - host side of the decode kernel (w4a16_decode_kernel.hpp): launch
// geometry and dispatch on activation type and weight format.
#include "w4a16_decode_kernel.hpp"

namespace w4a16 {

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

// Launch geometry. SW: with x in LDS and one 16-row tile, the widest tile (4 strips for
// fp16 with 128-k groups, else 2) that still leaves at least one tile per compute unit;
// otherwise 1. W: enough waves for about 16 per compute unit, capped so that every wave
// streams at least one whole group.
DecodeConfig geometry(int M, int K, int N, int group_size, int act, bool x_in_lds) {
  DecodeConfig c;
  c.KC = ceil_div(K, 128);
  c.NT = N / 16;
  c.rows = M < 64 ? M : 64;
  c.MT = ceil_div(c.rows, 16);
  c.x_in_lds = x_in_lds;
  const int cus = cu_count();
  const int wmax = c.MT == 1 ? kMaxWavesMt1 : kMaxWavesMtN;
  c.SW = 1;
  if (c.x_in_lds && c.MT == 1) {
    if (act == ACT_F16 && group_size == 128 && c.NT % 4 == 0 && c.NT / 4 >= cus) c.SW = 4;
    else if (c.NT % 2 == 0 && c.NT / 2 >= cus) c.SW = 2;
  }
  c.tiles = c.NT / c.SW;
  const int D = c.x_in_lds ? 4 / c.SW : 1;  // k-blocks per pipeline group
  int W = ceil_div(16 * cus, c.tiles);
  const int wfull = c.KC / D;  // waves that each still get a whole group
  if (W > wfull) W = wfull;
  if (W > wmax) W = wmax;
  if (W < 1) W = 1;
  c.slice = ceil_div(c.KC, W);
  c.W = ceil_div(c.KC, c.slice);  // drop waves left without blocks
  c.xstride = c.slice * 128 + 8;
  c.xslice = c.x_in_lds ? c.rows * c.xstride : 0;
  c.lds_bytes = (size_t)c.W * c.SW * c.rows * 16 * 4 + (size_t)c.W * c.xslice * 2;
  c.workspace_bytes = 0;
  return c;
}

}  // namespace

// x goes to LDS when it fits beside the reduction area; otherwise it is read per k-block
DecodeConfig decode_config(int M, int K, int N, int group_size, int act) {
  const int rows = M < 64 ? M : 64;
  const size_t xbytes = (size_t)rows * ceil_div(K, 128) * 128 * 2;
  if (xbytes <= kXldsBytes) {
    const DecodeConfig c = geometry(M, K, N, group_size, act, true);
    if (c.lds_bytes <= kMaxLds) return c;
  }
  return geometry(M, K, N, group_size, act, false);
}

const char* decode_name(int M, int K, int N, int group_size, int act) {
  static const char* names[3][3] = {
      {"w4a16_decode_mt1_sw1", "w4a16_decode_mt1_sw2", "w4a16_decode_mt1_sw4"},
      {"w4a16_decode_mt2_sw1", "w4a16_decode_mt2_sw2", "w4a16_decode_mt2_sw4"},
      {"w4a16_decode_mt4_sw1", "w4a16_decode_mt4_sw2", "w4a16_decode_mt4_sw4"}};
  const DecodeConfig c = decode_config(M, K, N, group_size, act);
  return names[c.MT == 1 ? 0 : c.MT == 2 ? 1 : 2][c.SW == 1 ? 0 : c.SW == 2 ? 1 : 2];
}

hipError_t launch_decode(const GemmArgs& a) {
  const size_t osz = a.out_dtype == 2 ? 4 : 2;
  for (int r0 = 0; r0 < a.M; r0 += 64) {
    const int rows = a.M - r0 < 64 ? a.M - r0 : 64;
    const DecodeConfig c = decode_config(rows, a.K, a.N, a.group_size, a.act);
    DecodeParams p;
    p.x = static_cast<const uint16_t*>(a.x) + (size_t)r0 * a.K;
    p.M = rows;
    p.K = a.K;
    p.N = a.N;
    p.packed = reinterpret_cast<const u4_t*>(a.packed);
    p.scales = static_cast<const uint16_t*>(a.scales);
    p.qzeros = a.qzeros;
    p.codebook = a.codebook;
    p.out = static_cast<char*>(a.out) + (size_t)r0 * a.N * osz;
    p.out_dtype = a.out_dtype;
    p.KC = c.KC;
    p.NG = a.K / a.group_size;
    p.W = c.W;
    p.slice = c.slice;
    p.tiles = c.tiles;
    p.xstride = c.xstride;
    p.xslice = c.xslice;
    p.GPC = 128 / a.group_size;
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
  }
  return hipSuccess;
}

}  // namespace w4a16
