// w4a16_api.hip - the C ABI declared in include/w4a16.h: host-side argument checks, then
// dispatch on M to the decode or batched (tiled) kernels. Nothing is launched
// unless every check passes; there is no fallback path.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "w4a16.h"
#include "w4a16_launch.hpp"

namespace {

using w4a16::GemmArgs;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_gs(int g) { return g == 32 || g == 64 || g == 128; }

// shape checks common to every entry point that reads the packed weight
w4a16_status check_shape(int K, int N, int gs) {
  if (K <= 0 || N <= 0 || !valid_gs(gs)) return W4A16_ERR_ARG;
  if (K % 8 || K % gs) return W4A16_ERR_ARG;
  if (N % 8) return W4A16_ERR_ARG;
  if (N % 16) return W4A16_ERR_UNSUPPORTED;
  if ((long long)K * N >= (1LL << 34)) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

w4a16_status from_hip(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP; }

enum Path { PATH_DECODE = 0, PATH_SKINNY = 1, PATH_TILED = 2, PATH_AUTO = 3 };

// W4A16_FORCE_KERNEL=decode|skinny|tiled pins the kernel for every shape (for benchmarking one
// path against another); read once per process. Any other value, or none, leaves the choice
// to the shape rules below.
Path forced_path() {
  static const Path forced = [] {
    const char* v = getenv("W4A16_FORCE_KERNEL");
    if (!v) return PATH_AUTO;
    if (!strcmp(v, "decode")) return PATH_DECODE;
    if (!strcmp(v, "skinny")) return PATH_SKINNY;
    if (!strcmp(v, "tiled")) return PATH_TILED;
    return PATH_AUTO;
  }();
  return forced;
}

// M <= 16 runs the decode kernel (one 16-row MFMA tile). 17..32 rows run the skinny kernel
// (K split across the eight waves of a workgroup, reduced in LDS) on weights at most 8192 deep
// with up to 1024 64-column tiles (four launch rounds); measured at M=32 against the batched
// kernel, e.g. 4096x14336 12.8 against 21.7 us, 8192x57344 69.8 against 78.3 us (wider N is
// unmeasured and stays on the batched kernel). Weights of at most 2^24 elements keep the decode kernel up to 32 rows, in
// 16-row launches (their tiles cannot fill the chip otherwise: 4096x4096 at M=32 14.5 us). The
// other shapes past 16 rows run the batched kernel (its 64x256 tiles with K split, or the
// 128x512 tiles), e.g. 14336x4096 at M=32 23.1 us against 44.6 skinny. From 12 rows on, a large
// weight (K N >= 2^27) whose x does not fit the decode kernel's LDS staging (so every decode
// workgroup re-reads x from L2 with each group) leaves the decode kernel: for the skinny kernel
// when at most 8192 deep (8192x57344 at M=12: 103.6 decode, 90.3 batched, 83.2 us skinny), for
// the batched kernel otherwise (28672x8192 at M=12: 50.1 decode, 44.8 us batched).
// Measured on MI355X (fp16 g128, 17..256 rows): the skinny kernel wins wherever its workgroups
// (64 columns by 32 or 64 rows, all of K) stream at most 8192-deep K and fit in one launch
// round, by 10-40% (4096x14336 at M=64: 17.3 against 25.5 us; 4096x4096 at M=128: 14.2
// against 23.0 us, at M=256: 16.7 against 26.3 us); at 17-32 rows also in up to four rounds
// (above). Where 64-row tiles would take more than one round at 65-128 rows and K <= 4096, its
// 128-row tiles (four waves, one per SIMD) still win (4096x14336 at M=96: 26.0 against 30.1 us,
// M=128: 27.8 against 32.0 us; at M=192 and 256 they lose, 49.4 and 53.6 against 34.1 and
// 39.6 us), also on 8192-deep K (8192x10240 at M=96/128: a tie at g128, 8-12% for g32, NF4
// and bf16). Up to 6144-deep K the 64-row rule holds without the column-tile condition (5120x5120 at
// M=96/128: 19.5/19.4 against 21.7/23.1 us; 5120x13824 at M=96: 30.5 against 34.0). Past 128
// rows the skinny kernel takes one round of 64-row tiles filling at least half the chip
// (5120x5120 at M=160/192: 21.4/20.5 against 28.2/27.1 us), and one round of 128-row tiles
// from 224 rows on 3072..6144-deep weights (4096x6144 at M=256: 25.8 against 29.3 us;
// 2048x8192 loses, 21.1 against 20.4) and from 160 rows on 4096..6144-deep ones (4096x6144
// at M=160/192: g128 -2/-4%, g32 -9/-12%, NF4 -10/-14%, bf16 -13/-17%; at 3072x8192 the
// batched kernel still wins by 7-9% for g128 and ties for g32 and NF4). At 33+ rows on 8192-deep K with fewer than 160 column
// tiles the batched kernel's split K wins (8192x8192 at M=64: 21.9 against 26.4 us), and so it
// does for deeper K, wider N and more rows.
Path choose_path(const GemmArgs& a) {
  const Path f = forced_path();
  if (f != PATH_AUTO) return f;
  const long long kn = (long long)a.K * a.N;
  const long long col_tiles = (a.N + 63) / 64;
  if (a.M > 256) return PATH_TILED;
  if (a.M > 16) {
    if (a.M <= 32 && kn < (1LL << 24)) return PATH_DECODE;
    if (a.K > 8192) return PATH_TILED;
    if (a.M <= 32) return col_tiles <= 1024 ? PATH_SKINNY : PATH_TILED;
    const long long cus = w4a16::device_cu_count();
    const long long wgs = col_tiles * ((a.M + 63) / 64);    // 64-row tiles
    const long long wgs4 = col_tiles * ((a.M + 127) / 128);  // 128-row tiles
    const bool mid_k = a.K <= 6144;
    if (a.M <= 128) {
      if (wgs <= cus && (mid_k || col_tiles >= 160)) return PATH_SKINNY;
      // 128-row tiles (K <= 8192) where 64-row tiles would take a second round
      return wgs > cus && wgs4 <= cus ? PATH_SKINNY : PATH_TILED;
    }
    // 129..256 rows: one round of 64-row tiles that fills at least half the chip, or one round
    // of 128-row tiles from 160 rows on 4096..6144-deep weights and from 224 rows on 3072-deep
    if (mid_k && wgs <= cus && 2 * wgs > cus) return PATH_SKINNY;
    const bool deep_enough = a.M >= 224 ? a.K >= 3072 : a.M >= 160 && a.K >= 4096;
    return deep_enough && mid_k && wgs4 <= cus ? PATH_SKINNY : PATH_TILED;
  }
  // 4..16 rows where one round of skinny workgroups fills more than half the chip: the skinny
  // kernel from the row count where the decode kernel's cost per row overtakes it, earlier for
  // the dearer dequantizations of groups of 32 or 64 (and NF4's 64-blocks) (4096x14336: NF4 at
  // M=4/8/16 16.0/17.3/19.3 -> 12.7/12.7/12.8 us; g32 at M=4/8/16 13.0/15.7/18.4 ->
  // 12.2/12.2/12.3; g128 at M=8/16 11.7/13.8 -> 11.6/11.8, 8192x10240 at M=8 17.4 -> 15.2).
  // Fewer column tiles (4096x4096, 8192x8192, 14336x4096) or more (4096x28672) keep the
  // decode kernel. The rule reads the group size only, so the name the logging call reports
  // for a shape is the kernel that runs.
  // With a quarter to a half of the chip's worth of column tiles, the skinny kernel wins only
  // from 16 rows, on 3072..6144-deep weights (5120x5120 at M=16: 13.0 -> 11.4 us; 3072x8192
  // 9.6 -> 8.9; 2048x8192 stays: 6.0 against 6.3).
  // Groups of 32 or 64 (NF4 64-blocks) make the decode kernel's rows dearer still: there the
  // skinny kernel also wins from 12 rows in the quarter-to-half band (5120x5120 g32 at M=12:
  // 14.3 -> 12.5 us; NF4 3072x8192 12.0 -> 10.2; at 8 rows it wins on some shapes and loses
  // up to 18% on others), and from 4 rows over one to two rounds of column tiles (8192x28672
  // g32 at M=4/8: 40.8/45.6 -> 36.7/37.4 us; NF4 45.2/45.8 -> 38.4/40.0). Measured against
  // the previous rules in one run over an 11-shape x 13-batch grid: g32 -0.5%, NF4 -0.9%,
  // bf16 -0.5% in total, g128 unchanged.
  {
    const long long cus = w4a16::device_cu_count();
    const bool dear = a.group_size <= 64;
    if (a.K <= 8192 && col_tiles <= cus) {
      if (2 * col_tiles > cus && a.M >= (dear ? 4 : 8)) return PATH_SKINNY;
      if (4 * col_tiles > cus && a.K >= 3072 && a.K <= 6144 && a.M >= (dear ? 12 : 16))
        return PATH_SKINNY;
    }
    if (dear && a.K <= 8192 && col_tiles > cus && col_tiles <= 2 * cus && a.M >= 4) return PATH_SKINNY;
  }
  if (a.M < 12 || kn < (1LL << 27)) return PATH_DECODE;
  if (w4a16::decode_config(a.M, a.K, a.N, a.group_size, a.glu).x_in_lds) return PATH_DECODE;
  return a.K <= 8192 ? PATH_SKINNY : PATH_TILED;
}

size_t workspace_need(int M, int K, int N, int gs) {
  GemmArgs a{};
  a.M = M; a.K = K; a.N = N; a.group_size = gs;
  switch (choose_path(a)) {
    case PATH_TILED: return w4a16::tiled_workspace_bytes(M, K, N);
    case PATH_SKINNY: return 0;
    default: return w4a16::decode_config(M < 16 ? M : 16, K, N, gs, false).workspace_bytes;
  }
}

// AWQ-scaled x: decode launches whose x does not fit in LDS, skinny launches, and batched
// launches on the large tile scale it into the workspace first
size_t awq_workspace_need(int M, int K, int N, int gs) {
  GemmArgs a{};
  a.M = M; a.K = K; a.N = N; a.group_size = gs;
  switch (choose_path(a)) {
    case PATH_TILED: return w4a16::tiled_awq_workspace_bytes(M, K, N);
    case PATH_SKINNY: return w4a16::skinny_awq_workspace_bytes(M, K, N);
    default: return w4a16::decode_awq_workspace_bytes(M < 16 ? M : 16, K, N, gs);
  }
}

w4a16_status gemm_common(GemmArgs& a, w4a16_dtype act, w4a16_dtype out_dtype) {
  if (a.M < 0) return W4A16_ERR_ARG;
  w4a16_status st = check_shape(a.K, a.N, a.group_size);
  if (st != W4A16_OK) return st;
  if (act != W4A16_F16 && act != W4A16_BF16) return W4A16_ERR_ARG;
  if (out_dtype != act && out_dtype != W4A16_F32) return W4A16_ERR_ARG;
  if (a.M == 0) return W4A16_OK;
  if (!a.x || !a.packed || !a.scales || !a.out) return W4A16_ERR_ARG;
  if (a.nf4 && !a.codebook) return W4A16_ERR_ARG;
  if (a.glu && a.N % 32) return W4A16_ERR_UNSUPPORTED;  // each half whole 16-column strips
  if (!aligned(a.x, 16) || !aligned(a.packed, 16) || !aligned(a.out, 16)) return W4A16_ERR_ARG;
  if (!aligned(a.scales, 2) || (a.qzeros && !aligned(a.qzeros, 4))) return W4A16_ERR_ARG;
  if (a.codebook && !aligned(a.codebook, 2)) return W4A16_ERR_ARG;
  if (a.xscale && !aligned(a.xscale, 16)) return W4A16_ERR_ARG;
  a.act = act == W4A16_F16 ? w4a16::ACT_F16 : w4a16::ACT_BF16;
  a.out_dtype = (int)out_dtype;
  const size_t need = a.xscale ? awq_workspace_need(a.M, a.K, a.N, a.group_size)
                               : workspace_need(a.M, a.K, a.N, a.group_size);
  if (need && (!a.workspace || !aligned(a.workspace, 256) || a.workspace_bytes < need))
    return W4A16_ERR_WORKSPACE;
  switch (choose_path(a)) {
    case PATH_TILED: return from_hip(w4a16::launch_tiled(a));
    case PATH_SKINNY: return from_hip(w4a16::launch_skinny(a));
    default: return from_hip(w4a16::launch_decode(a));
  }
}

// Scratch of w4a16_gemm_static: one file-scope device array per GPU (its split-K partial
// tiles), of W4A16_STATIC_SCRATCH_BYTES. On the host, `scratch` names a host-side stand-in,
// never the device memory: host code uses only the per-device address that
// hipGetSymbolAddress returns, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[W4A16_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {nullptr};

// the current device's copy of `scratch`, or nullptr if the lookup failed
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t w4a16_packed_bytes(int K, int N) {
  if (K <= 0 || N <= 0 || K % 8 || N % 16 || (long long)K * N >= (1LL << 34)) return 0;
  return (size_t)w4a16::ceil_div(K, 128) * 128 * (size_t)N / 2;
}

w4a16_status w4a16_pack(const int32_t* qweight, int K, int N, int32_t* packed, void* stream) {
  if (K <= 0 || N <= 0 || K % 8 || N % 8) return W4A16_ERR_ARG;
  if (N % 16 || (long long)K * N >= (1LL << 34)) return W4A16_ERR_UNSUPPORTED;
  if (!qweight || !packed || !aligned(qweight, 4) || !aligned(packed, 16)) return W4A16_ERR_ARG;
  if ((const void*)qweight == (const void*)packed) return W4A16_ERR_ARG;
  return from_hip(w4a16::launch_pack(reinterpret_cast<const uint32_t*>(qweight), K, N,
                                     reinterpret_cast<uint32_t*>(packed),
                                     static_cast<hipStream_t>(stream)));
}

size_t w4a16_workspace_bytes(int M, int K, int N, int group_size) {
  if (M < 0 || check_shape(K, N, group_size) != W4A16_OK) return 0;
  if (M == 0) return 0;
  return workspace_need(M, K, N, group_size);
}

w4a16_status w4a16_gemm(const void* x, int M, int K, int N, w4a16_dtype act,
                        const int32_t* packed, const void* scales, const int32_t* qzeros,
                        int group_size, void* out, w4a16_dtype out_dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  GemmArgs a{};
  a.x = x; a.M = M; a.K = K; a.N = N;
  a.packed = reinterpret_cast<const uint32_t*>(packed);
  a.scales = scales;
  a.qzeros = reinterpret_cast<const uint32_t*>(qzeros);
  a.codebook = nullptr; a.nf4 = false;
  a.group_size = group_size;
  a.out = out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.stream = static_cast<hipStream_t>(stream);
  return gemm_common(a, act, out_dtype);
}

w4a16_status w4a16_gemm_static(const void* x, int M, int K, int N, w4a16_dtype act,
                               const int32_t* packed, const void* scales, const int32_t* qzeros,
                               int group_size, void* out, w4a16_dtype out_dtype, void* stream) {
  // the same checks as w4a16_gemm first; then the scratch this shape needs against the
  // static maximum, before the device array is touched
  if (M < 0) return W4A16_ERR_ARG;
  const w4a16_status st = check_shape(K, N, group_size);
  if (st != W4A16_OK) return st;
  if (M == 0) return W4A16_OK;
  const size_t need = workspace_need(M, K, N, group_size);
  if (need > (size_t)W4A16_STATIC_SCRATCH_BYTES) return W4A16_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need) {
    ws = device_scratch();
    if (!ws) return W4A16_ERR_HIP;
  }
  GemmArgs a{};
  a.x = x; a.M = M; a.K = K; a.N = N;
  a.packed = reinterpret_cast<const uint32_t*>(packed);
  a.scales = scales;
  a.qzeros = reinterpret_cast<const uint32_t*>(qzeros);
  a.codebook = nullptr; a.nf4 = false;
  a.group_size = group_size;
  a.out = out;
  a.workspace = ws; a.workspace_bytes = need ? (size_t)W4A16_STATIC_SCRATCH_BYTES : 0;
  a.stream = static_cast<hipStream_t>(stream);
  return gemm_common(a, act, out_dtype);
}

size_t w4a16_awq_workspace_bytes(int M, int K, int N, int group_size) {
  if (M < 0 || check_shape(K, N, group_size) != W4A16_OK) return 0;
  if (M == 0) return 0;
  return awq_workspace_need(M, K, N, group_size);
}

w4a16_status w4a16_gemm_awq(const void* x, const void* s_inv, int M, int K, int N,
                            w4a16_dtype act, const int32_t* packed, const void* scales,
                            const int32_t* qzeros, int group_size, void* out,
                            w4a16_dtype out_dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (M > 0 && !s_inv) return W4A16_ERR_ARG;
  GemmArgs a{};
  a.x = x; a.M = M; a.K = K; a.N = N;
  a.xscale = s_inv;
  a.packed = reinterpret_cast<const uint32_t*>(packed);
  a.scales = scales;
  a.qzeros = reinterpret_cast<const uint32_t*>(qzeros);
  a.codebook = nullptr; a.nf4 = false;
  a.group_size = group_size;
  a.out = out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.stream = static_cast<hipStream_t>(stream);
  return gemm_common(a, act, out_dtype);
}

size_t w4a16_w4a8_workspace_bytes(int M, int K, int N) {
  if (M <= 0 || K <= 0 || N <= 0 || K % 32 || N % 16 || (long long)K * N >= (1LL << 34)) return 0;
  return w4a16::w4a8_workspace_bytes(M, K, N);
}

const char* w4a16_w4a8_kernel_name(int M, int K, int N) {
  if (M <= 0 || K <= 0 || N <= 0 || K % 32 || N % 16) return "none";
  return w4a16::w4a8_name(M, K, N);
}

w4a16_status w4a16_gemm_w4a8(const void* x, int M, int K, int N, w4a16_dtype act,
                             const int32_t* packed, const void* wscale, void* out,
                             w4a16_dtype out_dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (M < 0 || K <= 0 || N <= 0 || K % 8 || N % 8) return W4A16_ERR_ARG;
  if (K % 32 || N % 16 || (long long)K * N >= (1LL << 34)) return W4A16_ERR_UNSUPPORTED;
  if (act != W4A16_F16 && act != W4A16_BF16) return W4A16_ERR_ARG;
  if (out_dtype != act && out_dtype != W4A16_F32) return W4A16_ERR_ARG;
  if (M == 0) return W4A16_OK;
  if (!x || !packed || !wscale || !out) return W4A16_ERR_ARG;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(out, 16) || !aligned(wscale, 2))
    return W4A16_ERR_ARG;
  const size_t need = w4a16::w4a8_workspace_bytes(M, K, N);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return W4A16_ERR_WORKSPACE;
  GemmArgs a{};
  a.x = x; a.M = M; a.K = K; a.N = N;
  a.act = act == W4A16_F16 ? w4a16::ACT_F16 : w4a16::ACT_BF16;
  a.packed = reinterpret_cast<const uint32_t*>(packed);
  a.scales = wscale;
  a.out = out; a.out_dtype = (int)out_dtype;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.stream = static_cast<hipStream_t>(stream);
  return from_hip(w4a16::launch_w4a8(a));
}

w4a16_status w4a16_quantize_act_int8(const void* x, int M, int K, w4a16_dtype act, int8_t* xq,
                                     float* sx, void* stream) {
  if (M < 0 || K <= 0 || K % 8) return W4A16_ERR_ARG;
  if (act != W4A16_F16 && act != W4A16_BF16) return W4A16_ERR_ARG;
  if (M == 0) return W4A16_OK;
  if (!x || !xq || !sx || !aligned(x, 16) || !aligned(xq, 8) || !aligned(sx, 4)) return W4A16_ERR_ARG;
  return from_hip(w4a16::launch_quantize_act(x, M, K, act == W4A16_F16 ? w4a16::ACT_F16 : w4a16::ACT_BF16,
                                             false, xq, sx, nullptr, static_cast<hipStream_t>(stream)));
}

w4a16_status w4a16_gemm_swiglu(const void* x, int M, int K, int N2, w4a16_dtype act,
                               const int32_t* packed, const void* scales, const int32_t* qzeros,
                               int group_size, void* out, w4a16_dtype out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  GemmArgs a{};
  a.x = x; a.M = M; a.K = K; a.N = N2;
  a.packed = reinterpret_cast<const uint32_t*>(packed);
  a.scales = scales;
  a.qzeros = reinterpret_cast<const uint32_t*>(qzeros);
  a.codebook = nullptr; a.nf4 = false; a.glu = true;
  a.group_size = group_size;
  a.out = out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.stream = static_cast<hipStream_t>(stream);
  return gemm_common(a, act, out_dtype);
}

w4a16_status w4a16_gemm_nf4_swiglu(const void* x, int M, int K, int N2, w4a16_dtype act,
                                   const int32_t* packed, const uint16_t* absmax,
                                   const uint16_t* codebook, int block_size, void* out,
                                   w4a16_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  GemmArgs a{};
  a.x = x; a.M = M; a.K = K; a.N = N2;
  a.packed = reinterpret_cast<const uint32_t*>(packed);
  a.scales = absmax;
  a.qzeros = nullptr;
  a.codebook = codebook; a.nf4 = true; a.glu = true;
  a.group_size = block_size;
  a.out = out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.stream = static_cast<hipStream_t>(stream);
  return gemm_common(a, act, out_dtype);
}

w4a16_status w4a16_gemm_nf4(const void* x, int M, int K, int N, w4a16_dtype act,
                            const int32_t* packed, const uint16_t* absmax,
                            const uint16_t* codebook, int block_size, void* out,
                            w4a16_dtype out_dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  GemmArgs a{};
  a.x = x; a.M = M; a.K = K; a.N = N;
  a.packed = reinterpret_cast<const uint32_t*>(packed);
  a.scales = absmax;
  a.qzeros = nullptr;
  a.codebook = codebook; a.nf4 = true;
  a.group_size = block_size;
  a.out = out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.stream = static_cast<hipStream_t>(stream);
  return gemm_common(a, act, out_dtype);
}

static w4a16_status dequant_common(GemmArgs& a, w4a16_dtype wdtype) {
  w4a16_status st = check_shape(a.K, a.N, a.group_size);
  if (st != W4A16_OK) return st;
  if (wdtype != W4A16_F16 && wdtype != W4A16_BF16) return W4A16_ERR_ARG;
  if (!a.packed || !a.scales || !a.out || (a.nf4 && !a.codebook)) return W4A16_ERR_ARG;
  if (!aligned(a.packed, 16) || !aligned(a.scales, 2) || !aligned(a.out, 2)) return W4A16_ERR_ARG;
  if (a.qzeros && !aligned(a.qzeros, 4)) return W4A16_ERR_ARG;
  a.act = wdtype == W4A16_F16 ? w4a16::ACT_F16 : w4a16::ACT_BF16;
  return from_hip(w4a16::launch_dequant(a));
}

w4a16_status w4a16_dequant(const int32_t* packed, const void* scales, const int32_t* qzeros,
                           int K, int N, int group_size, w4a16_dtype wdtype, void* w_out,
                           void* stream) {
  GemmArgs a{};
  a.K = K; a.N = N; a.M = 0;
  a.packed = reinterpret_cast<const uint32_t*>(packed);
  a.scales = scales;
  a.qzeros = reinterpret_cast<const uint32_t*>(qzeros);
  a.nf4 = false;
  a.group_size = group_size;
  a.out = w_out;
  a.stream = static_cast<hipStream_t>(stream);
  return dequant_common(a, wdtype);
}

w4a16_status w4a16_dequant_nf4(const int32_t* packed, const uint16_t* absmax,
                               const uint16_t* codebook, int K, int N, int block_size,
                               w4a16_dtype wdtype, void* w_out, void* stream) {
  GemmArgs a{};
  a.K = K; a.N = N; a.M = 0;
  a.packed = reinterpret_cast<const uint32_t*>(packed);
  a.scales = absmax;
  a.qzeros = nullptr;
  a.codebook = codebook; a.nf4 = true;
  a.group_size = block_size;
  a.out = w_out;
  a.stream = static_cast<hipStream_t>(stream);
  return dequant_common(a, wdtype);
}

const char* w4a16_kernel_name(int M, int K, int N, int group_size) {
  if (M <= 0) return "none";
  GemmArgs a{};
  a.M = M; a.K = K; a.N = N; a.group_size = group_size;
  switch (choose_path(a)) {
    case PATH_TILED: return w4a16::tiled_name(M, K, N, group_size);
    case PATH_SKINNY: return w4a16::skinny_name(M, K, N);
    default: return w4a16::decode_name(M, K, N, group_size, w4a16::ACT_F16);
  }
}

const char* w4a16_status_string(w4a16_status s) {
  // a C caller may pass any int: read it as one (loading an enum outside its enumerators'
  // range is undefined in C++)
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_ARG: return "invalid argument";
    case W4A16_ERR_UNSUPPORTED: return "unsupported shape";
    case W4A16_ERR_HIP: return "HIP launch failed";
    case W4A16_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
  }
  return "unknown status";
}

w4a16_status w4a16_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return W4A16_OK;
  if (!buf || !sink || bytes % 16 || !aligned(buf, 16) || !aligned(sink, 4)) return W4A16_ERR_ARG;
  return from_hip(w4a16::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

const char* w4a16_version(void) { return "w4a16-gfx950 0.1"; }

}  // extern "C"
