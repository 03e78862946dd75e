// w4a16_api.hip - the C ABI declared in include/w4a16.h: host-side argument checks, then
// dispatch on M to the decode or batched (tiled) kernels. Nothing is launched
// unless every check passes; there is no fallback path.
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

// M above 16 goes to the batched kernel: past one 16-row MFMA tile the decode kernel's
// activation traffic per weight byte outgrows the batched kernel's dequantization cost
// (4096x14336: M=32 takes 33.7 us on the decode kernel, M=64 24.8 us on the batched one)
// The exception: from 12 rows on, a large weight (K N >= 2^27) whose x does not fit the decode
// kernel's LDS staging (so every workgroup re-reads x from L2 with each group) runs faster on
// the batched kernel (M=16: 8192x57344 118 -> 101 us, 28672x8192 58.7 -> 50.7 us; smaller
// weights such as 8192x10240 and 14336x4096 stay faster on the decode kernel).
// Small weights (K N <= 2^24) keep the decode kernel, in 16-row launches, up to 32 rows: their
// batched tiles cannot fill the chip (4096x4096: M=17 15.8 -> 11.3 us, M=32 17.7 -> 14.5 us).
bool use_tiled(const GemmArgs& a) {
  if (!w4a16::tiled_supported(a)) return false;
  if (a.M > 32) return true;
  if (a.M > 16) return (long long)a.K * a.N > (1LL << 24);
  if (a.M < 12 || (long long)a.K * a.N < (1LL << 27)) return false;
  return !w4a16::decode_config(a.M, a.K, a.N, a.group_size, a.glu).x_in_lds;
}

size_t workspace_need(int M, int K, int N, int gs) {
  GemmArgs a{};
  a.M = M; a.K = K; a.N = N; a.group_size = gs;
  if (use_tiled(a)) return w4a16::tiled_workspace_bytes(M, K, N);
  return w4a16::decode_config(M < 16 ? M : 16, K, N, gs, false).workspace_bytes;
}

// AWQ-scaled x: decode launches whose x does not fit in LDS, and batched launches on the
// large tile, scale it into the workspace first
size_t awq_workspace_need(int M, int K, int N, int gs) {
  GemmArgs a{};
  a.M = M; a.K = K; a.N = N; a.group_size = gs;
  if (use_tiled(a)) return w4a16::tiled_awq_workspace_bytes(M, K, N);
  return w4a16::decode_awq_workspace_bytes(M < 16 ? M : 16, K, N, gs);
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
  if (use_tiled(a)) return from_hip(w4a16::launch_tiled(a));
  return from_hip(w4a16::launch_decode(a));
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
  if (use_tiled(a)) return w4a16::tiled_name(M, K, N);
  return w4a16::decode_name(M, K, N, group_size, w4a16::ACT_F16);
}

const char* w4a16_status_string(w4a16_status s) {
  switch (s) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_ARG: return "invalid argument";
    case W4A16_ERR_UNSUPPORTED: return "unsupported shape";
    case W4A16_ERR_HIP: return "HIP launch failed";
    case W4A16_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
  }
  return "unknown status";
}

const char* w4a16_version(void) { return "w4a16-gfx950 0.1"; }

}  // extern "C"
