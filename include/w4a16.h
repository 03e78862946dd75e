/*
 * w4a16.h - C ABI of the W4A16 fused dequantize-GEMM library for MI355X (gfx950).
 *
 * Operation ("4.3 Weight-only INT4", section 1, W4A16 storage and compute; section 4,
 * Marlin): y[M,N] = x[M,K] * W_hat[K,N], where W_hat is rebuilt on-chip from 4-bit codes
 * and per-group metadata, multiplied with 16-bit activations, accumulated in fp32.
 * K is the reduction axis (input features), N the output features.
 *
 *   affine:  W_hat[k,n] = RN_t((q[k,n] - z[k/g,n]) * s[k/g,n])     (one rounding)
 *   NF4:     W_hat[k,n] = RN_t(c[q[k,n]] * a[k/64,n])
 *
 * with t the activation type (fp16 or bf16), RN round-to-nearest-even, q the 4-bit code,
 * s the group scale, z the 4-bit zero-point (8 when qzeros is NULL: symmetric codes
 * -8..7 stored offset-binary), c a 16-entry fp16 codebook and a an fp16 absmax.
 *
 * Canonical input formats ("INT4 and Low-Bit Inference", section 6-9, packed layout):
 *   qweight  int32 [K/8][N]     eight codes along K per word, code j in bits 4j..4j+3
 *   scales   t     [K/g][N]     one scale per group of g consecutive k, per column
 *   qzeros   int32 [K/g][N/8]   eight zero-points along N per word, same nibble order
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library never
 *     allocates, frees or synchronizes; all work is enqueued on `stream` (a hipStream_t;
 *     NULL = the null stream) and is complete only when the caller synchronizes it.
 *   - Arrays are dense and row-major. x, out and the packed weight need 16-byte aligned
 *     base addresses; scales 2-byte; qzeros 4-byte.
 *   - Arguments are checked on the host before anything is enqueued. A bad argument
 *     returns W4A16_ERR_ARG, a shape the kernels do not implement W4A16_ERR_UNSUPPORTED;
 *     nothing is launched in either case. A failed launch returns W4A16_ERR_HIP.
 *     Faults during execution surface at the caller's next synchronization.
 *   - There is no slow or CPU fallback path.
 *   - The only global state is a per-device cache of the compute-unit count. Calls on
 *     different streams may run concurrently if they use distinct workspaces.
 *
 * Supported shapes: K % 32 == 0, K % group_size == 0, N % 16 == 0, M >= 0, K, N > 0,
 * group_size in {32, 64, 128}; K * N < 2^34 (packed weight below 8 GiB).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { W4A16_F16 = 0, W4A16_BF16 = 1, W4A16_F32 = 2 } w4a16_dtype;

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_ARG = 1,          /* null pointer, misalignment, inconsistent shape or dtype */
  W4A16_ERR_UNSUPPORTED = 2,  /* well-formed but not implemented (e.g. N % 16 != 0)    */
  W4A16_ERR_HIP = 3,          /* the HIP runtime rejected a launch                       */
  W4A16_ERR_WORKSPACE = 4     /* workspace missing, misaligned or smaller than required  */
} w4a16_status;

/* Bytes of the device-layout weight for a K x N matrix: K_pad * N / 2 with
 * K_pad = K rounded up to a multiple of 128. Returns 0 for unsupported shapes. */
size_t w4a16_packed_bytes(int K, int N);

/* Load-time re-layout of the weight codes ("INT4 and Low-Bit Inference", section 5,
 * Marlin's tricks: weights are re-ordered once at load so run-time unpacking is
 * branch-free and reads are coalesced; "4.3 Weight-only INT4", section 4).
 *   qweight   [in]  canonical int32 [K/8][N]
 *   packed    [out] w4a16_packed_bytes(K, N) bytes; an opaque order private to this
 *                   library, read only by the GEMM and dequant entry points below.
 * Must not alias qweight. */
w4a16_status w4a16_pack(const int32_t* qweight, int K, int N, int32_t* packed, void* stream);

/* Bytes of scratch device memory w4a16_gemm / w4a16_gemm_nf4 need for this shape on the
 * current device: zero for the decode kernel (M <= 16, see w4a16_gemm); for the batched kernel
 * zero unless it splits K across workgroups, then the fp32 partial tiles of the K slices
 * (summed in slice order by a second kernel on the same stream). The caller allocates it;
 * it needs no initialization and holds nothing between calls. Calls that may run
 * concurrently (different streams) need distinct workspaces. Returns 0 for bad shapes. */
size_t w4a16_workspace_bytes(int M, int K, int N, int group_size);

/* The W4A16 GEMM with affine (asymmetric) or symmetric INT4 weights.
 *   x         [in]  act [M][K], act = W4A16_F16 or W4A16_BF16
 *   packed    [in]  output of w4a16_pack for this K, N
 *   scales    [in]  act [K/group_size][N]
 *   qzeros    [in]  int32 [K/group_size][N/8], or NULL for symmetric codes (zero 8)
 *   out       [out] out_dtype [M][N], out_dtype = act or W4A16_F32
 *   workspace [in/out] >= w4a16_workspace_bytes(M, K, N, group_size) bytes, 256-byte
 *                   aligned (may be NULL when that size is 0)
 * M = 0 is a no-op. Results are deterministic: partial sums are combined in a fixed
 * order, never with floating-point atomics. Three kernels share the work, chosen by shape
 * (w4a16_kernel_name names the one a shape gets): the memory-bound decode kernel for up to 16
 * rows (and up to 32 on weights with K * N < 2^24, one launch per 16 rows); the skinny kernel
 * (K split across the waves of one workgroup) for about 4..256 rows on weights at most 8192
 * deep whose 64-column workgroups fill the chip in one to four launch rounds; the batched MFMA
 * kernel for the other shapes past 16 rows, and for 12..16 rows on weights with K * N >= 2^27
 * deeper than 8192 whose activations do not fit the decode kernel's LDS staging. */
w4a16_status w4a16_gemm(const void* x, int M, int K, int N, w4a16_dtype act,
                        const int32_t* packed, const void* scales, const int32_t* qzeros,
                        int group_size, void* out, w4a16_dtype out_dtype, void* workspace,
                        size_t workspace_bytes, void* stream);

/* The W4A16 GEMM with NF4 weights ("INT4 and Low-Bit Inference", section 5, The formats;
 * "INT4", section INT4, FP4, and NF4 are not identical).
 *   absmax    [in]  fp16 [K/block_size][N] per-block absmax scales
 *   codebook  [in]  16 fp16 values (device memory), code i -> codebook[i]
 *   block_size      32, 64 or 128
 * Other arguments as for w4a16_gemm. */
w4a16_status w4a16_gemm_nf4(const void* x, int M, int K, int N, w4a16_dtype act,
                            const int32_t* packed, const uint16_t* absmax,
                            const uint16_t* codebook, int block_size, void* out,
                            w4a16_dtype out_dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/* The fused gate+up projection of a gated MLP with its SwiGLU epilogue: the kernels form
 * g = x W_gate and u = x W_up in fp32 and store only h = SiLU(g) * u = g / (1 + exp(-g)) * u
 * (the pages' next step after the linear layer, "4.3 Weight-only INT4", closing section:
 * operator fusion; the MLP is the Llama one whose shapes the pages' decode examples use).
 *   packed, scales, qzeros  the (K, N2) weight holding W_gate in columns [0, N2/2) and W_up
 *                   in [N2/2, N2), packed and laid out exactly as for w4a16_gemm
 *   out       [out] out_dtype [M][N2/2]
 *   workspace       >= w4a16_workspace_bytes(M, K, N2, group_size) bytes (as for w4a16_gemm)
 * N2 must be a multiple of 32 (W4A16_ERR_UNSUPPORTED otherwise). Other arguments, errors and
 * determinism as for w4a16_gemm; one launch per call for M <= 16 (two with a K split). */
w4a16_status w4a16_gemm_swiglu(const void* x, int M, int K, int N2, w4a16_dtype act,
                               const int32_t* packed, const void* scales, const int32_t* qzeros,
                               int group_size, void* out, w4a16_dtype out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Maximum scratch of w4a16_gemm_static, in bytes (a static device array on each GPU). */
#define W4A16_STATIC_SCRATCH_BYTES (64u << 20)

/* w4a16_gemm for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels and results as
 * w4a16_gemm, bit for bit, with the split-K scratch taken from a file-scope device array of
 * W4A16_STATIC_SCRATCH_BYTES per GPU instead of a workspace argument. The array is held by
 * each GPU the library runs on until the process ends; the first call on a device looks up
 * its address (hipGetSymbolAddress). The call allocates and frees nothing.
 *   Arguments, checks and errors as for w4a16_gemm, plus W4A16_ERR_WORKSPACE when the shape
 *   needs more scratch than W4A16_STATIC_SCRATCH_BYTES (w4a16_workspace_bytes gives the
 *   need), and W4A16_ERR_HIP when the array's address cannot be obtained.
 * Every call on one GPU shares that GPU's array and the array keeps the last call's partial
 * sums; nothing in it needs to start at zero (each call writes every partial it reads). Calls
 * whose executions overlap on one GPU (different streams, or concurrent host threads) race
 * on it and give wrong results: serialize them, or use w4a16_gemm with one workspace each. */
w4a16_status w4a16_gemm_static(const void* x, int M, int K, int N, w4a16_dtype act,
                               const int32_t* packed, const void* scales, const int32_t* qzeros,
                               int group_size, void* out, w4a16_dtype out_dtype, void* stream);

/* Bytes of scratch device memory w4a16_gemm_awq needs for this shape on the current device:
 * as w4a16_workspace_bytes, plus room for the scaled activations where they are formed by a
 * pre-pass: M * K * 2 bytes (256-byte multiples) for decode shapes (M <= 16) whose
 * activations do not fit the kernel's LDS staging, and for batched shapes on the 128 x 512
 * tile. Returns 0 for bad shapes. */
size_t w4a16_awq_workspace_bytes(int M, int K, int N, int group_size);

/* The W4A16 GEMM of AWQ-scaled activations ("4.3 Weight-only INT4", section 3.2: the weight
 * is deployed as the regular INT4 format of S W, and the product is Y_hat = (X S^-1) D(Q(S W))
 * with S = diag(s) one factor per input channel):
 *   y = x' @ W_hat,  x'[m][k] = RN_act(x[m][k] * s_inv[k])
 * one round-to-nearest-even of the exact product of two act values, formed as x is staged
 * for the MFMAs (decode shapes whose x does not fit in LDS, and batched shapes on the
 * 128 x 512 tile: by a first small kernel into the workspace).
 *   s_inv     [in]  act [K], the per-input-channel S^-1, 16-byte aligned
 *   workspace [in/out] >= w4a16_awq_workspace_bytes(M, K, N, group_size) bytes, 256-byte
 *                   aligned (may be NULL when that size is 0)
 * Other arguments, errors and determinism as for w4a16_gemm (s_inv NULL with M > 0, or
 * misaligned: W4A16_ERR_ARG). */
w4a16_status w4a16_gemm_awq(const void* x, const void* s_inv, int M, int K, int N,
                            w4a16_dtype act, const int32_t* packed, const void* scales,
                            const int32_t* qzeros, int group_size, void* out,
                            w4a16_dtype out_dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Bytes of scratch device memory w4a16_gemm_w4a8 needs on the current device: the INT8
 * activations (M * K), their scales and code sums (M * 4 each), and, when the shape's output
 * tiles leave compute units idle and K is split into S slices, the slices' int32 sums
 * (S * M * N * 4); each part 256-byte aligned. 0 for M = 0 or bad shapes. */
size_t w4a16_w4a8_workspace_bytes(int M, int K, int N);

/* Name of the W4A8 GEMM configuration a shape gets ("w4a8_64x256", "w4a8_128x512", with
 * "_splitk" when K is split); "none" for bad shapes. */
const char* w4a16_w4a8_kernel_name(int M, int K, int N);

/* W4A8: INT4 weights with per-token INT8 activations on the integer MFMA ("INT4 LLMs: What
 * 4-Bit Quantization Means…", weight-only section: [-8, 7] weights unpacked to INT8, an
 * INT8 x INT8 product, the result dequantized with the input and per-channel scales; "INT8 vs
 * INT4 Quantization, in depth", section "Two regimes": past the crossover only the math rate
 * counts).
 *   y[m][n] = sx[m] * sw[n] * sum_k xq[m][k] * (u[k][n] - 8)
 *   sx[m] = RN_f32(max_k |x[m][k]| / 127),  xq = clip(rint(RN_f32(x / sx)), -127, 127)
 * The integer sum is exact; the epilogue multiplies it by the two scales in fp32. With K split,
 * the slices' int32 sums are added exactly by a second kernel before the same epilogue, so the
 * result does not depend on the split.
 *   x         [in]  act [M][K], finite (quantized per row by a first kernel into the workspace)
 *   packed    [in]  output of w4a16_pack of symmetric codes (u = q + 8, as for w4a16_gemm with
 *                   qzeros = NULL)
 *   wscale    [in]  act [N], one scale per output channel
 *   out       [out] out_dtype [M][N], out_dtype = act or W4A16_F32
 *   workspace [in/out] >= w4a16_w4a8_workspace_bytes(M, K, N), 256-byte aligned
 * K % 32 == 0 (else W4A16_ERR_UNSUPPORTED); other arguments and errors as for w4a16_gemm. */
w4a16_status w4a16_gemm_w4a8(const void* x, int M, int K, int N, w4a16_dtype act,
                             const int32_t* packed, const void* wscale, void* out,
                             w4a16_dtype out_dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Test hook: the per-token INT8 quantization w4a16_gemm_w4a8 applies, in k order.
 *   xq [out] int8 [M][K] (8-byte aligned), sx [out] float [M]. K % 8 == 0. */
w4a16_status w4a16_quantize_act_int8(const void* x, int M, int K, w4a16_dtype act, int8_t* xq,
                                     float* sx, void* stream);

/* NF4 counterpart of w4a16_gemm_swiglu (absmax [K/block_size][N2] fp16, codebook as for
 * w4a16_gemm_nf4). */
w4a16_status w4a16_gemm_nf4_swiglu(const void* x, int M, int K, int N2, w4a16_dtype act,
                                   const int32_t* packed, const uint16_t* absmax,
                                   const uint16_t* codebook, int block_size, void* out,
                                   w4a16_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Test hook: write W_hat[K][N] (row-major, in `wdtype` = F16 or BF16) using the same
 * device dequantization routine the GEMM kernels use where they form W_hat (the batched
 * kernel, and the decode kernel for bf16 activations and NF4). The fp16 affine decode
 * kernel multiplies the exact integers (q - z) and applies s to the fp32 sum of each
 * group, which skips W_hat's rounding to fp16: its result differs from the rounded-W_hat
 * product by rounding noise only, within the 1e-3 bound. scales are in wdtype. */
w4a16_status w4a16_dequant(const int32_t* packed, const void* scales, const int32_t* qzeros,
                           int K, int N, int group_size, w4a16_dtype wdtype, void* w_out,
                           void* stream);

/* Test hook: NF4 counterpart of w4a16_dequant (absmax and codebook are fp16). */
w4a16_status w4a16_dequant_nf4(const int32_t* packed, const uint16_t* absmax,
                               const uint16_t* codebook, int K, int N, int block_size,
                               w4a16_dtype wdtype, void* w_out, void* stream);

/* Name of the kernel w4a16_gemm / w4a16_gemm_nf4 launch for this shape (static string),
 * so a caller can log which path ran ("4.3 Weight-only INT4", section 4.1). */
const char* w4a16_kernel_name(int M, int K, int N, int group_size);

/* Static description of a status code. */
const char* w4a16_status_string(w4a16_status status);

/* Measurement hook, not part of the GEMM path: the device's practical HBM read ceiling, for
 * reporting beside the published peak. Reads every 16-byte chunk of buf[0, bytes) once, each
 * wave streaming a contiguous run with the 16-byte non-temporal loads the GEMM kernels use for
 * the packed codes, and XORs folds of the words into the sink words (so no load is dead code):
 * afterwards the XOR of the 256 sink words has changed by the XOR of all words of buf.
 *   buf   [in]     device buffer, 16-byte aligned; bytes a multiple of 16 (0: no-op)
 *   sink  [in/out] 256 device uint32 words, 4-byte aligned
 * Bad arguments return W4A16_ERR_ARG before anything is launched. */
w4a16_status w4a16_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Library version string. */
const char* w4a16_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
