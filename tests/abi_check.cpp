// Host-side check of the C ABI's argument validation, built with the host address and
// undefined-behaviour sanitizers (tests/test_abi_sanitized.py). Every call below must be
// rejected, or be a documented no-op, before anything is enqueued: the pointers are
// placeholders that are never dereferenced, and no GPU is needed. Exit status 0 means every
// expectation held; each failure prints its line.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "w4a16.h"

// tests/abi_check_c.c: w4a16_status_string called from C with an int
extern "C" const char* abi_check_status_string_of_int(int v);

static int failures = 0;

#define EXPECT(cond)                                          \
  do {                                                        \
    if (!(cond)) {                                            \
      fprintf(stderr, "abi_check:%d: %s\n", __LINE__, #cond); \
      ++failures;                                             \
    }                                                         \
  } while (0)

int main() {
  // placeholders: 256-byte aligned addresses (never dereferenced), and one misaligned
  void* const P = reinterpret_cast<void*>(uintptr_t{1} << 20);
  void* const Q = reinterpret_cast<void*>((uintptr_t{1} << 20) + 4096);
  void* const ODD = reinterpret_cast<void*>((uintptr_t{1} << 20) + 1);
  const int32_t* const PK = static_cast<const int32_t*>(P);
  const uint16_t* const CB = static_cast<const uint16_t*>(Q);
  const w4a16_dtype F16 = W4A16_F16, BF16 = W4A16_BF16, F32 = W4A16_F32;

  // sizes: K rounded up to whole 128-k blocks, half a byte per weight
  EXPECT(w4a16_packed_bytes(4096, 4096) == 4096u * 4096u / 2);
  EXPECT(w4a16_packed_bytes(4160, 48) == 4224u * 48u / 2);
  EXPECT(w4a16_packed_bytes(4096, 24) == 0);  // N % 16: unsupported

  // pack
  EXPECT(w4a16_pack(nullptr, 128, 64, static_cast<int32_t*>(Q), nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_pack(PK, 128, 64, nullptr, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_pack(PK, 100, 64, static_cast<int32_t*>(Q), nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_pack(PK, 128, 24, static_cast<int32_t*>(Q), nullptr) == W4A16_ERR_UNSUPPORTED);
  EXPECT(w4a16_pack(PK, 128, 64, static_cast<int32_t*>(P), nullptr) == W4A16_ERR_ARG);  // in place
  EXPECT(w4a16_pack(PK, 128, 64, static_cast<int32_t*>(ODD), nullptr) == W4A16_ERR_ARG);

  // gemm: shapes, dtypes, pointers, alignment, workspace
  EXPECT(w4a16_gemm(P, -1, 256, 64, F16, PK, Q, nullptr, 128, P, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(P, 1, 256, 64, F16, PK, Q, nullptr, 48, P, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(P, 1, 288, 64, F16, PK, Q, nullptr, 128, P, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(P, 1, 256, 24, F16, PK, Q, nullptr, 128, P, F16, nullptr, 0, nullptr) == W4A16_ERR_UNSUPPORTED);
  EXPECT(w4a16_gemm(P, 1, 256, 64, F32, PK, Q, nullptr, 128, P, F32, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(P, 1, 256, 64, F16, PK, Q, nullptr, 128, P, BF16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(nullptr, 1, 256, 64, F16, PK, Q, nullptr, 128, P, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(P, 1, 256, 64, F16, nullptr, Q, nullptr, 128, P, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(P, 1, 256, 64, F16, PK, nullptr, nullptr, 128, P, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(P, 1, 256, 64, F16, PK, Q, nullptr, 128, nullptr, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(ODD, 1, 256, 64, F16, PK, Q, nullptr, 128, P, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(P, 1, 256, 64, F16, PK, Q, static_cast<const int32_t*>(ODD), 128, P, F16, nullptr, 0,
                    nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm(nullptr, 0, 256, 64, F16, nullptr, nullptr, nullptr, 128, nullptr, F16, nullptr, 0,
                    nullptr) == W4A16_OK);  // M = 0: nothing to do
  // a shape whose batched launch splits K needs scratch: none given, or too little
  const size_t need = w4a16_workspace_bytes(200, 2048, 64, 128);
  EXPECT(need > 0);
  EXPECT(w4a16_gemm(P, 200, 2048, 64, F16, PK, Q, nullptr, 128, P, F16, nullptr, 0, nullptr) == W4A16_ERR_WORKSPACE);
  EXPECT(w4a16_gemm(P, 200, 2048, 64, F16, PK, Q, nullptr, 128, P, F16, Q, need - 256, nullptr) ==
         W4A16_ERR_WORKSPACE);
  EXPECT(w4a16_gemm(P, 200, 2048, 64, F16, PK, Q, nullptr, 128, P, F16, ODD, need, nullptr) == W4A16_ERR_WORKSPACE);

  // NF4, SwiGLU, static scratch, AWQ
  EXPECT(w4a16_gemm_nf4(P, 1, 256, 64, F16, PK, CB, nullptr, 64, P, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm_nf4(P, 1, 256, 64, F16, PK, CB, CB, 48, P, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm_swiglu(P, 1, 256, 48, F16, PK, Q, nullptr, 128, P, F16, nullptr, 0, nullptr) ==
         W4A16_ERR_UNSUPPORTED);  // each half must be whole 16-column strips
  EXPECT(w4a16_gemm_nf4_swiglu(P, 1, 256, 48, F16, PK, CB, CB, 64, P, F16, nullptr, 0, nullptr) ==
         W4A16_ERR_UNSUPPORTED);
  EXPECT(w4a16_gemm_static(P, -1, 256, 64, F16, PK, Q, nullptr, 128, P, F16, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm_static(nullptr, 1, 256, 64, F16, PK, Q, nullptr, 128, P, F16, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm_awq(P, ODD, 1, 256, 64, F16, PK, Q, nullptr, 128, P, F16, nullptr, 0, nullptr) ==
         W4A16_ERR_ARG);

  // W4A8 and its quantizer
  EXPECT(w4a16_gemm_w4a8(P, 1, 240, 64, F16, PK, Q, P, F16, nullptr, 0, nullptr) == W4A16_ERR_UNSUPPORTED);
  EXPECT(w4a16_gemm_w4a8(P, -1, 256, 64, F16, PK, Q, P, F16, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm_w4a8(P, 1, 256, 64, F32, PK, Q, P, F32, nullptr, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_quantize_act_int8(P, 2, 100, F16, static_cast<int8_t*>(Q), static_cast<float*>(P), nullptr) ==
         W4A16_ERR_ARG);
  EXPECT(w4a16_quantize_act_int8(nullptr, 0, 128, F16, nullptr, nullptr, nullptr) == W4A16_OK);

  // test hooks
  EXPECT(w4a16_dequant(nullptr, Q, nullptr, 256, 64, 128, F16, P, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_dequant(PK, Q, nullptr, 256, 64, 128, F32, P, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_dequant_nf4(PK, CB, nullptr, 256, 64, 64, F16, P, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_read_probe(P, 100, static_cast<uint32_t*>(Q), nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_read_probe(nullptr, 0, nullptr, nullptr) == W4A16_OK);

  // names and strings: static, never null, whatever the input
  for (int s = 0; s < 5; ++s) EXPECT(strlen(w4a16_status_string(static_cast<w4a16_status>(s))) > 0);
  EXPECT(strcmp(abi_check_status_string_of_int(99), "unknown status") == 0);
  EXPECT(strcmp(w4a16_kernel_name(0, 4096, 4096, 128), "none") == 0);
  EXPECT(strncmp(w4a16_kernel_name(1, 4096, 4096, 128), "w4a16_decode", 12) == 0);
  EXPECT(strncmp(w4a16_kernel_name(2048, 8192, 28672, 128), "w4a16_tiled", 11) == 0);
  EXPECT(w4a16_w4a8_kernel_name(16, 4100, 4096) != nullptr);
  EXPECT(w4a16_version() != nullptr && strlen(w4a16_version()) > 0);

  if (failures) fprintf(stderr, "abi_check: %d expectation(s) failed\n", failures);
  else printf("abi_check: all expectations held\n");
  return failures ? 1 : 0;
}
