// w4a16_device.hpp - device-side building blocks shared by every W4A16 kernel on gfx950:
// the private packed weight layout, nibble unpacking, the one-rounding dequantization and
// thin MFMA wrappers. Every kernel that forms W_hat calls the routines below, so the
// dequant test hook and the GEMMs compute bit-identical weights. (The fp16 decode kernel
// instead multiplies the exact integers q - z, or the bare NF4 levels, and scales the fp32
// group sums; see unpack_biased_f16 and nf4_levels_f16.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a16_launch.hpp"

namespace w4a16 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));


// ---------------------------------------------------------------------------------------
// Packed device layout (written by the pack kernel, read by GEMM and dequant kernels).
//
// The weight is cut into blocks of 128 k x 16 n (KC = ceil(K/128) blocks per column
// strip, NT = N/16 strips). Block (nt, kc) is 1 KiB at word offset (nt*KC + kc)*256:
// lane l (0..63) of a wave owns 16 bytes, words 4l..4l+3; word j of lane l holds the 8
// codes of column n = 16*nt + l%16 at k = 128*kc + 32*j + 8*(l/16) + i, i = 0..7.
// That is exactly the B operand a lane feeds to v_mfma_f32_16x16x32 for k-step j of the
// block, so one 16-byte load per lane brings four MFMA steps and a wave reads 1 KiB
// contiguously. Codes past K are zero-filled.
//
// Within a word the codes are stored in nibble order [q0 q2 q4 q6 q1 q3 q5 q7] so the
// fp16 unpack below needs one shift and four and-or operations for eight codes.
// ---------------------------------------------------------------------------------------
__host__ __device__ inline uint32_t permute_nibbles(uint32_t canon) {
  // canonical code i sits in nibble i; device nibble p holds code perm[p],
  // perm = {0, 2, 4, 6, 1, 3, 5, 7}
  uint32_t out = 0;
  out |= ((canon >> 0) & 0xFu) << 0;
  out |= ((canon >> 8) & 0xFu) << 4;
  out |= ((canon >> 16) & 0xFu) << 8;
  out |= ((canon >> 24) & 0xFu) << 12;
  out |= ((canon >> 4) & 0xFu) << 16;
  out |= ((canon >> 12) & 0xFu) << 20;
  out |= ((canon >> 20) & 0xFu) << 24;
  out |= ((canon >> 28) & 0xFu) << 28;
  return out;
}

__host__ __device__ inline size_t block_word_offset(int nt, int kc, int KC) {
  return ((size_t)nt * KC + kc) * 256;
}

// ---------------------------------------------------------------------------------------
// fp16 dequantization of one packed word: W_hat = RN_fp16((q - z) * s).
//
// Magic-number unpack: OR-ing a code into the mantissa of 0x6400 (1024.0) gives 1024 + q
// exactly; a code shifted up by 4 bits into 0x5400 (64.0) gives 64 + q exactly (the
// mantissa step of 64.0 is 1/16). Subtracting 1024 + z or 64 + z (exact in fp16: both are
// integers below 2048) leaves q - z exactly, and one packed multiply by s rounds once.
// ---------------------------------------------------------------------------------------
struct ZeroF16 {
  uint32_t c1024;  // half2 (1024 + z, 1024 + z)
  uint32_t c64;    // half2 (64 + z, 64 + z)
};

__device__ inline ZeroF16 make_zero_f16(uint32_t z) {
  ZeroF16 r;
  r.c1024 = (0x6400u | z) * 0x00010001u;
  r.c64 = (0x5400u | (z << 4)) * 0x00010001u;
  return r;
}

__device__ inline h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

// (a & mask) | c as one gfx950 v_bitop3_b32. The 8-bit immediate is the truth table of
// the function over (src0, src1, src2) with the conventional operand patterns 0xF0, 0xCC,
// 0xAA: (0xF0 & 0xCC) | 0xAA = 0xEA. Left to itself the compiler emits v_and + v_or.
__device__ inline uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  constexpr uint32_t A = 0xF0, B = 0xCC, C = 0xAA;
  return __builtin_amdgcn_bitop3_b32(a, mask, c, (A & B) | C);
}

__device__ inline h8_t dequant_word_f16(uint32_t w, ZeroF16 zc, h2_t s2) {
  const uint32_t w8 = w >> 8;
  const uint32_t v0 = and_or(w, 0x000F000Fu, 0x64006400u);   // (q0, q1) + 1024
  const uint32_t v1 = and_or(w, 0x00F000F0u, 0x54005400u);   // (q2, q3) + 64
  const uint32_t v2 = and_or(w8, 0x000F000Fu, 0x64006400u);  // (q4, q5) + 1024
  const uint32_t v3 = and_or(w8, 0x00F000F0u, 0x54005400u);  // (q6, q7) + 64
  const h2_t d0 = (as_h2(v0) - as_h2(zc.c1024)) * s2;
  const h2_t d1 = (as_h2(v1) - as_h2(zc.c64)) * s2;
  const h2_t d2 = (as_h2(v2) - as_h2(zc.c1024)) * s2;
  const h2_t d3 = (as_h2(v3) - as_h2(zc.c64)) * s2;
  h8_t r;
  r[0] = d0[0]; r[1] = d0[1]; r[2] = d1[0]; r[3] = d1[1];
  r[4] = d2[0]; r[5] = d2[1]; r[6] = d3[0]; r[7] = d3[1];
  return r;
}

// ---------------------------------------------------------------------------------------
// Integer-valued MFMA operands for the decode kernels (scale applied after the products).
//
// unpack_biased_*: the eight codes of a word as exact 16-bit floats biased by a constant
// (fp16: 1024 + q for the low nibble of each byte, 64 + q for the high one; bf16: 128 + q).
// neg_bias_*: the matching -(bias + z) for every k of the word. Multiplying x by both and
// summing in fp32 gives sum_k x_k (q_k - z) over a scale group; the group's scale is then
// applied to that fp32 partial sum once. All products are exact (an 11- or 8-bit
// significand times an integer below 2^11), so the only roundings are the fp32 sums.
// ---------------------------------------------------------------------------------------
__device__ inline h8_t unpack_biased_f16(uint32_t w) {
  const uint32_t w8 = w >> 8;
  u4_t r;
  r[0] = and_or(w, 0x000F000Fu, 0x64006400u);   // (q0, q1) + 1024
  r[1] = and_or(w, 0x00F000F0u, 0x54005400u);   // (q2, q3) + 64
  r[2] = and_or(w8, 0x000F000Fu, 0x64006400u);  // (q4, q5) + 1024
  r[3] = and_or(w8, 0x00F000F0u, 0x54005400u);  // (q6, q7) + 64
  return __builtin_bit_cast(h8_t, r);
}

__device__ inline h8_t neg_bias_f16(uint32_t z) {
  const uint32_t n1024 = (0xE400u | z) * 0x00010001u;         // -(1024 + z), twice
  const uint32_t n64 = (0xD400u | (z << 4)) * 0x00010001u;    // -(64 + z), twice
  return __builtin_bit_cast(h8_t, u4_t{n1024, n64, n1024, n64});
}

__device__ inline b8_t unpack_biased_bf16(uint32_t w) {
  // device nibble p holds code perm[p] = {0, 2, 4, 6, 1, 3, 5, 7}: bits 0-3 and 16-19 are
  // codes 0 and 1, bits 4-7 and 20-23 codes 2 and 3, and so on
  u4_t r;
  r[0] = and_or(w, 0x000F000Fu, 0x43004300u);          // (q0, q1) + 128
  r[1] = and_or(w >> 4, 0x000F000Fu, 0x43004300u);     // (q2, q3) + 128
  r[2] = and_or(w >> 8, 0x000F000Fu, 0x43004300u);     // (q4, q5) + 128
  r[3] = and_or(w >> 12, 0x000F000Fu, 0x43004300u);    // (q6, q7) + 128
  return __builtin_bit_cast(b8_t, r);
}

__device__ inline b8_t neg_bias_bf16(uint32_t z) {
  const uint32_t n = (0xC300u | z) * 0x00010001u;  // -(128 + z), twice
  return __builtin_bit_cast(b8_t, u4_t{n, n, n, n});
}

// ---------------------------------------------------------------------------------------
// bf16 dequantization of one packed word: W_hat = RN_bf16((q - z) * s).
//
// q - z is formed exactly in fp16 (as for the fp16 path), multiplied by s in fp32, where
// the product of a 5-bit integer and an 8-bit significand is exact, and rounded once by the
// fp32 -> bf16 conversion (nearest-even).
// ---------------------------------------------------------------------------------------
struct ZeroF32 {
  float s;     // the group scale
  uint32_t z;  // the 4-bit zero-point
};

__device__ inline ZeroF32 make_zero_f32(uint32_t z, float s) {
  ZeroF32 r;
  r.s = s;
  r.z = z;
  return r;
}

__device__ inline b8_t dequant_word_bf16(uint32_t w, ZeroF32 zs) {
  // q - z exactly, as fp16 pairs, by the magic-number unpack of dequant_word_f16 (codes in
  // k order); then (q - z) * s exactly in fp32 (5-bit integer times 8-bit significand) and
  // one round-to-nearest-even to bf16. fma(d, s, +0) equals d * s for every d here (a zero
  // d is +0), and takes the fp16 d directly (v_fma_mix_f32).
  const ZeroF16 zc = make_zero_f16(zs.z);
  const uint32_t w8 = w >> 8;
  const h2_t d0 = as_h2(and_or(w, 0x000F000Fu, 0x64006400u)) - as_h2(zc.c1024);   // q0, q1
  const h2_t d1 = as_h2(and_or(w, 0x00F000F0u, 0x54005400u)) - as_h2(zc.c64);     // q2, q3
  const h2_t d2 = as_h2(and_or(w8, 0x000F000Fu, 0x64006400u)) - as_h2(zc.c1024);  // q4, q5
  const h2_t d3 = as_h2(and_or(w8, 0x00F000F0u, 0x54005400u)) - as_h2(zc.c64);    // q6, q7
  const h2_t d[4] = {d0, d1, d2, d3};
  b8_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    r[2 * p] = (__bf16)__builtin_fmaf((float)d[p][0], zs.s, 0.0f);
    r[2 * p + 1] = (__bf16)__builtin_fmaf((float)d[p][1], zs.s, 0.0f);
  }
  return r;
}

// ---------------------------------------------------------------------------------------
// NF4 dequantization: W_hat = RN_t(c[q] * a), with the 16 fp16 levels c a kernel argument.
// ---------------------------------------------------------------------------------------
__device__ inline uint32_t perm_b32(uint32_t hi_word, uint32_t lo_word, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_word, lo_word, sel);
}

// NF4 level pairs keyed by one byte of a packed word (two codes): entry b holds the fp16
// levels of codes b & 15 and b >> 4 as a half2, 256 entries (1 KiB) in LDS, filled once per
// workgroup. A word then costs four LDS reads and their byte offsets instead of a 16-way
// select per code in registers (two byte tables through v_perm_b32 and a select on code bit
// 3, about 27 operations per word).
constexpr int kNf4PairEntries = 256;
__device__ inline void nf4_pair_table_fill(uint32_t* tab, const uint16_t* codebook) {
  for (int i = threadIdx.x; i < kNf4PairEntries; i += blockDim.x)
    tab[i] = (uint32_t)codebook[i & 15] | ((uint32_t)codebook[i >> 4] << 16);
}

// The eight fp16 codebook levels of one packed word from the pair table, in the word's byte
// order: byte b holds device nibbles 2b and 2b + 1, i.e. k = 0, 2, 4, 6, 1, 3, 5, 7 (the
// kernel's activations are staged in that order too).
__device__ inline h8_t nf4_levels_f16_pairs(uint32_t w, const uint32_t* tab) {
  const u4_t r{tab[w & 0xFFu], tab[(w >> 8) & 0xFFu], tab[(w >> 16) & 0xFFu], tab[w >> 24]};
  return __builtin_bit_cast(h8_t, r);
}

// The same eight levels in k order (four byte permutes on the pair-order words).
__device__ inline u4_t nf4_levels_k_order(uint32_t w, const uint32_t* tab) {
  const uint32_t p0 = tab[w & 0xFFu], p1 = tab[(w >> 8) & 0xFFu];     // (c0, c2), (c4, c6)
  const uint32_t p2 = tab[(w >> 16) & 0xFFu], p3 = tab[w >> 24];      // (c1, c3), (c5, c7)
  return u4_t{perm_b32(p2, p0, 0x05040100u), perm_b32(p2, p0, 0x07060302u),
              perm_b32(p3, p1, 0x05040100u), perm_b32(p3, p1, 0x07060302u)};
}

// W_hat = RN_t(c[q] * a) for one packed word, levels from the pair table: the level times the
// absmax is exact in fp32 (11 x 11 significant bits), so the product rounds once.
__device__ inline h8_t dequant_word_nf4_f16_tab(uint32_t w, const uint32_t* tab, h2_t a2) {
  const u4_t c = nf4_levels_k_order(w, tab);
  h8_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const h2_t d = as_h2(c[p]) * a2;
    r[2 * p] = d[0];
    r[2 * p + 1] = d[1];
  }
  return r;
}

__device__ inline b8_t dequant_word_nf4_bf16_tab(uint32_t w, const uint32_t* tab, float a) {
  const u4_t c = nf4_levels_k_order(w, tab);
  b8_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const h2_t h = as_h2(c[p]);
    // fp16 level * fp16 absmax: exact in fp32 (11 x 11 significant bits); one rounding
    r[2 * p] = (__bf16)((float)h[0] * a);
    r[2 * p + 1] = (__bf16)((float)h[1] * a);
  }
  return r;
}

// Eight 16-bit activations (k order) rearranged to k = 0, 2, 4, 6, 1, 3, 5, 7.
__device__ inline u4_t act8_to_pair_order(u4_t v) {
  return u4_t{perm_b32(v[1], v[0], 0x05040100u), perm_b32(v[3], v[2], 0x05040100u),
              perm_b32(v[1], v[0], 0x07060302u), perm_b32(v[3], v[2], 0x07060302u)};
}

// ---------------------------------------------------------------------------------------
// MFMA wrappers (gfx950): D(16x16, fp32) += A(16x32) * B(32x16).
// Lane l: A row l%16, k = 8*(l/16)+i; B column l%16, same k; D column l%16, rows
// 4*(l/16)+r, r = 0..3.
// ---------------------------------------------------------------------------------------
__device__ inline f4_t mfma16(h8_t a, h8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline f4_t mfma16(b8_t a, b8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32, fp32) += A(32x16) * B(16x32). Lane l: A row l%32, k = 8*(l/32)+i; B column l%32,
// same k; D column l%32, rows 8*(i/4) + 4*(l/32) + i%4, i = 0..15.
__device__ inline f16v_t mfma32(h8_t a, h8_t b, f16v_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ inline f16v_t mfma32(b8_t a, b8_t b, f16v_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// AWQ input scaling of eight activations ("4.3 Weight-only INT4", section 3.2: the GEMM
// multiplies X S^-1): x' = RN_t(x * s_inv) per element, both operands of type t. fp16: one
// IEEE fp16 multiply (nearest-even). bf16: the product of two 8-bit significands is exact
// in fp32, then one nearest-even conversion.
template <int ACT>
__device__ inline u4_t scale_act8(u4_t x, u4_t s) {
  u4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (ACT == ACT_F16) {
      r[i] = __builtin_bit_cast(uint32_t, as_h2(x[i]) * as_h2(s[i]));
    } else {
      const float lo = __builtin_bit_cast(float, x[i] << 16) * __builtin_bit_cast(float, s[i] << 16);
      const float hi = __builtin_bit_cast(float, x[i] & 0xFFFF0000u) *
                       __builtin_bit_cast(float, s[i] & 0xFFFF0000u);
      r[i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
    }
  }
  return r;
}

// ---------------------------------------------------------------------------------------
// Buffer loads. A buffer resource (gfx9 V#) holds a 64-bit base, no stride, num_records bytes
// and a dword-3 word with a 32-bit data format, which untyped loads require. A load of
// base + voffset + soffset whose offset lies at or past num_records returns zeros. The GEMM
// kernels keep the per-lane part of every address in one VGPR (voffset) and advance the
// per-block part in an SGPR (soffset), so their K loops spend no vector instructions on
// addresses.
// ---------------------------------------------------------------------------------------
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;  // a voffset past every num_records used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// 16 bytes per lane from global memory straight into LDS (buffer_load_dwordx4 ... lds): lane l
// writes dst + 16 l (dst is the same for the whole wave)
__device__ __forceinline__ void buffer_copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                     uint16_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)voff,
                                           (int)soff, 0, 0);
}

// fp32 -> output element
__device__ inline void store_out(void* out, size_t idx, float v, int out_dtype) {
  if (out_dtype == 2) {
    static_cast<float*>(out)[idx] = v;
  } else if (out_dtype == 0) {
    static_cast<_Float16*>(out)[idx] = (_Float16)v;
  } else {
    static_cast<__bf16*>(out)[idx] = (__bf16)v;
  }
}

}  // namespace w4a16
