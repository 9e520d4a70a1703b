// Device building blocks for gfx950: buffer loads, the per-format decoders and
// the MFMA step shared by the GEMV, SwiGLU, MoE and dequant kernels.
//
// Decoding follows the formats of the NInfer article (section 2: groupwise
// 4/5-bit integers, NVFP4), the RustingStrata page (Q8_0-style int8) and the
// Decapybara page (NVFP4 GEMV). Each decoder turns one lane's 8 codes of one
// 32-column group into the bf16x8 B operand of v_mfma_f32_16x16x32_bf16:
//   int4 / int5  bf16(B + q) with B = 16 (int4) or 32 (int5), the smallest
//                power of two above the largest code: the code sits in the
//                top mantissa bits under the exponent of B, so the value is
//                exact; the bias B * sum(x) is removed in the group epilogue
//                (int5's decoder lives with the k-loop: it decodes a whole
//                k-step)
//   int8         bf16(q), exact (|q| <= 128)
//   nvfp4        bf16(e2m1), exact, via v_cvt_scalef32_pk_bf16_fp4 with scale 1
//                (that instruction only applies the exponent of its scale, so
//                the E4M3 block scale is applied in fp32 afterwards)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Raw buffer descriptor (gfx9 word 3: 32-bit data format, no swizzle). A load
// whose offset lies past num_records returns zeros and touches no memory,
// which is how masked-off lanes get zero operands without branches.
constexpr int kBufWord3 = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kNonTemporal = 2;   // cache-policy bit "nt" on gfx94x/gfx950

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kBufWord3);
}

__device__ __forceinline__ u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x4 ld128_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
}
__device__ __forceinline__ u32x2 ld64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// voff: per-lane offset, soff: wave-uniform offset (an SGPR). Masked lanes
// use a voff of 2^31 or more; every soff here stays below 2^31, so the sum
// cannot wrap back into range.
__device__ __forceinline__ u32x4 ld128s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ u32x4 ld128s_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNonTemporal);
}
__device__ __forceinline__ u32x2 ld64s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld32s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld32s_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNonTemporal);
}
__device__ __forceinline__ uint32_t ld16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float f16_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// (a & b) | c in one gfx950 v_bitop3_b32 (truth table 0xEA, S0 the most
// significant input); VOP3 takes no 32-bit literal here, so plain C becomes
// an AND and an OR with literals.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0xEA);
}

// ---- decoders: 8 codes of one lane and group -> bf16x8 (slot e = element e)

// Code bias of the asymmetric int formats (see the header comment): bf16
// bit pattern of B in both halves of a dword, and 1 / B.
constexpr uint32_t kBias4Bits = 0x41804180u;   // bf16(16) twice
constexpr uint32_t kBias5Bits = 0x42004200u;   // bf16(32) twice
template <int B_OF_FMT>
struct CodeBias;
template <> struct CodeBias<1> { static constexpr uint32_t bits = kBias4Bits; static constexpr float inv = 0.0625f; };
template <> struct CodeBias<2> { static constexpr uint32_t bits = kBias5Bits; static constexpr float inv = 0.03125f; };

// int4 dword: slot e in nibble (e even ? e/2 : 4 + e/2), so the nibble pairs
// (0,4), (1,5), (2,6), (3,7) are the slot pairs (0,1), (2,3), (4,5), (6,7).
// bf16(16 + q): the 4-bit code lands in mantissa bits 3..6 (one ulp of 16
// is 1/8), so each half is shifted there and OR-ed under the exponent of 16.
__device__ __forceinline__ bf16x8 dec_int4(uint32_t v) {
  u32x4 r;
  r.x = and_or(v << 3, 0x00780078u, kBias4Bits);
  r.y = and_or(v >> 1, 0x00780078u, kBias4Bits);
  r.z = and_or(v >> 5, 0x00780078u, kBias4Bits);
  r.w = and_or(v >> 9, 0x00780078u, kBias4Bits);
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t v, int sh) {
  f32x2 f;
  f.x = (float)(int8_t)(v >> sh);
  f.y = (float)(int8_t)(v >> (sh + 8));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// int8: two dwords, slots 0..3 then 4..7, one byte each (two's complement)
__device__ __forceinline__ bf16x8 dec_int8(uint32_t a, uint32_t b) {
  u32x4 r;
  r.x = i8pair_to_bf16x2(a, 0);
  r.y = i8pair_to_bf16x2(a, 16);
  r.z = i8pair_to_bf16x2(b, 0);
  r.w = i8pair_to_bf16x2(b, 16);
  return __builtin_bit_cast(bf16x8, r);
}

// nvfp4: byte i holds slots 2i (low nibble) and 2i+1 (high nibble)
__device__ __forceinline__ bf16x8 dec_nvfp4(uint32_t v) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// OCP E4M3 byte J of v -> fp32 (gfx950 converts OCP FP8)
template <int J>
__device__ __forceinline__ float e4m3_byte(uint32_t v) {
  return __builtin_amdgcn_cvt_f32_fp8((int)v, J);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 bf16x8_splat(uint32_t pair) {
  const u32x4 r = {pair, pair, pair, pair};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float bf16_to_f32(__bf16 b) { return (float)b; }

}  // namespace qg
