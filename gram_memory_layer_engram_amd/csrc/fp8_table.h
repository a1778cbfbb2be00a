// fp8 table rows -> bf16, the dequantization done on lookup.
//
// "vllm.models.deepseek_v4_1.common.engram", ParallelEngramEmbedding
// (docstring and __init__): the table is float8_e4m3fn [rows, head_dim] with
// one uint8 ue8m0 scale per row and 32 consecutive elements
// ([rows, head_dim / 32]), and rows are dequantized to bf16 on lookup. The
// value of element j is e4m3(code_j) * 2^(byte - 127) (E8M0: byte 255 is
// NaN), rounded to bf16 nearest-even. Both factors are exact in fp32 and so
// is their product (at most 4 significant bits, magnitudes 2^-136 .. 448 *
// 2^127, the top end overflowing to inf), so the only rounding is the final
// fp32 -> bf16 one.
#pragma once

#include "common.h"

namespace engram {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// E8M0 byte -> 2^(b - 127) as fp32 (byte 0 is the fp32 subnormal 2^-127);
// byte 255 -> NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  if (b == 255u) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(b ? (b << 23) : 0x00400000u);
}

// One word of 4 codes (element i is byte i) under the scale value s -> 2
// words of bf16 pairs (element 2i low, 2i+1 high). The e4m3 -> fp32
// conversion is gfx950's v_cvt_pk_f32_fp8 (OCP e4m3fn).
__device__ __forceinline__ void fp8_word_to_bf16(uint32_t codes, float s, uint32_t* out) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, true);
  out[0] = pack_bf16x2(lo[0] * s, lo[1] * s);
  out[1] = pack_bf16x2(hi[0] * s, hi[1] * s);
}

// One 32-element block: codes in 8 words, its scale byte -> 16 words of
// bf16 pairs.
__device__ __forceinline__ void fp8_block_to_bf16(const uint32_t* codes, uint32_t scale_byte, uint32_t* out) {
  const float s = e8m0_to_f32(scale_byte);
#pragma unroll
  for (int w = 0; w < 8; ++w) fp8_word_to_bf16(codes[w], s, out + 2 * w);
}

}  // namespace engram
