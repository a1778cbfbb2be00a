// The OCP MX v1.0 conversion of 32 bf16 values to MXFP8-E4M3, used by the
// quantizer kernels in mxq.hip (which states the rule and why it is used).
#pragma once

#include "common.h"

namespace engram {

// |v| as fp32 with v in [0, 512): e4m3fn magnitude code (0..0x7E).
__device__ __forceinline__ uint32_t e4m3_mag_code(float v) {
  const uint32_t u = __float_as_uint(v);
  if (u >= 0x43e00000u) return 0x7eu;  // >= 448: saturate
  if (u < 0x3c800000u) {               // < 2^-6: subnormal step 2^-9
    return (uint32_t)__builtin_rintf(v * 512.0f);  // 0..8 (8 = 2^-6, code 0x08)
  }
  // normal: keep 3 of fp32's 23 mantissa bits, nearest-even; a carry moves
  // into the exponent field, which the code layout absorbs.
  const uint32_t r = u + 0x7ffffu + ((u >> 20) & 1u);
  uint32_t code = (r >> 20) - (120u << 3);  // exponent bias 127 -> 7
  return code > 0x7eu ? 0x7eu : code;
}

// floor(log2(a)) of a non-zero bf16 magnitude given by its 15 low bits.
__device__ __forceinline__ int bf16_floor_log2(uint32_t mag) {
  const int e = (int)(mag >> 7);
  if (e > 0) return e - 127;
  // subnormal: m * 2^-133 with 1 <= m < 128
  return (31 - __builtin_clz(mag)) - 133;
}

// Quantize one 32-element block (16 words of bf16 pairs) -> 8 code words + scale byte.
// A block holding an infinity or a NaN gets scale byte 255 (the E8M0 NaN)
// and every code 0x7F (the e4m3fn NaN).
__device__ __forceinline__ int mx_block(const uint32_t* w, uint32_t* packed) {
  uint32_t amax = 0;  // bf16 magnitudes order like unsigned integers
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = max(amax, w[i] & 0x7fffu);
    amax = max(amax, (w[i] >> 16) & 0x7fffu);
  }
  if (amax >= 0x7f80u) {
    // an infinity or a NaN in the block: no finite shared exponent; the block
    // becomes the E8M0 NaN scale with e4m3fn NaN codes (decodes to NaN)
#pragma unroll
    for (int i = 0; i < 8; ++i) packed[i] = 0x7f7f7f7fu;
    return 255;
  }
  int byte = 0;
  if (amax != 0) {
    const int X = bf16_floor_log2(amax) - 8;
    byte = min(max(X + 127, 0), 254);
  }
  // 2^(127 - byte): byte <= 246 for any finite bf16 input, a normal float
  const float inv_scale = __uint_as_float((uint32_t)(254 - byte) << 23);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * i + j;  // element index within the block
      const uint32_t bits = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu);
      const float mag = __uint_as_float((bits & 0x7fffu) << 16) * inv_scale;
      const uint32_t code = e4m3_mag_code(mag) | ((bits >> 8) & 0x80u);
      word |= code << (8 * j);
    }
    packed[i] = word;
  }
  return byte;
}


}  // namespace engram
