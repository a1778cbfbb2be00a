// MXFP8 quantization of the bf16 wkv input (staged rows viewed [T, K]).
//
// The pages quantize the WKV input to MXFP8 before the scaled GEMM
// ("vllm.models.deepseek_v41.nvidia.specialized_decode.engram.prefetch",
// module docstring; "vllm.models.deepseek_v41.amd.mono.attention.gemv",
// module docstring) without stating the rule. The rule implemented is the OCP
// Microscaling Formats (MX) v1.0 conversion to MXFP8-E4M3, per token and per
// 32 consecutive K elements:
//   X      = floor(log2(max |x|)) - 8          (8: exponent of e4m3's 448)
//   byte   = clamp(X + 127, 0, 254); 0 for an all-zero block
//   code   = e4m3fn(x * 2^(127 - byte)), nearest-even, saturating at 448,
//            sign bit kept
// All of it is integer work on the bf16 bit patterns plus one exact
// power-of-two multiply, so codes are reproducible bit for bit.
#include "common.h"

namespace engram {

namespace {

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

__global__ __launch_bounds__(256) void mx_quantize_kernel(
    const uint4* __restrict__ x, int64_t nblocks, uint4* __restrict__ xq,
    uint8_t* __restrict__ xs) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  uint4 in[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) in[i] = x[b * 4 + i];
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[4 * i + 0] = in[i].x; w[4 * i + 1] = in[i].y;
    w[4 * i + 2] = in[i].z; w[4 * i + 3] = in[i].w;
  }
  uint32_t amax = 0;  // bf16 magnitudes order like unsigned integers
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = max(amax, w[i] & 0x7fffu);
    amax = max(amax, (w[i] >> 16) & 0x7fffu);
  }
  int byte = 0;
  if (amax != 0) {
    const int X = bf16_floor_log2(amax) - 8;
    byte = min(max(X + 127, 0), 254);
  }
  // 2^(127 - byte): byte <= 246 for any finite bf16 input, a normal float
  const float inv_scale = __uint_as_float((uint32_t)(254 - byte) << 23);
  uint32_t packed[8];
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
  xq[b * 2 + 0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  xq[b * 2 + 1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  xs[b] = (uint8_t)byte;
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int64_t T, int K, uint8_t* xq,
                              uint8_t* xs, hipStream_t s) {
  const int64_t nblocks = T * (K / 32);
  const int grid = (int)((nblocks + 255) / 256);
  hipLaunchKernelGGL(mx_quantize_kernel, dim3(grid), dim3(256), 0, s,
                     (const uint4*)x, nblocks, (uint4*)xq, xs);
  return hipGetLastError();
}

}  // namespace engram
