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
// A block holding an infinity or a NaN has no finite maximum: it is given
// the E8M0 NaN scale (byte 255) and the e4m3fn NaN code 0x7F everywhere, so
// it decodes to NaN (an MX NaN scale makes its whole block NaN).
// The gather can be fused in front (gather_quantize_kernel): the bf16 staged
// rows then never reach HBM. All of it is integer work on the bf16 bit patterns plus one exact
// power-of-two multiply, so codes are reproducible bit for bit.
#include "common.h"
#include "fp8_table.h"
#include "mx_rule.h"

namespace engram {

namespace {

__global__ __launch_bounds__(256) void mx_quantize_kernel(
    const uint4* __restrict__ x, int64_t nblocks, uint4* __restrict__ xq,
    uint8_t* __restrict__ xs) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  uint32_t w[16], packed[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = x[b * 4 + i];
    w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  const int byte = mx_block(w, packed);
  xq[b * 2 + 0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  xq[b * 2 + 1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  xs[b] = (uint8_t)byte;
}

// Row gather fused with the quantizer: block b of token t is 32 elements of
// staged row c = (b*32) / head_dim, so the bf16 rows are never written. With
// an fp8 table (scales != nullptr) the block is dequantized to bf16 first
// (fp8_table.h), then quantized by the same MX rule.
template <bool FP8>
__global__ __launch_bounds__(256) void gather_quantize_kernel(
    const uint4* __restrict__ table, const uint8_t* __restrict__ scales, int64_t num_rows, int head_dim,
    const int32_t* __restrict__ ids, int64_t st, int64_t sc, int n_cols,
    int64_t nblocks, uint4* __restrict__ xq, uint8_t* __restrict__ xs,
    int32_t* __restrict__ err) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const int bpr = head_dim / 32;                 // blocks per staged row
  const int64_t row = b / bpr;                   // (t, c) flattened
  const int part = (int)(b - row * bpr);
  const int64_t t = row / n_cols;
  const int c = (int)(row - t * n_cols);
  const int64_t id = ids[t * st + (int64_t)c * sc];
  uint32_t w[16], packed[8];
  if (id >= 0 && id < num_rows) {
    if constexpr (FP8) {
      const int64_t blk = id * bpr + part;
      const uint4 c0 = table[blk * 2], c1 = table[blk * 2 + 1];
      const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      fp8_block_to_bf16(cw, scales[blk], w);
    } else {
      const uint4* src = table + (id * head_dim + part * 32) / 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = src[i];
        w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = 0u;
    if (err) atomicOr(err, 1);
  }
  const int byte = mx_block(w, packed);
  xq[b * 2 + 0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  xq[b * 2 + 1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  xs[b] = (uint8_t)byte;
}

}  // namespace

hipError_t launch_gather_quantize(const void* table, const uint8_t* table_scales, int64_t num_rows,
                                  int head_dim, const int32_t* ids, int64_t st, int64_t sc, int64_t T,
                                  int n_cols, uint8_t* xq, uint8_t* xs, int32_t* err, hipStream_t s) {
  const int64_t nblocks = T * n_cols * (head_dim / 32);
  const int grid = (int)((nblocks + 255) / 256);
  if (table_scales)
    hipLaunchKernelGGL(gather_quantize_kernel<true>, dim3(grid), dim3(256), 0, s, (const uint4*)table,
                       table_scales, num_rows, head_dim, ids, st, sc, n_cols, nblocks, (uint4*)xq, xs, err);
  else
    hipLaunchKernelGGL(gather_quantize_kernel<false>, dim3(grid), dim3(256), 0, s, (const uint4*)table,
                       nullptr, num_rows, head_dim, ids, st, sc, n_cols, nblocks, (uint4*)xq, xs, err);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(const void* x, int64_t T, int K, uint8_t* xq,
                              uint8_t* xs, hipStream_t s) {
  const int64_t nblocks = T * (K / 32);
  const int grid = (int)((nblocks + 255) / 256);
  hipLaunchKernelGGL(mx_quantize_kernel, dim3(grid), dim3(256), 0, s,
                     (const uint4*)x, nblocks, (uint4*)xq, xs);
  return hipGetLastError();
}

}  // namespace engram
