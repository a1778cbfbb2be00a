// Measurement probes: not steps of the layer. They measure the rates this
// chip sustains, so that each kernel's achieved rate can be quoted against
// a measured ceiling as well as against the datasheet peak:
//  * a register-only MFMA loop (bf16 32x32x16, or MXFP8 32x32x64 scaled):
//    the matrix cores' rate at the clock the chip holds with nothing but
//    MFMAs running;
//  * a streaming read, and an R:1 streaming read/write (R = 1: a copy) of
//    16-byte pieces (HBM).
#include "common.h"

namespace engram {

namespace {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_CHAINS = 8;        // independent accumulators per wave
constexpr int PROBE_MFMA_WG_PER_CU = 2;
constexpr int PROBE_OUT_WG_PER_CU = 4;   // out words: this many workgroups' threads per CU
// 16-byte pieces per thread. The memory probes run as one pass of
// short-lived workgroups that covers the buffer (four pieces per thread,
// all loads issued before the first use): on MI355X that streams faster
// than a grid of a few workgroups per compute unit looping over the buffer
// (6.1 against 5.4 TB/s read, 5.8 against 4.5 TB/s copy, 4 GiB).
constexpr int PROBE_UNROLL = 4;

// Every lane runs PROBE_CHAINS independent accumulator chains, so a wave can
// issue MFMAs back to back (a chain's next MFMA comes 8 MFMAs later, past
// the instruction's latency). Operands are constants: bf16 2^-8 (each step
// adds 16 * 2^-16 = 2^-12 to every accumulator) or e4m3 1.0 with E8M0 scale
// 2^0 (each step adds 64). The lane's sum of its accumulators is stored, so
// nothing is dead code and the result is known in closed form.
template <bool FP8>
__global__ __launch_bounds__(PROBE_THREADS) void mfma_probe_kernel(int iters, float* __restrict__ out) {
  f32x16 acc[PROBE_CHAINS];
#pragma unroll
  for (int j = 0; j < PROBE_CHAINS; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
  if constexpr (FP8) {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x38383838;   // e4m3 1.0
      b[e] = 0x38383838;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < PROBE_CHAINS; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 127);
    }
  } else {
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)0.00390625f;   // 2^-8
      b[e] = (__bf16)0.00390625f;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < PROBE_CHAINS; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < PROBE_CHAINS; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(int64_t)blockIdx.x * PROBE_THREADS + threadIdx.x] = s;
}

// An empty asm that takes v as an in/out operand and clobbers memory: loads
// cannot move below it and no use of v can move above it.
__device__ __forceinline__ void pin(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)::"memory");
}

__device__ __forceinline__ uint32_t xor4(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }
__device__ __forceinline__ uint4 xor16(const uint4& a, const uint4& b) {
  return make_uint4(a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w);
}

// Streaming read of n16 16-byte pieces: each thread issues its PROBE_UNROLL
// loads (pieces base + u*stride, clamped to the last piece, so no branch
// stands between them) before it uses any; the grid covers the buffer, so
// clamped pieces occur only in the tail, and they are not counted. The XOR
// of every word read ends up in out.
__global__ __launch_bounds__(PROBE_THREADS) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                   uint32_t* __restrict__ out, int64_t n_out) {
  const int64_t stride = (int64_t)gridDim.x * PROBE_THREADS;
  uint32_t x = 0;
  for (int64_t base = (int64_t)blockIdx.x * PROBE_THREADS + threadIdx.x; base < n16;
       base += PROBE_UNROLL * stride) {
    uint4 v[PROBE_UNROLL];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = src[min(base + u * stride, n16 - 1)];
    // every load is issued before the first use: the values are pinned here
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) pin(v[u]);
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u)
      if (base + u * stride < n16) x ^= xor4(v[u]);
  }
  // XOR over the wave, then one atomic XOR per wave into out (zeroed by the
  // caller), folding waves beyond out's n_out words onto it
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  const int64_t wave = ((int64_t)blockIdx.x * PROBE_THREADS + threadIdx.x) >> 6;
  if ((threadIdx.x & 63) == 0) atomicXor(out + wave % n_out, x);
}

// Streaming R:1 read/write: dst piece d = XOR over j < R of src piece
// j*n16 + d (R coalesced read streams, one write stream; R = 1 is a copy).
// Loads of a sweep all go out before the first store, as above.
template <int R>
__global__ __launch_bounds__(PROBE_THREADS) void stream_probe_kernel(const uint4* __restrict__ src,
                                                                     uint4* __restrict__ dst, int64_t n16) {
  constexpr int U = PROBE_UNROLL / 2 > 0 ? PROBE_UNROLL / 2 : 1;
  const int64_t stride = (int64_t)gridDim.x * PROBE_THREADS;
  for (int64_t base = (int64_t)blockIdx.x * PROBE_THREADS + threadIdx.x; base < n16; base += U * stride) {
    uint4 v[R][U];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) v[j][u] = src[j * n16 + min(base + u * stride, n16 - 1)];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) pin(v[j][u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint4 o = v[0][u];
#pragma unroll
      for (int j = 1; j < R; ++j) o = xor16(o, v[j][u]);
      if (base + u * stride < n16) dst[base + u * stride] = o;
    }
  }
}

// Workgroups for one pass over n16 pieces at `unroll` pieces per thread
// (capped at 2^30; past that the threads loop).
int64_t mem_grid(int64_t n16, int unroll) {
  const int64_t per_block = (int64_t)PROBE_THREADS * unroll;
  const int64_t b = (n16 + per_block - 1) / per_block;
  return b < 1 ? 1 : (b > (1 << 30) ? (1 << 30) : b);
}

}  // namespace

int probe_mfma_blocks() { return dev_info().num_cus * PROBE_MFMA_WG_PER_CU; }
int probe_mem_blocks() { return dev_info().num_cus * PROBE_OUT_WG_PER_CU; }

int probe_threads() { return PROBE_THREADS; }
int probe_chains() { return PROBE_CHAINS; }

hipError_t launch_probe_mfma(bool fp8, int iters, float* out, hipStream_t s) {
  const dim3 grid(probe_mfma_blocks()), block(PROBE_THREADS);
  if (fp8)
    hipLaunchKernelGGL(mfma_probe_kernel<true>, grid, block, 0, s, iters, out);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<false>, grid, block, 0, s, iters, out);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, int64_t n16, uint32_t* out, hipStream_t s) {
  // out holds probe_mem_blocks() * PROBE_THREADS words: a one-pass grid
  // larger than that folds onto them (XOR is order-free)
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)mem_grid(n16, PROBE_UNROLL)), dim3(PROBE_THREADS), 0, s,
                     (const uint4*)src, n16, out, (int64_t)probe_mem_blocks() * PROBE_THREADS);
  return hipGetLastError();
}

hipError_t launch_probe_stream(const void* src, void* dst, int64_t n16, int ratio, hipStream_t s) {
  const dim3 grid((unsigned)mem_grid(n16, PROBE_UNROLL / 2)), block(PROBE_THREADS);
  const uint4* a = (const uint4*)src;
  uint4* b = (uint4*)dst;
  switch (ratio) {
    case 1: hipLaunchKernelGGL(stream_probe_kernel<1>, grid, block, 0, s, a, b, n16); break;
    case 2: hipLaunchKernelGGL(stream_probe_kernel<2>, grid, block, 0, s, a, b, n16); break;
    case 3: hipLaunchKernelGGL(stream_probe_kernel<3>, grid, block, 0, s, a, b, n16); break;
    default: hipLaunchKernelGGL(stream_probe_kernel<4>, grid, block, 0, s, a, b, n16); break;
  }
  return hipGetLastError();
}

}  // namespace engram
