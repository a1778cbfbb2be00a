// wkv projection for decode, MXFP8 weights: kv[T, N] = bf16(deq(xq) . deq(W)^T).
//
// Weight format: "vllm.models.deepseek_v41.amd.mono.attention.gemv", module
// docstring -- row-major e4m3 W[N, K] with one E8M0 byte per 32x32 block,
// S[N/32, K/32]. The activations arrive as MXFP8 rows (e4m3 codes [T, K] and
// one E8M0 byte per token and 32-element K block, [T, K/32]), produced by the
// quantize kernel.
//
// Operand layout of gfx950's scaled MFMAs (measured on the hardware with
// one-hot operands and distinct per-lane scales; the same layout for A and B):
//   v_mfma_scale_f32_16x16x128_f8f6f4: lane l holds row l%16; with g = l/16
//     its bytes 0..15 are k = 16g..16g+15 and bytes 16..31 are
//     k = 64+16g..64+16g+15; the E8M0 byte supplied by lane group g scales
//     the k block [32g, 32g+32).
//   v_mfma_scale_f32_32x32x64_f8f6f4: lane l holds row l%32; with g = l/32
//     bytes 0..15 are k = 16g.., bytes 16..31 are k = 32+16g..; lane group g
//     supplies the scale of k block [32g, 32g+32).
// So a row-major 128-byte (or 64-byte) k step is read as two 16-byte pieces
// per lane, and each lane passes the scale byte of k block g.
//
// Decode GEMV (T <= 64): weight-streaming. A workgroup owns 16 W rows;
//    its four waves split K into contiguous quarters, every lane keeps all of
//    its weight pieces in flight at once, tokens are padded to 16 on the MFMA
//    N side, and the four partial 16x16 tiles are summed in LDS in wave order
//    (fixed order, so results are deterministic).
#include "common.h"

namespace engram {

namespace {

__device__ __forceinline__ i32x8 cat(const uint4& lo, const uint4& hi) {
  const i32x4 a = __builtin_bit_cast(i32x4, lo);
  const i32x4 b = __builtin_bit_cast(i32x4, hi);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ------------------------------------------------------------------ GEMV --

constexpr int GV_THREADS = 256;
constexpr int GV_WAVES = 4;
constexpr int GV_ROWS = 16;

template <int NT, int SPW>  // token tiles of 16; 128-byte k steps per wave
__global__ __launch_bounds__(GV_THREADS) void gemv_mxfp8_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int T,
    int K, const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    int N, uint16_t* __restrict__ kv) {
  __shared__ f32x4 red[GV_WAVES][NT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * GV_ROWS;
  const int g = lane >> 4, r = lane & 15;
  const int kb = K / 32;
  const int nsteps = K / 128;
  const int step0 = wave * SPW;  // this wave's contiguous k range

  // weight operands of this wave's steps, all in flight
  uint4 wlo[SPW], whi[SPW];
  int wsc[SPW];
  const uint8_t* wrow = w + (int64_t)(n0 + r) * K;
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    wlo[s] = whi[s] = make_uint4(0, 0, 0, 0);
    wsc[s] = 0;
    if (step0 + s < nsteps) {
      const int kbyte = (step0 + s) * 128 + 16 * g;
      wlo[s] = *reinterpret_cast<const uint4*>(wrow + kbyte);
      whi[s] = *reinterpret_cast<const uint4*>(wrow + kbyte + 64);
      wsc[s] = ws[(n0 / 32) * kb + (step0 + s) * 4 + g];
    }
  }

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = j * 16 + r;
    const bool live = t < T;
    const uint8_t* xrow = xq + (int64_t)(live ? t : 0) * K;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (step0 + s >= nsteps) break;  // uniform per wave
      const int kbyte = (step0 + s) * 128 + 16 * g;
      uint4 xlo = make_uint4(0, 0, 0, 0), xhi = make_uint4(0, 0, 0, 0);
      int xsc = 0;
      if (live) {
        xlo = *reinterpret_cast<const uint4*>(xrow + kbyte);
        xhi = *reinterpret_cast<const uint4*>(xrow + kbyte + 64);
        xsc = xs[(int64_t)t * kb + (step0 + s) * 4 + g];
      }
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          cat(wlo[s], whi[s]), cat(xlo, xhi), acc[j], 0, 0, 0, wsc[s], 0, xsc);
    }
  }

#pragma unroll
  for (int j = 0; j < NT; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  // thread (tile, lane) sums the four waves' partials in wave order
  if (tid < NT * 64) {
    const int j = tid >> 6, l = tid & 63;
    f32x4 sum = red[0][j][l];
#pragma unroll
    for (int v = 1; v < GV_WAVES; ++v) {
      const f32x4 p = red[v][j][l];
      sum[0] += p[0]; sum[1] += p[1]; sum[2] += p[2]; sum[3] += p[3];
    }
    // C layout: lane l holds rows 4*(l/16)+i, token l%16
    const int t = j * 16 + (l & 15);
    if (t < T) {
      const int n = n0 + 4 * (l >> 4);
      uint2 o;
      o.x = pack_bf16x2(sum[0], sum[1]);
      o.y = pack_bf16x2(sum[2], sum[3]);
      *reinterpret_cast<uint2*>(kv + (int64_t)t * N + n) = o;
    }
  }
}

template <int NT>
hipError_t gemv_nt(const uint8_t* xq, const uint8_t* xs, int T, int K,
                   const uint8_t* w, const uint8_t* ws, int N, void* kv,
                   hipStream_t s) {
  const int spw = (K / 128 + GV_WAVES - 1) / GV_WAVES;
  const dim3 grid(N / GV_ROWS), block(GV_THREADS);
  switch (spw) {
#define GV_CASE(S)                                                            \
  case S:                                                                     \
    hipLaunchKernelGGL((gemv_mxfp8_kernel<NT, S>), grid, block, 0, s, xq, xs, \
                       T, K, w, ws, N, (uint16_t*)kv);                        \
    break;
    GV_CASE(1) GV_CASE(2) GV_CASE(3) GV_CASE(4) GV_CASE(5) GV_CASE(6)
    GV_CASE(7) GV_CASE(8)
#undef GV_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_mxfp8(const uint8_t* xq, const uint8_t* xs, int64_t T,
                             int K, const uint8_t* w, const uint8_t* ws, int N,
                             void* kv, hipStream_t s) {
  const int nt = (int)((T + 15) / 16);
  switch (nt) {
    case 1: return gemv_nt<1>(xq, xs, (int)T, K, w, ws, N, kv, s);
    case 2: return gemv_nt<2>(xq, xs, (int)T, K, w, ws, N, kv, s);
    case 3: return gemv_nt<3>(xq, xs, (int)T, K, w, ws, N, kv, s);
    case 4: return gemv_nt<4>(xq, xs, (int)T, K, w, ws, N, kv, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace engram
