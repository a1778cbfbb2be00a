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
// Decode GEMV (T <= 64): weight-streaming on the 16x16x128 scaled MFMA with
// tokens padded to 16 on the MFMA N side; the layout of the workgroups is
// described above the kernel.
#include "common.h"

namespace engram {

namespace {

__device__ __forceinline__ i32x8 cat(const uint4& lo, const uint4& hi) {
  const i32x4 a = __builtin_bit_cast(i32x4, lo);
  const i32x4 b = __builtin_bit_cast(i32x4, hi);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ------------------------------------------------------------------ GEMV --
//
// A workgroup of 8 waves owns RT tiles of 16 W rows (16*RT rows) and all T
// tokens (NT tiles of 16). Wave w takes the contiguous k steps
// [w*SPW, (w+1)*SPW) of every row tile, issues all of its weight loads first
// (RT*SPW*32 bytes per lane in flight), then its activation loads, then the
// MFMAs. The 8 partial 16x16 tiles of each (row tile, token tile) are summed
// through LDS in wave order. Fewer, larger workgroups mean each activation
// byte is re-read from L2 by N/(16*RT) workgroups instead of N/16.

constexpr int GV_WAVES = 8;
constexpr int GV_THREADS = GV_WAVES * 64;

template <int RT, int NT, int SPW>
__global__ __launch_bounds__(GV_THREADS) void gemv_mxfp8_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int T,
    int K, const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    int N, uint16_t* __restrict__ kv) {
  __shared__ f32x4 red[GV_WAVES][RT * NT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16 * RT;
  const int g = lane >> 4, r = lane & 15;
  const int kb = K / 32;
  const int nsteps = K / 128;
  const int step0 = wave * SPW;

  // Every load is issued before the first MFMA: weights, then activations.
  // Each sits behind its own (uniform) bounds test, which also keeps the
  // compiler from moving it next to its use; a padding token reloads token
  // 0 (its MFMA column only feeds outputs that are not stored).
  uint4 wlo[RT][SPW], whi[RT][SPW];
  int wsc[RT][SPW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int nrow = n0 + rt * 16;
    const uint8_t* wrow = w + (int64_t)(nrow + r) * K;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      wlo[rt][s] = whi[rt][s] = make_uint4(0, 0, 0, 0);
      wsc[rt][s] = 0;
      if (step0 + s < nsteps) {
        const int kbyte = (step0 + s) * 128 + 16 * g;
        wlo[rt][s] = *reinterpret_cast<const uint4*>(wrow + kbyte);
        whi[rt][s] = *reinterpret_cast<const uint4*>(wrow + kbyte + 64);
        wsc[rt][s] = ws[(nrow / 32) * kb + (step0 + s) * 4 + g];
      }
    }
  }
  uint4 xlo[NT][SPW], xhi[NT][SPW];
  int xsc[NT][SPW];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = j * 16 + r < T ? j * 16 + r : 0;
    const uint8_t* xrow = xq + (int64_t)t * K;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      xlo[j][s] = xhi[j][s] = make_uint4(0, 0, 0, 0);
      xsc[j][s] = 0;
      if (step0 + s < nsteps) {
        const int kbyte = (step0 + s) * 128 + 16 * g;
        xlo[j][s] = *reinterpret_cast<const uint4*>(xrow + kbyte);
        xhi[j][s] = *reinterpret_cast<const uint4*>(xrow + kbyte + 64);
        xsc[j][s] = xs[(int64_t)t * kb + (step0 + s) * 4 + g];
      }
    }
  }

  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (step0 + s >= nsteps) break;  // uniform per wave
      const i32x8 xb = cat(xlo[j][s], xhi[j][s]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            cat(wlo[rt][s], whi[rt][s]), xb, acc[rt][j], 0, 0, 0, wsc[rt][s], 0, xsc[j][s]);
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[wave][rt * NT + j][lane] = acc[rt][j];
  __syncthreads();
  // thread (tile pair, lane) sums the waves' partials in wave order
  for (int idx = tid; idx < RT * NT * 64; idx += GV_THREADS) {
    const int pair = idx >> 6, l = idx & 63;
    const int rt = pair / NT, j = pair - rt * NT;
    f32x4 sum = red[0][pair][l];
#pragma unroll
    for (int v = 1; v < GV_WAVES; ++v) {
      const f32x4 p = red[v][pair][l];
      sum[0] += p[0]; sum[1] += p[1]; sum[2] += p[2]; sum[3] += p[3];
    }
    // C layout: lane l holds rows 4*(l/16)+i, token l%16
    const int t = j * 16 + (l & 15);
    if (t < T) {
      const int n = n0 + rt * 16 + 4 * (l >> 4);
      uint2 o;
      o.x = pack_bf16x2(sum[0], sum[1]);
      o.y = pack_bf16x2(sum[2], sum[3]);
      *reinterpret_cast<uint2*>(kv + (int64_t)t * N + n) = o;
    }
  }
}

// The same GEMV for 2..4 token tiles with x staged in LDS. Holding all of
// x's fragments in registers limited the row tiles per workgroup (RT*NT <= 8:
// 640 workgroups at 64 tokens, each re-reading all of x, 84 MB of L2 reads for
// a 42 MB weight); here each workgroup copies x (codes and scale bytes) into
// LDS once with direct-to-LDS DMAs issued after its weight loads, so RT = 5
// at any NT: 256 workgroups of 80 rows. LDS row R (a token) holds its k
// pieces with piece p at p ^ (R & 15) inside each 256-byte run, so the 16 rows
// a fragment read touches fall on distinct banks. After the MFMAs the same
// LDS holds the waves' partial tiles for the fixed-order sum.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int RT, int NT>
constexpr int xlds_bytes(int K) {
  const int x = NT * 16 * K + ((NT * 16 * (K / 32) + 1023) & ~1023);
  const int red = GV_WAVES * RT * NT * 1024;
  return x > red ? x : red;
}

template <int RT, int NT, int SPW>
__global__ __launch_bounds__(GV_THREADS) void gemv_mxfp8_xlds_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int T,
    int K, const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws,
    int N, uint16_t* __restrict__ kv) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 16 * RT;
  const int g = lane >> 4, r = lane & 15;
  const int kb = K / 32;
  const int nsteps = K / 128;
  const int step0 = wave * SPW;
  constexpr int ROWS = NT * 16;

  uint4 wlo[RT][SPW], whi[RT][SPW];
  int wsc[RT][SPW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int nrow = n0 + rt * 16;
    const uint8_t* wrow = w + (int64_t)(nrow + r) * K;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      wlo[rt][s] = whi[rt][s] = make_uint4(0, 0, 0, 0);
      wsc[rt][s] = 0;
      if (step0 + s < nsteps) {
        const int kbyte = (step0 + s) * 128 + 16 * g;
        wlo[rt][s] = *reinterpret_cast<const uint4*>(wrow + kbyte);
        whi[rt][s] = *reinterpret_cast<const uint4*>(wrow + kbyte + 64);
        wsc[rt][s] = ws[(nrow / 32) * kb + (step0 + s) * 4 + g];
      }
    }
  }
  // x -> LDS: instruction q writes LDS bytes [1024q, 1024q + 1024), lane l
  // the 16 bytes at 1024q + 16l, i.e. row R, position p of that row; it
  // fetches piece p ^ (R & 15) of token R (zeros past T: the range check)
  {
    const rsrc_t rx = make_rsrc(xq, (uint32_t)(T * K));
    const rsrc_t rs = make_rsrc(xs, (uint32_t)(T * kb));
    const int pieces_row = K / 16;
    const int nq = ROWS * K / 1024;
    for (int q = wave; q < nq; q += GV_WAVES) {
      const int P = q * 64 + lane;             // LDS piece index
      const int R = P / pieces_row, p = P - R * pieces_row;
      const uint32_t voff = (uint32_t)R * (uint32_t)K + (uint32_t)((p ^ (R & 15)) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(lds + q * 1024), 16, voff, 0, 0, 0);
    }
    const int nqs = (ROWS * kb + 1023) / 1024;
    for (int q = wave; q < nqs; q += GV_WAVES)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(lds + ROWS * K + q * 1024), 16,
                                               (uint32_t)(q * 1024 + lane * 16), 0, 0, 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int R = j * 16 + r;
    const char* xrow = lds + R * K;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (step0 + s >= nsteps) break;  // uniform per wave
      const int P0 = (step0 + s) * 8 + g;     // the piece of k bytes 128*step + 16g; +4 is 64 bytes on
      const uint4 lo = *reinterpret_cast<const uint4*>(xrow + ((P0 ^ (R & 15)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(xrow + (((P0 + 4) ^ (R & 15)) << 4));
      const int xsc = (int)(uint8_t)lds[ROWS * K + R * kb + (step0 + s) * 4 + g];
      const i32x8 xb = cat(lo, hi);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            cat(wlo[rt][s], whi[rt][s]), xb, acc[rt][j], 0, 0, 0, wsc[rt][s], 0, xsc);
    }
  }

  __syncthreads();   // every wave is done with x in LDS
  f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[(wave * RT * NT + rt * NT + j) * 64 + lane] = acc[rt][j];
  __syncthreads();
  for (int idx = tid; idx < RT * NT * 64; idx += GV_THREADS) {
    const int pair = idx >> 6, l = idx & 63;
    const int rt = pair / NT, j = pair - rt * NT;
    f32x4 sum = red[pair * 64 + l];
#pragma unroll
    for (int v = 1; v < GV_WAVES; ++v) {
      const f32x4 pv = red[(v * RT * NT + pair) * 64 + l];
      sum[0] += pv[0]; sum[1] += pv[1]; sum[2] += pv[2]; sum[3] += pv[3];
    }
    const int t = j * 16 + (l & 15);
    if (t < T) {
      const int n = n0 + rt * 16 + 4 * (l >> 4);
      uint2 o;
      o.x = pack_bf16x2(sum[0], sum[1]);
      o.y = pack_bf16x2(sum[2], sum[3]);
      *reinterpret_cast<uint2*>(kv + (int64_t)t * N + n) = o;
    }
  }
}

template <int RT, int NT>
hipError_t gemv_xlds(const uint8_t* xq, const uint8_t* xs, int T, int K, const uint8_t* w, const uint8_t* ws,
                     int N, void* kv, hipStream_t s) {
  const int spw = (K / 128 + GV_WAVES - 1) / GV_WAVES;
  const int lds = xlds_bytes<RT, NT>(K);
  const dim3 grid(N / (16 * RT)), block(GV_THREADS);
  hipError_t e;
  switch (spw) {
#define GX_CASE(S)                                                                                     \
  case S:                                                                                              \
    e = hipFuncSetAttribute((const void*)gemv_mxfp8_xlds_kernel<RT, NT, S>,                            \
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);                          \
    if (e != hipSuccess) return e;                                                                     \
    hipLaunchKernelGGL((gemv_mxfp8_xlds_kernel<RT, NT, S>), grid, block, lds, s, xq, xs, T, K, w, ws, N, \
                       (uint16_t*)kv);                                                                 \
    break;
    GX_CASE(1) GX_CASE(2)
#undef GX_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int RT, int NT>
hipError_t gemv_rt(const uint8_t* xq, const uint8_t* xs, int T, int K,
                   const uint8_t* w, const uint8_t* ws, int N, void* kv,
                   hipStream_t s) {
  const int spw = (K / 128 + GV_WAVES - 1) / GV_WAVES;
  const dim3 grid(N / (16 * RT)), block(GV_THREADS);
  switch (spw) {
#define GV_CASE(S)                                                                \
  case S:                                                                         \
    hipLaunchKernelGGL((gemv_mxfp8_kernel<RT, NT, S>), grid, block, 0, s, xq, xs, \
                       T, K, w, ws, N, (uint16_t*)kv);                            \
    break;
    GV_CASE(1) GV_CASE(2) GV_CASE(3) GV_CASE(4)
#undef GV_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Row tiles per workgroup: the largest of 5, 4, 2, 1 that divides N/16 and
// keeps RT*NT <= 8 (LDS for the cross-wave sum and registers in flight).
template <int NT>
hipError_t gemv_nt(const uint8_t* xq, const uint8_t* xs, int T, int K,
                   const uint8_t* w, const uint8_t* ws, int N, void* kv,
                   hipStream_t s) {
  const int tiles = N / 16;
  // two or more token tiles: x in LDS when it fits (K % 256 == 0 for the
  // swizzle, at most 2 k steps per wave)
  if constexpr (NT >= 2) {
    if (tiles % 5 == 0 && K % 256 == 0 && K / 128 <= 2 * GV_WAVES && xlds_bytes<5, NT>(K) <= 160 * 1024)
      return gemv_xlds<5, NT>(xq, xs, T, K, w, ws, N, kv, s);
  }
  if constexpr (5 * NT <= 8)
    if (tiles % 5 == 0) return gemv_rt<5, NT>(xq, xs, T, K, w, ws, N, kv, s);
  if constexpr (4 * NT <= 8)
    if (tiles % 4 == 0) return gemv_rt<4, NT>(xq, xs, T, K, w, ws, N, kv, s);
  if (tiles % 2 == 0) return gemv_rt<2, NT>(xq, xs, T, K, w, ws, N, kv, s);
  return gemv_rt<1, NT>(xq, xs, T, K, w, ws, N, kv, s);
}


}  // namespace

bool gemv_mxfp8_supported(int64_t T, int K) {
  return T >= 1 && T <= kGemvMaxT && K % 128 == 0 && (K / 128 + GV_WAVES - 1) / GV_WAVES <= 4;
}

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
