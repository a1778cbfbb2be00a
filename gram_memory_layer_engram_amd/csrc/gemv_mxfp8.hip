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
#include "mx_rule.h"

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

  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

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
      const i32x8 xb = cat(xlo, xhi);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            cat(wlo[rt][s], whi[rt][s]), xb, acc[rt][j], 0, 0, 0, wsc[rt][s], 0, xsc);
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
  if constexpr (5 * NT <= 8)
    if (tiles % 5 == 0) return gemv_rt<5, NT>(xq, xs, T, K, w, ws, N, kv, s);
  if constexpr (4 * NT <= 8)
    if (tiles % 4 == 0) return gemv_rt<4, NT>(xq, xs, T, K, w, ws, N, kv, s);
  if (tiles % 2 == 0) return gemv_rt<2, NT>(xq, xs, T, K, w, ws, N, kv, s);
  return gemv_rt<1, NT>(xq, xs, T, K, w, ws, N, kv, s);
}


// Fused decode projection (T <= 32): gather + MXFP8 quantize of the
// activations straight into LDS, then the same weight-streaming GEMV. Vector
// memory returns in order within a wave, so a wave that has its weight loads
// in flight cannot use a later load before all of them land; the workgroup
// therefore has 8 weight waves, which issue their loads at kernel start, and
// GQ_WAVES gather waves, which fetch ids and table rows (L2-resident after
// the first workgroup of each XCD touches them) and quantize them into LDS
// while the weight stream is in flight. Both meet at one barrier.
// LDS: x codes [TP][K + 16] (16-byte row pad: the 16 rows one MFMA operand
// read touches land in different banks), x scales [TP][K/32], and the
// cross-wave reduction buffer.
constexpr int GQ_WAVES = 4;
constexpr int DEC_THREADS = (GV_WAVES + GQ_WAVES) * 64;

template <int RT, int NT, int SPW>
__global__ __launch_bounds__(DEC_THREADS) void decode_wkv_kernel(
    const uint4* __restrict__ table, int64_t num_rows, int head_dim,
    const int32_t* __restrict__ ids, int64_t st, int64_t sc, int n_cols, int T, int K,
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, int N,
    uint16_t* __restrict__ kv, int32_t* __restrict__ err) {
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  constexpr int TP = NT * 16;
  const int pitch = K + 16;
  uint8_t* xq_s = dsm;
  uint8_t* xs_s = dsm + TP * pitch;
  f32x4* red = reinterpret_cast<f32x4*>(dsm + ((TP * pitch + TP * (K / 32) + 15) & ~15));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16 * RT;
  const int g = lane >> 4, r = lane & 15;
  const int kb = K / 32;
  const int nsteps = K / 128;
  const int step0 = wave * SPW;

  const bool wwave = wave < GV_WAVES;
  // 1. weight waves: the weight stream starts first
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
      if (wwave && step0 + s < nsteps) {
        const int kbyte = (step0 + s) * 128 + 16 * g;
        wlo[rt][s] = *reinterpret_cast<const uint4*>(wrow + kbyte);
        whi[rt][s] = *reinterpret_cast<const uint4*>(wrow + kbyte + 64);
        wsc[rt][s] = ws[(nrow / 32) * kb + (step0 + s) * 4 + g];
      }
    }
  }

  // 2. gather waves: gather + quantize x into LDS (tokens T..TP-1 are zero)
  if (!wwave) {
    const int bpr = head_dim / 32;
    const int nblk = TP * kb;
    for (int b = tid - GV_THREADS; b < nblk; b += GQ_WAVES * 64) {
      const int t = b / kb, blk = b - t * kb;
      uint32_t wv[16], packed[8];
#pragma unroll
      for (int i = 0; i < 16; ++i) wv[i] = 0u;
      if (t < T) {
        const int c = blk / bpr, part = blk - c * bpr;
        const int64_t id = ids[(int64_t)t * st + (int64_t)c * sc];
        if (id >= 0 && id < num_rows) {
          const uint4* src = table + (id * head_dim + part * 32) / 8;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 v = src[i];
            wv[4 * i + 0] = v.x; wv[4 * i + 1] = v.y; wv[4 * i + 2] = v.z; wv[4 * i + 3] = v.w;
          }
        } else if (err && blockIdx.x == 0) {
          atomicOr(err, 1);
        }
      }
      const int byte = mx_block(wv, packed);
      uint4* dst = reinterpret_cast<uint4*>(xq_s + t * pitch + blk * 32);
      dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      xs_s[t * kb + blk] = (uint8_t)byte;
    }
  }
  __syncthreads();

  // 3. MFMAs against the LDS activations
  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (!wwave) break;
    const int t = j * 16 + r;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (step0 + s >= nsteps) break;  // uniform per wave
      const int kbyte = (step0 + s) * 128 + 16 * g;
      const uint4 xlo = *reinterpret_cast<const uint4*>(xq_s + t * pitch + kbyte);
      const uint4 xhi = *reinterpret_cast<const uint4*>(xq_s + t * pitch + kbyte + 64);
      const int xsc = xs_s[t * kb + (step0 + s) * 4 + g];
      const i32x8 xb = cat(xlo, xhi);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            cat(wlo[rt][s], whi[rt][s]), xb, acc[rt][j], 0, 0, 0, wsc[rt][s], 0, xsc);
    }
  }

  // 4. wave-ordered reduction and bf16 store
  if (wwave) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int j = 0; j < NT; ++j) red[(wave * RT * NT + rt * NT + j) * 64 + lane] = acc[rt][j];
  }
  __syncthreads();
  for (int idx = tid; idx < RT * NT * 64; idx += DEC_THREADS) {
    const int pair = idx >> 6, l = idx & 63;
    const int rt = pair / NT, j = pair - rt * NT;
    f32x4 sum = red[pair * 64 + l];
#pragma unroll
    for (int v = 1; v < GV_WAVES; ++v) {
      const f32x4 p = red[(v * RT * NT + pair) * 64 + l];
      sum[0] += p[0]; sum[1] += p[1]; sum[2] += p[2]; sum[3] += p[3];
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
size_t decode_lds_bytes(int K) {
  constexpr int TP = NT * 16;
  const size_t x = (size_t)TP * (K + 16) + (size_t)TP * (K / 32);
  return ((x + 15) & ~(size_t)15) + (size_t)GV_WAVES * RT * NT * 64 * 16;
}

template <int RT, int NT>
hipError_t decode_rt(const void* table, int64_t num_rows, int head_dim, const int32_t* ids,
                     int64_t st, int64_t sc, int n_cols, int T, int K, const uint8_t* w,
                     const uint8_t* ws, int N, void* kv, int32_t* err, hipStream_t s) {
  const int spw = (K / 128 + GV_WAVES - 1) / GV_WAVES;
  const size_t lds = decode_lds_bytes<RT, NT>(K);
  const dim3 grid(N / (16 * RT)), block(DEC_THREADS);
  hipError_t e;
  switch (spw) {
#define DEC_CASE(S)                                                                              \
  case S:                                                                                        \
    e = hipFuncSetAttribute((const void*)decode_wkv_kernel<RT, NT, S>,                           \
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);               \
    if (e != hipSuccess) return e;                                                               \
    hipLaunchKernelGGL((decode_wkv_kernel<RT, NT, S>), grid, block, lds, s, (const uint4*)table, \
                       num_rows, head_dim, ids, st, sc, n_cols, T, K, w, ws, N, (uint16_t*)kv,   \
                       err);                                                                     \
    break;
    DEC_CASE(1) DEC_CASE(2)
#undef DEC_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool gemv_mxfp8_supported(int64_t T, int K) {
  return T >= 1 && T <= kGemvMaxT && K % 128 == 0 && (K / 128 + GV_WAVES - 1) / GV_WAVES <= 4;
}

bool decode_wkv_supported(int64_t T, int K, int N, int head_dim) {
  if (T < 1 || T > 32 || K % 128 != 0 || head_dim % 32 != 0 || N % 32 != 0) return false;
  // 12 waves per workgroup leave ~168 registers per lane: at most 2 k steps per wave
  if ((K / 128 + GV_WAVES - 1) / GV_WAVES > 2) return false;
  const size_t lds = T <= 16 ? decode_lds_bytes<5, 1>(K) : decode_lds_bytes<4, 2>(K);
  return lds <= 160 * 1024;
}

hipError_t launch_decode_wkv(const void* table, int64_t num_rows, int head_dim,
                             const int32_t* ids, int64_t st, int64_t sc, int n_cols, int64_t T,
                             int K, const uint8_t* w, const uint8_t* ws, int N, void* kv,
                             int32_t* err, hipStream_t s) {
  const int tiles = N / 16;
  if (T <= 16) {
    if (tiles % 5 == 0) return decode_rt<5, 1>(table, num_rows, head_dim, ids, st, sc, n_cols, (int)T, K, w, ws, N, kv, err, s);
    if (tiles % 4 == 0) return decode_rt<4, 1>(table, num_rows, head_dim, ids, st, sc, n_cols, (int)T, K, w, ws, N, kv, err, s);
    return decode_rt<2, 1>(table, num_rows, head_dim, ids, st, sc, n_cols, (int)T, K, w, ws, N, kv, err, s);
  }
  if (tiles % 4 == 0) return decode_rt<4, 2>(table, num_rows, head_dim, ids, st, sc, n_cols, (int)T, K, w, ws, N, kv, err, s);
  return decode_rt<2, 2>(table, num_rows, head_dim, ids, st, sc, n_cols, (int)T, K, w, ws, N, kv, err, s);
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
