// wkv projection, tiled GEMM for prefill: kv[T, N] = bf16(x[T, K] . W[N, K]^T)
// with bf16 weights (v_mfma_f32_32x32x16_bf16) or MXFP8 weights and MXFP8
// activations (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// "vllm.models.deepseek_v4_1.common.engram", Engram.__init__ / forward: wkv
// is a bias-free linear from n_hash_cols*head_dim (K) to dim*(hc_mult+1) (N)
// on the flattened staged rows. MXFP8 weight format: "vllm.models.
// deepseek_v41.amd.mono.attention.gemv", module docstring (row-major e4m3
// W[N, K], E8M0 byte per 32x32 block S[N/32, K/32]).
//
// MI355X design
//  * Both operands are K-contiguous, so an operand tile is 256 rows of 128
//    bytes per k stage (64 bf16 or 128 e4m3), i.e. 8 pieces of 16 bytes.
//  * A = W rows (n), B = x rows (tokens): an accumulator lane then holds 4
//    consecutive n of one token, written as one 8-byte bf16x4 store.
//  * Block tile 256 (n) x 256 (tokens); four waves in 2x2, each 128x128 =
//    4x4 MFMA tiles of 32x32 (256 fp32 accumulators per lane, in AGPRs).
//  * Global -> LDS with buffer_load ... lds (16 bytes per lane, written at
//    LDS base + lane*16): no staging registers, no ds_write, and the buffer
//    descriptor's range check returns zeros past the last row of W or x, so
//    ragged tiles need no branches. Two LDS stages (2 x 64 KiB); the loads of
//    stage k+1 are issued right after the barrier that ends stage k-1 and run
//    under stage k's MFMAs.
//  * LDS rows are 128 B; piece p of row r sits at p ^ ((r >> 1) & 7). The DMA
//    writes 64 consecutive pieces per instruction (8 rows), so each lane
//    fetches the global piece that belongs at its slot.
//  * MFMA operand fragments are double-buffered in registers: the ds_reads of
//    sub-step kk+1 are issued before the MFMAs of sub-step kk.
//  * Tile order is XCD-aware (workgroup ids are dealt round-robin over the 8
//    XCDs): ids are regrouped per XCD, then walked in groups of 4 token tiles
//    so the 32 workgroups an XCD runs at once share 4 x-tiles and 8 W-tiles
//    in its L2.
//  * MXFP8: gfx950's 32x32x64 scaled MFMA takes, in lane l (row l%32, group
//    g = l/32), k bytes 16g..16g+15 and 32+16g..32+16g+15 of its 64-k step,
//    and lane group g's E8M0 byte scales k block [32g, 32g+32) (measured on
//    the hardware). Each lane therefore reads pieces 4s+g and 4s+2+g of the
//    stage for sub-step s and passes byte 2s+g of the stage's 4 scale bytes.
#include "common.h"

namespace engram {

namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BM = 256;      // W rows per block
constexpr int BN = 256;      // tokens per block
constexpr int ROW_BYTES = 128;
constexpr int PIECES = ROW_BYTES / 16;
constexpr int THREADS = 256;
constexpr int TILE_BYTES = BM * ROW_BYTES;       // 32 KiB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;      // A + B
constexpr int LDS_BYTES = 2 * STAGE_BYTES;       // two stages
constexpr int GROUP_T = 4;
constexpr uint32_t RSRC_FLAGS = 0x00020000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, RSRC_FLAGS);
}

__device__ __forceinline__ int swz(int row, int piece) {
  return row * PIECES + (piece ^ ((row >> 1) & 7));
}

__device__ __forceinline__ void tile_of(int bid, int tiles_n, int tiles_t, int& tn, int& tt) {
  const int total = tiles_n * tiles_t;
  const int q = total / 8, r = total % 8;
  const int xcd = bid % 8, slot = bid / 8;
  const int logical = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
  const int per_group = GROUP_T * tiles_n;
  const int group = logical / per_group;
  const int first_t = group * GROUP_T;
  const int gsize = min(tiles_t - first_t, GROUP_T);
  const int in_group = logical - group * per_group;
  tt = first_t + in_group % gsize;
  tn = in_group / gsize;
}

__device__ __forceinline__ i32x8 cat8(const uint4& lo, const uint4& hi) {
  return __builtin_shufflevector(__builtin_bit_cast(i32x4, lo), __builtin_bit_cast(i32x4, hi),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// One k stage of both operand tiles, global -> LDS. Wave w issues 8 DMA
// instructions per operand; instruction i fills rows 8*(w + 4*i) .. +8.
// `kb` is the stage's byte offset inside a row; `row_bytes` the global row
// pitch; `kmax` the valid bytes of a row (pieces at or past it read zeros).
template <bool KTAIL>
__device__ __forceinline__ void stage_load(rsrc_t ra, rsrc_t rb, char* lds_stage, int wave, int lane,
                                           uint32_t row_bytes, uint32_t kb, uint32_t kmax) {
  const int sub = lane >> 3, pp = lane & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = wave + 4 * i;
    const int r = blk * 8 + sub;
    const int p = pp ^ ((r >> 1) & 7);
    uint32_t off = (uint32_t)r * row_bytes + kb + (uint32_t)p * 16u;
    if (KTAIL && kb + (uint32_t)p * 16u >= kmax) off = 0xfffffff0u;  // past the range: zeros
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(lds_stage + blk * 1024), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(lds_stage + TILE_BYTES + blk * 1024), 16, off, 0, 0, 0);
  }
}

template <bool KTAIL>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint16_t* __restrict__ x, int T, int K, const uint16_t* __restrict__ w,
                      int N, uint16_t* __restrict__ kv, int tiles_n, int tiles_t) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int tn, tt;
  tile_of(blockIdx.x, tiles_n, tiles_t, tn, tt);
  const int n0 = tn * BM, t0 = tt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = (wave >> 1) * 128, wt = (wave & 1) * 128;
  const uint32_t row_bytes = (uint32_t)K * 2u;
  const rsrc_t ra = make_rsrc(w + (int64_t)n0 * K, (uint32_t)min(BM, N - n0) * row_bytes);
  const rsrc_t rb = make_rsrc(x + (int64_t)t0 * K, (uint32_t)min(BN, T - t0) * row_bytes);
  const int nk = (K + 63) / 64;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int lrow = lane & 31, lhalf = lane >> 5;
  stage_load<KTAIL>(ra, rb, smem, wave, lane, row_bytes, 0, row_bytes);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE_BYTES;
    if (kt + 1 < nk)
      stage_load<KTAIL>(ra, rb, smem + ((kt + 1) & 1) * STAGE_BYTES, wave, lane, row_bytes,
                        (uint32_t)(kt + 1) * 128u, row_bytes);
    const uint4* As = reinterpret_cast<const uint4*>(cur);
    const uint4* Bs = reinterpret_cast<const uint4*>(cur + TILE_BYTES);
    bf16x8_t a[2][4], b[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[0][i] = __builtin_bit_cast(bf16x8_t, As[swz(wn + i * 32 + lrow, lhalf)]);
      b[0][i] = __builtin_bit_cast(bf16x8_t, Bs[swz(wt + i * 32 + lrow, lhalf)]);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk & 1;
      if (kk < 3) {
        const int piece = (kk + 1) * 2 + lhalf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[c ^ 1][i] = __builtin_bit_cast(bf16x8_t, As[swz(wn + i * 32 + lrow, piece)]);
          b[c ^ 1][i] = __builtin_bit_cast(bf16x8_t, Bs[swz(wt + i * 32 + lrow, piece)]);
        }
      }
      // keep the next sub-step's LDS reads ahead of this sub-step's MFMAs
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // accumulator r of lane l: n = 8*(r/4) + 4*(l/32) + r%4, token = l%32
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + wt + j * 32 + lrow;
    if (t >= T) continue;
    uint16_t* krow = kv + (int64_t)t * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn + i * 32 + 8 * g + 4 * lhalf;
        if (n + 4 <= N) {
          uint2 o;
          o.x = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
          o.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *reinterpret_cast<uint2*>(krow + n) = o;
        }
      }
  }
}

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mxfp8_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int T, int K,
                       const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, int N,
                       uint16_t* __restrict__ kv, int tiles_n, int tiles_t) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int tn, tt;
  tile_of(blockIdx.x, tiles_n, tiles_t, tn, tt);
  const int n0 = tn * BM, t0 = tt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = (wave >> 1) * 128, wt = (wave & 1) * 128;
  const uint32_t row_bytes = (uint32_t)K;
  const rsrc_t ra = make_rsrc(w + (int64_t)n0 * K, (uint32_t)min(BM, N - n0) * row_bytes);
  const rsrc_t rb = make_rsrc(xq + (int64_t)t0 * K, (uint32_t)min(BN, T - t0) * row_bytes);
  const int nk = K / 128;
  const int kb = K / 32;
  const int lrow = lane & 31, lg = lane >> 5;

  // per-lane scale words (4 E8M0 bytes = one k stage) of its A and B tiles
  const uint32_t* wsa[4];
  const uint32_t* xsb[4];
  bool live_t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nb = min((n0 + wn + i * 32) / 32, N / 32 - 1);
    wsa[i] = reinterpret_cast<const uint32_t*>(ws + (int64_t)nb * kb);
    const int t = t0 + wt + i * 32 + lrow;
    live_t[i] = t < T;
    xsb[i] = reinterpret_cast<const uint32_t*>(xs + (int64_t)(live_t[i] ? t : 0) * kb);
  }
  uint32_t sa[4], sb[4];
  auto scale_load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = wsa[i][kt];
      sb[i] = live_t[i] ? xsb[i][kt] : 0u;
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  stage_load<false>(ra, rb, smem, wave, lane, row_bytes, 0, row_bytes);
  scale_load(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE_BYTES;
    uint32_t csa[4], csb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { csa[i] = sa[i]; csb[i] = sb[i]; }
    if (kt + 1 < nk) {
      stage_load<false>(ra, rb, smem + ((kt + 1) & 1) * STAGE_BYTES, wave, lane, row_bytes,
                        (uint32_t)(kt + 1) * 128u, row_bytes);
      scale_load(kt + 1);
    }
    const uint4* As = reinterpret_cast<const uint4*>(cur);
    const uint4* Bs = reinterpret_cast<const uint4*>(cur + TILE_BYTES);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int p_lo = 4 * s + lg, p_hi = 4 * s + 2 + lg;
      const int shift = 8 * (2 * s + lg);
      i32x8 b[4];
      int bsc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = wt + j * 32 + lrow;
        b[j] = cat8(Bs[swz(row, p_lo)], Bs[swz(row, p_hi)]);
        bsc[j] = (int)((csb[j] >> shift) & 0xffu);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wn + i * 32 + lrow;
        const i32x8 a = cat8(As[swz(row, p_lo)], As[swz(row, p_hi)]);
        const int asc = (int)((csa[i] >> shift) & 0xffu);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[j], acc[i][j], 0, 0, 0, asc, 0,
                                                                     bsc[j]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + wt + j * 32 + lrow;
    if (t >= T) continue;
    uint16_t* krow = kv + (int64_t)t * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn + i * 32 + 8 * g + 4 * lg;
        if (n + 4 <= N) {
          uint2 o;
          o.x = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
          o.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *reinterpret_cast<uint2*>(krow + n) = o;
        }
      }
  }
}

hipError_t set_lds(const void* fn) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
}

}  // namespace

hipError_t launch_gemm_bf16(const void* x, int64_t T, int K, const void* w, int N, void* kv,
                            hipStream_t s) {
  const int tiles_n = (N + BM - 1) / BM;
  const int tiles_t = (int)((T + BN - 1) / BN);
  const dim3 grid(tiles_n * tiles_t), block(THREADS);
  hipError_t e;
  if (K % 64 == 0) {
    if ((e = set_lds((const void*)gemm_bf16_kernel<false>)) != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_bf16_kernel<false>, grid, block, LDS_BYTES, s, (const uint16_t*)x, (int)T, K,
                       (const uint16_t*)w, N, (uint16_t*)kv, tiles_n, tiles_t);
  } else {
    if ((e = set_lds((const void*)gemm_bf16_kernel<true>)) != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_bf16_kernel<true>, grid, block, LDS_BYTES, s, (const uint16_t*)x, (int)T, K,
                       (const uint16_t*)w, N, (uint16_t*)kv, tiles_n, tiles_t);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_mxfp8(const uint8_t* xq, const uint8_t* xs, int64_t T, int K, const uint8_t* w,
                             const uint8_t* ws, int N, void* kv, hipStream_t s) {
  const int tiles_n = (N + BM - 1) / BM;
  const int tiles_t = (int)((T + BN - 1) / BN);
  hipError_t e = set_lds((const void*)gemm_mxfp8_kernel);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_mxfp8_kernel, dim3(tiles_n * tiles_t), dim3(THREADS), LDS_BYTES, s, xq, xs,
                     (int)T, K, w, ws, N, (uint16_t*)kv, tiles_n, tiles_t);
  return hipGetLastError();
}

}  // namespace engram
