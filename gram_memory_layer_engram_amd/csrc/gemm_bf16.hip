// wkv projection, bf16 weights: kv[T, N] = bf16(x[T, K] . W[N, K]^T).
//
// "vllm.models.deepseek_v4_1.common.engram", Engram.__init__ / forward: wkv
// is a bias-free linear from n_hash_cols*head_dim to dim*(hc_mult+1) applied
// to the flattened staged rows; its output row is [key_0 | ... | value].
//
// MI355X design
//  * Both operands are K-contiguous (x rows are staged rows, W is the
//    out x in linear weight), so each 256x64 operand tile is 256 rows of
//    128 bytes: 8 pieces of 16 B per row, loaded fully coalesced.
//  * The MFMA is v_mfma_f32_32x32x16_bf16 with A = W rows (n) and B = x rows
//    (tokens): an accumulator lane then holds 4 consecutive n of one token,
//    stored as one 8-byte bf16x4 write.
//  * Block tile 256 (n) x 256 (tokens) x 64 (k), four waves in a 2x2 grid,
//    each wave 128x128 = 4x4 MFMA tiles (256 fp32 accumulators per lane,
//    held in AGPRs). LDS holds two stages of both tiles (2 x 64 KiB).
//  * LDS rows are 128 B; piece p of row r lives at p ^ ((r >> 1) & 7) so the
//    16 rows one ds_read_b128 phase touches cover all 64 banks.
//  * Tile order is XCD-aware: consecutive workgroup ids land on different
//    XCDs, so ids are first regrouped per XCD, then walked in groups of 4
//    token tiles so that each XCD's 32 resident workgroups share 4 x-tiles
//    and 8 W-tiles in that XCD's L2.
#include "common.h"

namespace engram {

namespace {

constexpr int BM = 256;  // W rows (n) per block
constexpr int BN = 256;  // tokens per block
constexpr int BK = 64;   // k per stage (128 B of bf16 per row)
constexpr int THREADS = 256;
constexpr int PIECES = BK / 8;          // 16-byte pieces per tile row
constexpr int TILE_BYTES = BM * BK * 2; // 32 KiB per operand tile
constexpr int LOADS = BM * PIECES / THREADS;  // 8 pieces per thread per operand
constexpr int GROUP_T = 4;

__device__ __forceinline__ int swz(int row, int piece) {
  return row * PIECES + (piece ^ ((row >> 1) & 7));
}

// Map the linear workgroup id to (n tile, token tile), XCD-aware.
__device__ __forceinline__ void tile_of(int bid, int tiles_n, int tiles_t,
                                        int& tn, int& tt) {
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

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint4* __restrict__ x, int T, int K,
                      const uint4* __restrict__ w, int N,
                      uint16_t* __restrict__ kv, int tiles_n, int tiles_t) {
  extern __shared__ uint4 smem[];
  uint4* As = smem;                         // [2][BM*PIECES]
  uint4* Bs = smem + 2 * BM * PIECES;       // [2][BN*PIECES]

  int tn, tt;
  tile_of(blockIdx.x, tiles_n, tiles_t, tn, tt);
  const int n0 = tn * BM, t0 = tt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = (wave >> 1) * 128, wt = (wave & 1) * 128;
  const int kp = K / 8;  // 16-byte pieces per global row

  // global -> register staging
  uint4 ra[LOADS], rb[LOADS];
  auto gload = [&](int k0) {
    const int kpc = k0 / 8;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = tid + i * THREADS;
      const int row = q / PIECES, piece = q % PIECES;
      const int gp = kpc + piece;
      const int n = n0 + row, t = t0 + row;
      ra[i] = (n < N && gp < kp) ? w[(int64_t)n * kp + gp] : make_uint4(0, 0, 0, 0);
      rb[i] = (t < T && gp < kp) ? x[(int64_t)t * kp + gp] : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int stage) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = tid + i * THREADS;
      const int row = q / PIECES, piece = q % PIECES;
      As[stage * BM * PIECES + swz(row, piece)] = ra[i];
      Bs[stage * BN * PIECES + swz(row, piece)] = rb[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();

  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const uint4* Ast = As + stage * BM * PIECES;
    const uint4* Bst = Bs + stage * BN * PIECES;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int piece = kk * 2 + lhalf;
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = Ast[swz(wn + i * 32 + lrow, piece)];
        a[i] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 v = Bst[swz(wt + j * 32 + lrow, piece)];
        b[j] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: accumulator r of lane l is D[n][t] with
  //   n = 8*(r/4) + 4*(l/32) + r%4, t = l%32 inside each 32x32 tile.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + wt + j * 32 + lrow;
    if (t >= T) continue;
    uint16_t* krow = kv + (int64_t)t * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
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
}

}  // namespace

hipError_t launch_gemm_bf16(const void* x, int64_t T, int K, const void* w,
                            int N, void* kv, hipStream_t s) {
  const int tiles_n = (N + BM - 1) / BM;
  const int tiles_t = (int)((T + BN - 1) / BN);
  const size_t lds = 2 * (size_t)TILE_BYTES * 2;
  hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3(tiles_n * tiles_t), dim3(THREADS),
                     lds, s, (const uint4*)x, (int)T, K, (const uint4*)w, N,
                     (uint16_t*)kv, tiles_n, tiles_t);
  return hipGetLastError();
}

}  // namespace engram
