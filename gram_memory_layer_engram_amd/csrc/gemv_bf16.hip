// wkv projection for small batches with bf16 weights: kv[T, N] = bf16(x[T, K] . W[N, K]^T)
// for T <= 64, fp32 accumulation.
//
// "vllm.models.deepseek_v4_1.common.engram", Engram.__init__ / forward: wkv
// is a bias-free linear from n_hash_cols*head_dim (K) to dim*(hc_mult+1) (N)
// on the flattened staged rows; with few tokens it is a stream of the weight
// (the decode shape "vllm.models.deepseek_v41.amd.mono.attention.gemv" is
// written for: weight loads in flight before the activations, split over k).
//
// The tiled GEMM spends ~10 us of fixed cost per round of 256x256 tiles,
// which at T <= 64 is all of its time; here the weight streams through
// registers instead. Layout as in the MXFP8 decode GEMV: a workgroup of 8
// waves owns RT tiles of 16 W rows and all T tokens (NT tiles of 16); wave w
// takes the k steps [w*SPW, (w+1)*SPW) of every row tile (a step is 32
// elements, one v_mfma_f32_16x16x32_bf16), issues all of its weight loads,
// then its activation loads, then the MFMAs; the 8 partial 16x16 tiles of
// each (row tile, token tile) are summed through LDS in wave order.
//
// Operand layout of v_mfma_f32_16x16x32_bf16: lane l holds row l%16 of A
// (a W row) and column l%16 of B (a token), each with k elements
// 8*(l/16) .. 8*(l/16)+7 of the step; C lane l holds rows 4*(l/16)+i,
// column l%16.
#include "common.h"

namespace engram {

namespace {

constexpr int GB_WAVES = 8;
constexpr int GB_THREADS = GB_WAVES * 64;

template <int RT, int NT, int SPW>
__global__ __launch_bounds__(GB_THREADS) void gemv_bf16_kernel(
    const uint16_t* __restrict__ x, int T, int K, const uint16_t* __restrict__ w, int N,
    uint16_t* __restrict__ kv) {
  __shared__ f32x4 red[GB_WAVES][RT * NT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16 * RT;
  const int g = lane >> 4, r = lane & 15;
  const int nsteps = K / 32;
  const int step0 = wave * SPW;

  // Every load is issued before the first MFMA, weights first; each sits
  // behind its own uniform bounds test, which also keeps the compiler from
  // moving it next to its use. A padding token reloads token 0 (its MFMA
  // column only feeds outputs that are not stored).
  uint4 wv[RT][SPW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const uint16_t* wrow = w + (int64_t)(n0 + rt * 16 + r) * K + 8 * g;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      wv[rt][s] = make_uint4(0, 0, 0, 0);
      if (step0 + s < nsteps) wv[rt][s] = *reinterpret_cast<const uint4*>(wrow + (step0 + s) * 32);
    }
  }
  uint4 xv[NT][SPW];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = j * 16 + r < T ? j * 16 + r : 0;
    const uint16_t* xrow = x + (int64_t)t * K + 8 * g;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      xv[j][s] = make_uint4(0, 0, 0, 0);
      if (step0 + s < nsteps) xv[j][s] = *reinterpret_cast<const uint4*>(xrow + (step0 + s) * 32);
    }
  }

  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    if (step0 + s >= nsteps) break;  // uniform per wave
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const bf16x8_t xb = __builtin_bit_cast(bf16x8_t, xv[j][s]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv[rt][s]), xb,
                                                             acc[rt][j], 0, 0, 0);
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[wave][rt * NT + j][lane] = acc[rt][j];
  __syncthreads();
  // thread (tile pair, lane) sums the waves' partials in wave order
  for (int idx = tid; idx < RT * NT * 64; idx += GB_THREADS) {
    const int pair = idx >> 6, l = idx & 63;
    const int rt = pair / NT, j = pair - rt * NT;
    f32x4 sum = red[0][pair][l];
#pragma unroll
    for (int v = 1; v < GB_WAVES; ++v) {
      const f32x4 p = red[v][pair][l];
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

// Registers a lane holds in flight: weights, activations, accumulators
// (8 waves per workgroup: 256 registers per lane at most).
constexpr int gb_regs(int rt, int nt, int spw) { return 4 * spw * (rt + nt) + 4 * rt * nt; }
constexpr int kGbRegBudget = 224;

// Steps per wave, rounded up to the instantiated 1, 2, 4, 8 (0: K too large).
int gb_spw(int K) {
  const int spw = (K / 32 + GB_WAVES - 1) / GB_WAVES;
  return spw <= 1 ? 1 : spw <= 2 ? 2 : spw <= 4 ? 4 : spw <= 8 ? 8 : 0;
}

template <int RT, int NT>
hipError_t gemv_bf16_rt(const void* x, int T, int K, const void* w, int N, void* kv, hipStream_t s) {
  const int spw = gb_spw(K);
  const dim3 grid(N / (16 * RT)), block(GB_THREADS);
  switch (spw) {
#define GB_CASE(S)                                                                                    \
  case S:                                                                                             \
    if constexpr (gb_regs(RT, NT, S) <= kGbRegBudget) {                                               \
      hipLaunchKernelGGL((gemv_bf16_kernel<RT, NT, S>), grid, block, 0, s, (const uint16_t*)x, T, K,  \
                         (const uint16_t*)w, N, (uint16_t*)kv);                                       \
      return hipGetLastError();                                                                       \
    }                                                                                                 \
    return hipErrorInvalidValue;
    GB_CASE(1) GB_CASE(2) GB_CASE(4) GB_CASE(8)
#undef GB_CASE
    default: return hipErrorInvalidValue;
  }
}

// The largest row-tile count of 5, 4, 2, 1 that divides N/16 and keeps the
// lane's registers in budget.
template <int NT>
int gb_rt(int N, int spw) {
  const int tiles = N / 16;
  for (int rt : {5, 4, 2, 1})
    if (tiles % rt == 0 && gb_regs(rt, NT, spw) <= kGbRegBudget) return rt;
  return 0;
}

int gb_rt_for(int nt, int N, int spw) {
  switch (nt) {
    case 1: return gb_rt<1>(N, spw);
    case 2: return gb_rt<2>(N, spw);
    case 3: return gb_rt<3>(N, spw);
    case 4: return gb_rt<4>(N, spw);
    default: return 0;
  }
}

template <int NT>
hipError_t gemv_bf16_nt(const void* x, int T, int K, const void* w, int N, void* kv, hipStream_t s) {
  switch (gb_rt<NT>(N, gb_spw(K))) {
    case 5: return gemv_bf16_rt<5, NT>(x, T, K, w, N, kv, s);
    case 4: return gemv_bf16_rt<4, NT>(x, T, K, w, N, kv, s);
    case 2: return gemv_bf16_rt<2, NT>(x, T, K, w, N, kv, s);
    case 1: return gemv_bf16_rt<1, NT>(x, T, K, w, N, kv, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Taken where it beats the tiled GEMM: the register budget leaves enough
// rows per workgroup for at most two workgroups per compute unit (measured
// at K 2048, N 20480: T 1 / 16 / 32 in 20 / 25 / 34 us against the GEMM's
// 40-41 us; T 64, 640 workgroups of 32 rows, 46 against 42 us).
bool gemv_bf16_supported(int64_t T, int K, int N) {
  if (T < 1 || T > kGemvMaxT || K % 32 != 0 || N % 16 != 0) return false;
  const int spw = gb_spw(K);
  if (spw == 0) return false;
  const int rt = gb_rt_for((int)((T + 15) / 16), N, spw);
  return rt != 0 && N / (16 * rt) <= 2 * dev_info().num_cus;
}

hipError_t launch_gemv_bf16(const void* x, int64_t T, int K, const void* w, int N, void* kv, hipStream_t s) {
  switch ((T + 15) / 16) {
    case 1: return gemv_bf16_nt<1>(x, (int)T, K, w, N, kv, s);
    case 2: return gemv_bf16_nt<2>(x, (int)T, K, w, N, kv, s);
    case 3: return gemv_bf16_nt<3>(x, (int)T, K, w, N, kv, s);
    case 4: return gemv_bf16_nt<4>(x, (int)T, K, w, N, kv, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace engram
