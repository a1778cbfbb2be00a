// Row gather: staged rows [T, C, head_dim] bf16 from the HBM-resident table.
//
// "vllm.models.deepseek_v4_1.common.engram", ParallelEngramEmbedding.lookup:
// ids [T, heads] -> [T, heads, head_dim] rows; the page launches a persistent
// grid near the compute-unit count because the table is far larger than the
// TLB reach. Here each thread moves 16-byte pieces of rows (head_dim*2/16
// pieces per row), keeps UNROLL independent pieces in flight (id load, then
// row load, then store), and strides over the whole [T*C*pieces] range.
#include "common.h"

namespace engram {

namespace {

constexpr int kLookupThreads = 256;
constexpr int kLookupUnroll = 4;

template <int CPR_T>  // 16-byte pieces per row; 0 = given at run time
__global__ __launch_bounds__(kLookupThreads) void lookup_kernel(
    const uint4* __restrict__ table, int64_t num_rows,
    const int32_t* __restrict__ ids, int64_t st, int64_t sc, int n_cols,
    int cpr_rt, int64_t total, uint4* __restrict__ out,
    int32_t* __restrict__ err) {
  const int CPR = CPR_T ? CPR_T : cpr_rt;
  const int64_t stride = (int64_t)gridDim.x * kLookupThreads;
  int bad = 0;
  for (int64_t base = (int64_t)blockIdx.x * kLookupThreads + threadIdx.x;
       base < total; base += stride * kLookupUnroll) {
    int64_t src[kLookupUnroll];
#pragma unroll
    for (int u = 0; u < kLookupUnroll; ++u) {
      const int64_t i = base + u * stride;
      src[u] = -1;
      if (i < total) {
        const int64_t row = i / CPR;
        const int piece = (int)(i - row * CPR);
        const int64_t t = row / n_cols;
        const int c = (int)(row - t * n_cols);
        const int64_t id = ids[t * st + (int64_t)c * sc];
        if (id >= 0 && id < num_rows) src[u] = id * CPR + piece;
        else bad = 1;
      }
    }
    uint4 v[kLookupUnroll];
#pragma unroll
    for (int u = 0; u < kLookupUnroll; ++u)
      v[u] = src[u] >= 0 ? table[src[u]] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kLookupUnroll; ++u) {
      const int64_t i = base + u * stride;
      if (i < total) out[i] = v[u];
    }
  }
  if (bad && err) atomicOr(err, 1);
}

template <int CPR_T>
hipError_t launch_cpr(const void* table, int64_t num_rows, const int32_t* ids,
                      int64_t st, int64_t sc, int64_t T, int n_cols, int cpr,
                      void* out, int32_t* err, hipStream_t s) {
  const int64_t total = T * n_cols * cpr;
  const int64_t need = (total + kLookupThreads * kLookupUnroll - 1) /
                       (kLookupThreads * kLookupUnroll);
  const int64_t cap = (int64_t)dev_info().num_cus * 8;
  const int grid = (int)(need < cap ? need : cap);
  hipLaunchKernelGGL(lookup_kernel<CPR_T>, dim3(grid), dim3(kLookupThreads), 0, s,
                     (const uint4*)table, num_rows, ids, st, sc, n_cols, cpr,
                     total, (uint4*)out, err);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lookup(const void* table, int64_t num_rows, int head_dim,
                         const int32_t* ids, int64_t st, int64_t sc, int64_t T,
                         int n_cols, void* out, int32_t* err, hipStream_t s) {
  const int cpr = head_dim / 8;
  switch (cpr) {
    case 1: return launch_cpr<1>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s);
    case 2: return launch_cpr<2>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s);
    case 4: return launch_cpr<4>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s);
    case 8: return launch_cpr<8>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s);
    case 16: return launch_cpr<16>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s);
    case 32: return launch_cpr<32>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s);
    case 64: return launch_cpr<64>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s);
    case 128: return launch_cpr<128>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s);
    default: return launch_cpr<0>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s);
  }
}

}  // namespace engram
