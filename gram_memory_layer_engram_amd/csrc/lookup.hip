// Row gather: staged rows [T, C, head_dim] bf16 from the HBM-resident table.
//
// "vllm.models.deepseek_v4_1.common.engram", ParallelEngramEmbedding.lookup:
// ids [T, heads] -> [T, heads, head_dim] rows; the page launches a persistent
// grid near the compute-unit count because the table is far larger than the
// TLB reach. Here each thread moves 16-byte pieces of rows (head_dim*2/16
// pieces per row), keeps UNROLL independent pieces in flight (id load, then
// row load, then store), and strides over the whole [T*C*pieces] range.
//
// fp8 tables (same page, ParallelEngramEmbedding: rows stay fp8 and are
// dequantized with their ue8m0 per-32 scales on lookup): a thread takes an
// 8-element piece, 8 code bytes + its block's scale byte in, 16 bf16 bytes
// out.
#include "common.h"
#include "fp8_table.h"

namespace engram {

namespace {

constexpr int kLookupThreads = 256;
constexpr int kLookupUnroll = 4;

// Idx: the index type of the piece / row arithmetic, 32-bit unless the
// piece count needs 64 (64-bit division is a branchy routine, and a branch
// between the id loads makes the compiler wait for each one).
template <int CPR_T, typename Idx>  // 16-byte pieces per row; 0 = given at run time
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
    // every id load first, without a branch (a piece past the end reloads the
    // last piece's id): behind a bounds test the compiler waited for each id
    // before loading the next, one round trip per piece
    int32_t idv[kLookupUnroll];
#pragma unroll
    for (int u = 0; u < kLookupUnroll; ++u) {
      const Idx i = (Idx)min(base + u * stride, total - 1);
      const Idx row = i / (Idx)CPR;
      const Idx t = row / (Idx)n_cols;
      const int c = (int)(row - t * (Idx)n_cols);
      idv[u] = ids[(int64_t)t * st + (int64_t)c * sc];
    }
    int64_t src[kLookupUnroll];
#pragma unroll
    for (int u = 0; u < kLookupUnroll; ++u) {
      const int64_t i = base + u * stride;
      const int64_t row = i / CPR;
      const int piece = (int)(i - row * CPR);
      const int64_t id = idv[u];
      src[u] = -1;
      if (i < total) {
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
                      void* out, int32_t* err, hipStream_t s, int max_grid) {
  const int64_t total = T * n_cols * cpr;
  const int64_t need = (total + kLookupThreads * kLookupUnroll - 1) /
                       (kLookupThreads * kLookupUnroll);
  const int64_t cap = max_grid > 0 ? (int64_t)max_grid : (int64_t)dev_info().num_cus * 8;
  const int grid = (int)(need < cap ? need : cap);
  if (total <= (int64_t)UINT32_MAX)
    hipLaunchKernelGGL((lookup_kernel<CPR_T, uint32_t>), dim3(grid), dim3(kLookupThreads), 0, s,
                       (const uint4*)table, num_rows, ids, st, sc, n_cols, cpr,
                       total, (uint4*)out, err);
  else
    hipLaunchKernelGGL((lookup_kernel<CPR_T, uint64_t>), dim3(grid), dim3(kLookupThreads), 0, s,
                       (const uint4*)table, num_rows, ids, st, sc, n_cols, cpr,
                       total, (uint4*)out, err);
  return hipGetLastError();
}

// fp8 rows: grid-stride over 8-element pieces of the output rows (total =
// T*C*head_dim/8), as lookup_kernel over its 16-byte pieces: a lane reads 8
// code bytes and its block's scale byte and writes 16 bf16 bytes, so a wave's
// loads and stores are contiguous runs (a lane per 32-element block wrote
// 64-byte runs at a 64-byte lane stride, four partial lines per store).
template <typename Idx>   // as in lookup_kernel
__global__ __launch_bounds__(kLookupThreads) void lookup_fp8_kernel(
    const uint2* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t num_rows, int cpr,
    const int32_t* __restrict__ ids, int64_t st, int64_t sc, int n_cols, int64_t total,
    uint4* __restrict__ out, int32_t* __restrict__ err) {
  const int64_t stride = (int64_t)gridDim.x * kLookupThreads;
  int bad = 0;
  for (int64_t base = (int64_t)blockIdx.x * kLookupThreads + threadIdx.x; base < total;
       base += stride * kLookupUnroll) {
    int32_t idv[kLookupUnroll];   // the id loads first, together
#pragma unroll
    for (int u = 0; u < kLookupUnroll; ++u) {
      const Idx i = (Idx)min(base + u * stride, total - 1);
      const Idx row = i / (Idx)cpr;
      const Idx t = row / (Idx)n_cols;
      const int c = (int)(row - t * (Idx)n_cols);
      idv[u] = ids[(int64_t)t * st + (int64_t)c * sc];
    }
    int64_t src[kLookupUnroll];
#pragma unroll
    for (int u = 0; u < kLookupUnroll; ++u) {
      const int64_t i = base + u * stride;
      const int64_t row = i / cpr;
      const int piece = (int)(i - row * cpr);
      const int64_t id = idv[u];
      src[u] = -1;
      if (i < total) {
        if (id >= 0 && id < num_rows) src[u] = id * cpr + piece;   // 8-code piece of the table
        else bad = 1;
      }
    }
    uint2 cv[kLookupUnroll];
    uint32_t sb[kLookupUnroll];
#pragma unroll
    for (int u = 0; u < kLookupUnroll; ++u) {
      cv[u] = make_uint2(0, 0);
      sb[u] = 127u;                              // a bad id: zero codes, scale 1 -> zero piece
      if (src[u] >= 0) {
        cv[u] = codes[src[u]];
        sb[u] = scales[src[u] / 4];              // block id * head_dim/32 + piece/4 (cpr = 4 blocks' worth)
      }
    }
#pragma unroll
    for (int u = 0; u < kLookupUnroll; ++u) {
      const int64_t i = base + u * stride;
      if (i >= total) continue;
      const float s = e8m0_to_f32(sb[u]);
      uint32_t o[4];
      fp8_word_to_bf16(cv[u].x, s, o);
      fp8_word_to_bf16(cv[u].y, s, o + 2);
      out[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  if (bad && err) atomicOr(err, 1);
}

}  // namespace

hipError_t launch_lookup_fp8(const void* codes, const uint8_t* scales, int64_t num_rows, int head_dim,
                             const int32_t* ids, int64_t st, int64_t sc, int64_t T, int n_cols, void* out,
                             int32_t* err, hipStream_t s) {
  const int cpr = head_dim / 8;                  // 8-element pieces per row (head_dim % 32 == 0)
  const int64_t total = T * n_cols * cpr;
  const int64_t need = (total + kLookupThreads * kLookupUnroll - 1) / (kLookupThreads * kLookupUnroll);
  const int64_t cap = (int64_t)dev_info().num_cus * 8;
  const int grid = (int)(need < cap ? need : cap);
  if (total <= (int64_t)UINT32_MAX)
    hipLaunchKernelGGL(lookup_fp8_kernel<uint32_t>, dim3(grid), dim3(kLookupThreads), 0, s, (const uint2*)codes,
                       scales, num_rows, cpr, ids, st, sc, n_cols, total, (uint4*)out, err);
  else
    hipLaunchKernelGGL(lookup_fp8_kernel<uint64_t>, dim3(grid), dim3(kLookupThreads), 0, s, (const uint2*)codes,
                       scales, num_rows, cpr, ids, st, sc, n_cols, total, (uint4*)out, err);
  return hipGetLastError();
}

hipError_t launch_lookup(const void* table, int64_t num_rows, int head_dim,
                         const int32_t* ids, int64_t st, int64_t sc, int64_t T,
                         int n_cols, void* out, int32_t* err, hipStream_t s, int max_grid) {
  const int cpr = head_dim / 8;
  switch (cpr) {
    case 1: return launch_cpr<1>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s, max_grid);
    case 2: return launch_cpr<2>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s, max_grid);
    case 4: return launch_cpr<4>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s, max_grid);
    case 8: return launch_cpr<8>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s, max_grid);
    case 16: return launch_cpr<16>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s, max_grid);
    case 32: return launch_cpr<32>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s, max_grid);
    case 64: return launch_cpr<64>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s, max_grid);
    case 128: return launch_cpr<128>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s, max_grid);
    default: return launch_cpr<0>(table, num_rows, ids, st, sc, T, n_cols, cpr, out, err, s, max_grid);
  }
}

}  // namespace engram
