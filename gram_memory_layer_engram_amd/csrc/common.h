// Shared device helpers and launcher declarations of libengram (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace engram {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// bf16 halves of a packed 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The same rounding in one instruction (v_cvt_pk_bf16_f32: round to nearest,
// ties to even; identical to pack_bf16x2 for every non-NaN input, a NaN
// becomes the hardware's quiet NaN). Used where the conversion is on the
// critical path: the GEMM epilogue (a whole tile between the last MFMA and
// the stores) and the gate's output rows.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Device properties the launchers need (cached per device by the ABI layer).
struct DevInfo {
  int num_cus;
};

const DevInfo& dev_info();

// ---- launchers (each validates nothing: the ABI layer has done that) ----
// max_grid > 0 caps the persistent grid at that many workgroups (the
// background lookup: half the compute units); 0 = 8 per compute unit.
hipError_t launch_lookup(const void* table, int64_t num_rows, int head_dim,
                         const int32_t* ids, int64_t st, int64_t sc, int64_t T,
                         int n_cols, void* out, int32_t* err, hipStream_t s, int max_grid = 0);

hipError_t launch_gate(const void* hidden, const void* kv, const void* q,
                       const void* k, const uint8_t* mask, int64_t T, int hc,
                       int dim, float eps, float clamp, void* out,
                       float* gate_out, hipStream_t s);

// The gate from the prefill GEMM's epilogue: partials [hc, T, dim/256] and
// value [T, dim] in place of kv.
hipError_t launch_gate_parts(const void* hidden, const void* value, const float2* part,
                             const uint8_t* mask, int64_t T, int hc, int dim, float eps,
                             float clamp, void* out, float* gate_out, hipStream_t s);

hipError_t launch_mx_quantize(const void* x, int64_t T, int K, uint8_t* xq,
                              uint8_t* xs, hipStream_t s);

// Row gather fused with the MXFP8 quantizer (head_dim % 32 == 0); an fp8
// table when table_scales is not null.
hipError_t launch_gather_quantize(const void* table, const uint8_t* table_scales, int64_t num_rows,
                                  int head_dim, const int32_t* ids, int64_t st, int64_t sc, int64_t T,
                                  int n_cols, uint8_t* xq, uint8_t* xs, int32_t* err, hipStream_t s);

// Row gather from an fp8 table (e4m3 codes [rows, head_dim], ue8m0 bytes
// [rows, head_dim / 32]) into bf16 rows; head_dim % 32 == 0.
hipError_t launch_lookup_fp8(const void* codes, const uint8_t* scales, int64_t num_rows, int head_dim,
                             const int32_t* ids, int64_t st, int64_t sc, int64_t T, int n_cols, void* out,
                             int32_t* err, hipStream_t s);

// Optional epilogue of the prefill GEMMs: with hidden != nullptr the key
// tiles become the gate's per-(copy, token) partial sums over each 256-column
// tile and only the value columns are stored (dim % 256 == 0).
struct GateEpi {
  const uint16_t* hidden;   // [T, hc, dim]; nullptr: store kv [T, N]
  const uint16_t* q;        // [hc, dim]
  const uint16_t* k;        // [hc, dim]
  uint16_t* value;          // [T, dim]
  float2* part;             // [hc, T, dim/256]: (sum hidden*q*k*key, sum key^2)
  int hc, dim;
};

hipError_t launch_gemm_bf16(const void* x, int64_t T, int K, const void* w,
                            int N, void* kv, hipStream_t s, const GateEpi& ep);

hipError_t launch_gemm_mxfp8(const uint8_t* xq, const uint8_t* xs, int64_t T,
                             int K, const uint8_t* w, const uint8_t* ws, int N,
                             void* kv, hipStream_t s, const GateEpi& ep);

hipError_t launch_gemv_mxfp8(const uint8_t* xq, const uint8_t* xs, int64_t T,
                             int K, const uint8_t* w, const uint8_t* ws, int N,
                             void* kv, hipStream_t s);

// Largest T the decode GEMV serves; above it the tiled GEMM runs.
constexpr int kGemvMaxT = 64;

// Small-batch projection with bf16 weights (T <= kGemvMaxT): whether the
// weight-streaming GEMV takes (T, K, N), and its launch (plain kv store).
bool gemv_bf16_supported(int64_t T, int K, int N);
hipError_t launch_gemv_bf16(const void* x, int64_t T, int K, const void* w, int N, void* kv, hipStream_t s);

// Whether the decode GEMV takes (T, K): T <= kGemvMaxT and K small enough for
// its per-wave register budget.
bool gemv_mxfp8_supported(int64_t T, int K);

// Single-launch decode forward (MXFP8 wkv, T <= kGemvMaxT): shape support,
// scratch it needs besides the counter area (kDecodeSyncBytes at the front of
// the forward workspace: one counter and up to kDecodeMaxFlags per-workgroup
// flags), and the launcher.
constexpr size_t kDecodeSyncBytes = 64 * 1024;
constexpr int kDecodeMaxFlags = (int)(kDecodeSyncBytes / 4) - 64;
bool decode_forward_supported(int64_t T, int K, int N, int head_dim, int dim, int hc);
size_t decode_forward_scratch_bytes(int64_t T, int K, int N, int dim);
hipError_t launch_decode_forward(const void* table, int64_t num_rows, int head_dim, const int32_t* ids,
                                 int64_t st, int64_t sc, int n_cols, int64_t T, int K, const void* w,
                                 const uint8_t* w_scales, int N, const void* hidden, const void* q,
                                 const void* k, const uint8_t* mask, int hc, int dim, float eps,
                                 float clamp, void* out, float* gate_out, int32_t* err, uint32_t* sync,
                                 uint8_t* scratch, hipStream_t s);

// Measurement probes (not steps of the layer): grid sizes and launchers.
int probe_mfma_blocks();
int probe_mem_blocks();
int probe_threads();
int probe_chains();
hipError_t launch_probe_mfma(bool fp8, int iters, float* out, hipStream_t s);
hipError_t launch_probe_read(const void* src, int64_t n16, uint32_t* out, hipStream_t s);
hipError_t launch_probe_stream(const void* src, void* dst, int64_t n16, int ratio, hipStream_t s);


}  // namespace engram
