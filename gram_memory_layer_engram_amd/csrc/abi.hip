// C ABI of libengram: argument validation, workspace layout and dispatch.
// Every compute entry point only enqueues work on the caller's stream
// (engram_host_alloc / engram_host_free manage host memory and block).
#include "../../include/engram.h"
#include <algorithm>
#include <mutex>

#include "common.h"

#include <string.h>

namespace engram {

// Filled once per device under a lock, so calls from several host threads
// are safe; entries never change once filled.
const DevInfo& dev_info() {
  static DevInfo info[64];
  static bool ready[64] = {false};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!ready[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    info[dev].num_cus = cus;
    ready[dev] = true;
  }
  return info[dev];
}

}  // namespace engram

using namespace engram;

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? ENGRAM_OK : ENGRAM_EHIP; }

constexpr size_t kAlign = 256;
inline size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// MXFP8 activation staging inside a workspace: codes [T, K] then scales [T, K/32].
size_t mx_stage_bytes(int64_t T, int32_t K) {
  return round_up((size_t)T * K) + round_up((size_t)T * (K / 32));
}

int check_wkv(const void* x, int64_t T, int32_t K, const void* w,
              const uint8_t* w_scales, int32_t w_format, int32_t N, void* kv) {
  if (T < 0 || K <= 0 || N <= 0) return ENGRAM_EINVAL;
  if (T > 0 && (!x || !w || !kv)) return ENGRAM_EINVAL;
  if (T > 0 && (!aligned16(x) || !aligned16(w) || !aligned16(kv))) return ENGRAM_EINVAL;
  if (T > INT32_MAX || K > (1 << 20)) return ENGRAM_EUNSUPPORTED;  // 32-bit buffer offsets
  if (w_format == ENGRAM_W_BF16) {
    if (K % 8 != 0 || N % 4 != 0) return ENGRAM_EUNSUPPORTED;
  } else if (w_format == ENGRAM_W_MXFP8) {
    if (T > 0 && (!w_scales || ((uintptr_t)w_scales & 3u))) return ENGRAM_EINVAL;
    if (K % 128 != 0 || N % 32 != 0) return ENGRAM_EUNSUPPORTED;
  } else {
    return ENGRAM_EINVAL;
  }
  return ENGRAM_OK;
}

// MXFP8 projection from already-quantized activations: decode GEMV for small
// T (which stores kv; `ep` is for the tiled GEMM only), tiled scaled-MFMA
// GEMM otherwise.
hipError_t run_mx_projection(const uint8_t* xq, const uint8_t* xs, int64_t T, int32_t K,
                             const void* w, const uint8_t* w_scales, int32_t N, void* kv,
                             hipStream_t s, const GateEpi& ep) {
  return gemv_mxfp8_supported(T, K)
             ? launch_gemv_mxfp8(xq, xs, T, K, (const uint8_t*)w, w_scales, N, kv, s)
             : launch_gemm_mxfp8(xq, xs, T, K, (const uint8_t*)w, w_scales, N, kv, s, ep);
}

constexpr GateEpi kPlainStore{nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0};

// Enqueue the projection given a workspace already checked to be large enough.
int run_wkv(const void* x, int64_t T, int32_t K, const void* w,
            const uint8_t* w_scales, int32_t w_format, int32_t N, void* kv,
            void* workspace, hipStream_t s, const GateEpi& ep = kPlainStore) {
  if (T == 0) return ENGRAM_OK;
  if (w_format == ENGRAM_W_BF16)
    return hip_status(!ep.hidden && gemv_bf16_supported(T, K, N) ? launch_gemv_bf16(x, T, K, w, N, kv, s)
                                                                 : launch_gemm_bf16(x, T, K, w, N, kv, s, ep));
  uint8_t* xq = (uint8_t*)workspace;
  uint8_t* xs = xq + round_up((size_t)T * K);
  hipError_t e = launch_mx_quantize(x, T, K, xq, xs, s);
  if (e != hipSuccess) return ENGRAM_EHIP;
  return hip_status(run_mx_projection(xq, xs, T, K, w, w_scales, N, kv, s, ep));
}

// MXFP8 quantize + tiled scaled-MFMA GEMM whatever T is (the gate epilogue
// lives in the tiled GEMM only).
int run_wkv_tiled(const void* x, int64_t T, int32_t K, const void* w, const uint8_t* w_scales,
                  int32_t w_format, int32_t N, void* kv, void* workspace, hipStream_t s, const GateEpi& ep) {
  if (T == 0) return ENGRAM_OK;
  if (w_format == ENGRAM_W_BF16) return hip_status(launch_gemm_bf16(x, T, K, w, N, kv, s, ep));
  uint8_t* xq = (uint8_t*)workspace;
  uint8_t* xs = xq + round_up((size_t)T * K);
  if (launch_mx_quantize(x, T, K, xq, xs, s) != hipSuccess) return ENGRAM_EHIP;
  return hip_status(launch_gemm_mxfp8(xq, xs, T, K, (const uint8_t*)w, w_scales, N, kv, s, ep));
}

int check_gate(const void* hidden, const void* kv, const void* q, const void* k,
               int64_t T, int32_t hc, int32_t dim, void* out) {
  if (T < 0 || hc <= 0 || dim <= 0) return ENGRAM_EINVAL;
  if (hc > 8 || dim % 8 != 0 || dim > 16384) return ENGRAM_EUNSUPPORTED;
  if (T > INT32_MAX) return ENGRAM_EUNSUPPORTED;
  if (T > 0) {
    if (!hidden || !kv || !q || !k || !out) return ENGRAM_EINVAL;
    if (!aligned16(hidden) || !aligned16(kv) || !aligned16(q) || !aligned16(k) || !aligned16(out))
      return ENGRAM_EINVAL;
  }
  return ENGRAM_OK;
}

int check_lookup(const void* table, int64_t num_rows, int32_t head_dim,
                 const int32_t* ids, int64_t st, int64_t sc, int64_t T,
                 int32_t n_cols, void* rows_out) {
  if (T < 0 || n_cols <= 0 || head_dim <= 0 || num_rows < 0 || st < 0 || sc < 0)
    return ENGRAM_EINVAL;
  if (head_dim % 8 != 0 || head_dim > 1024) return ENGRAM_EUNSUPPORTED;
  if (T > 0) {
    if (!table || !ids || !rows_out) return ENGRAM_EINVAL;
    if (!aligned16(table) || !aligned16(rows_out) || ((uintptr_t)ids & 3u)) return ENGRAM_EINVAL;
  }
  return ENGRAM_OK;
}

int check_lookup_fp8(const void* codes, const uint8_t* scales, int64_t num_rows, int32_t head_dim,
                     const int32_t* ids, int64_t st, int64_t sc, int64_t T, int32_t n_cols, void* rows_out) {
  int st_ = check_lookup(codes, num_rows, head_dim, ids, st, sc, T, n_cols, rows_out);
  if (st_ != ENGRAM_OK) return st_;
  if (head_dim % 32 != 0) return ENGRAM_EUNSUPPORTED;
  if (T > 0 && !scales) return ENGRAM_EINVAL;
  return ENGRAM_OK;
}

}  // namespace

extern "C" {

int engram_abi_version(void) { return ENGRAM_ABI_VERSION; }

const char* engram_status_string(int status) {
  switch (status) {
    case ENGRAM_OK: return "ok";
    case ENGRAM_EINVAL: return "invalid argument";
    case ENGRAM_EUNSUPPORTED: return "unsupported shape";
    case ENGRAM_EHIP: return "HIP runtime error";
    case ENGRAM_ENOSPACE: return "input larger than the fixed scratch buffer";
    default: return "unknown status";
  }
}

int engram_lookup(const void* table, int64_t num_rows, int32_t head_dim,
                  const int32_t* hash_ids, int64_t ids_stride_t,
                  int64_t ids_stride_c, int64_t T, int32_t n_cols,
                  void* rows_out, int32_t* err_flag, void* stream) {
  int st = check_lookup(table, num_rows, head_dim, hash_ids, ids_stride_t,
                        ids_stride_c, T, n_cols, rows_out);
  if (st != ENGRAM_OK || T == 0) return st;
  return hip_status(launch_lookup(table, num_rows, head_dim, hash_ids, ids_stride_t,
                                  ids_stride_c, T, n_cols, rows_out, err_flag,
                                  (hipStream_t)stream));
}

int engram_lookup_background(const void* table, int64_t num_rows, int32_t head_dim,
                             const int32_t* hash_ids, int64_t ids_stride_t,
                             int64_t ids_stride_c, int64_t T, int32_t n_cols,
                             void* rows_out, int32_t* err_flag, void* stream) {
  int st = check_lookup(table, num_rows, head_dim, hash_ids, ids_stride_t,
                        ids_stride_c, T, n_cols, rows_out);
  if (st != ENGRAM_OK || T == 0) return st;
  // the persistent grid at half the compute units: one workgroup per two CUs
  const int cap = std::max(1, dev_info().num_cus / 2);
  return hip_status(launch_lookup(table, num_rows, head_dim, hash_ids, ids_stride_t,
                                  ids_stride_c, T, n_cols, rows_out, err_flag,
                                  (hipStream_t)stream, cap));
}

int engram_host_alloc(size_t bytes, void** host_ptr, void** device_ptr) {
  if (!host_ptr || !device_ptr || bytes == 0) return ENGRAM_EINVAL;
  *host_ptr = nullptr;
  *device_ptr = nullptr;
  void* h = nullptr;
  if (hipHostMalloc(&h, bytes, hipHostMallocMapped | hipHostMallocPortable) != hipSuccess || !h)
    return ENGRAM_EHIP;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess || !d) {
    (void)hipHostFree(h);
    return ENGRAM_EHIP;
  }
  *host_ptr = h;
  *device_ptr = d;
  return ENGRAM_OK;
}

int engram_host_free(void* host_ptr) {
  if (!host_ptr) return ENGRAM_OK;
  // kernels enqueued earlier may still read the memory: let the current
  // device drain before it goes back to the host
  if (hipDeviceSynchronize() != hipSuccess) return ENGRAM_EHIP;
  return hip_status(hipHostFree(host_ptr));
}

int engram_lookup_fp8(const void* table_codes, const uint8_t* table_scales, int64_t num_rows,
                      int32_t head_dim, const int32_t* hash_ids, int64_t ids_stride_t,
                      int64_t ids_stride_c, int64_t T, int32_t n_cols, void* rows_out,
                      int32_t* err_flag, void* stream) {
  int st = check_lookup_fp8(table_codes, table_scales, num_rows, head_dim, hash_ids, ids_stride_t,
                            ids_stride_c, T, n_cols, rows_out);
  if (st != ENGRAM_OK || T == 0) return st;
  return hip_status(launch_lookup_fp8(table_codes, table_scales, num_rows, head_dim, hash_ids,
                                      ids_stride_t, ids_stride_c, T, n_cols, rows_out, err_flag,
                                      (hipStream_t)stream));
}

int engram_mx_quantize(const void* x, int64_t T, int32_t K, uint8_t* xq,
                       uint8_t* xs, void* stream) {
  if (T < 0 || K <= 0) return ENGRAM_EINVAL;
  if (K % 32 != 0) return ENGRAM_EUNSUPPORTED;
  if (T == 0) return ENGRAM_OK;
  if (!x || !xq || !xs || !aligned16(x) || !aligned16(xq)) return ENGRAM_EINVAL;
  return hip_status(launch_mx_quantize(x, T, K, xq, xs, (hipStream_t)stream));
}

size_t engram_wkv_workspace_size(int64_t T, int32_t K, int32_t N,
                                 int32_t w_format) {
  (void)N;
  if (T <= 0 || K <= 0) return 0;
  return w_format == ENGRAM_W_MXFP8 ? mx_stage_bytes(T, K) : 0;
}

int engram_wkv_gate_partials(const void* x, int64_t T, int32_t K, const void* w,
                             const uint8_t* w_scales, int32_t w_format, int32_t hc,
                             int32_t dim, const void* hidden, const void* q_weight,
                             const void* k_weight, void* value, float* partials,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (hc <= 0 || dim <= 0) return ENGRAM_EINVAL;
  if (hc > 8 || dim % 256 != 0) return ENGRAM_EUNSUPPORTED;
  const int64_t N64 = (int64_t)(hc + 1) * dim;
  if (N64 > INT32_MAX) return ENGRAM_EUNSUPPORTED;
  const int32_t N = (int32_t)N64;
  int st = check_wkv(x, T, K, w, w_scales, w_format, N, value);
  if (st != ENGRAM_OK) return st;
  st = check_gate(hidden, value, q_weight, k_weight, T, hc, dim, value);
  if (st != ENGRAM_OK) return st;
  if (T == 0) return ENGRAM_OK;
  if (!partials || ((uintptr_t)partials & 7u)) return ENGRAM_EINVAL;
  const size_t need = engram_wkv_workspace_size(T, K, N, w_format);
  if (workspace_bytes < need || (need && (!workspace || ((uintptr_t)workspace % kAlign))))
    return ENGRAM_EINVAL;
  const GateEpi ep{(const uint16_t*)hidden, (const uint16_t*)q_weight, (const uint16_t*)k_weight,
                   (uint16_t*)value, (float2*)partials, hc, dim};
  return run_wkv_tiled(x, T, K, w, w_scales, w_format, N, value, workspace, (hipStream_t)stream, ep);
}

int engram_wkv(const void* x, int64_t T, int32_t K, const void* w,
               const uint8_t* w_scales, int32_t w_format, int32_t N, void* kv,
               void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_wkv(x, T, K, w, w_scales, w_format, N, kv);
  if (st != ENGRAM_OK || T == 0) return st;
  const size_t need = engram_wkv_workspace_size(T, K, N, w_format);
  if (workspace_bytes < need || (need && (!workspace || ((uintptr_t)workspace % kAlign))))
    return ENGRAM_EINVAL;
  return run_wkv(x, T, K, w, w_scales, w_format, N, kv, workspace, (hipStream_t)stream);
}

int engram_gate_finish(const void* hidden, const void* value, const float* partials,
                       const uint8_t* token_mask, int64_t T, int32_t hc, int32_t dim, float eps,
                       float clamp, void* out, float* gate_out, void* stream) {
  int st = check_gate(hidden, value, value, value, T, hc, dim, out);
  if (st != ENGRAM_OK) return st;
  if (dim % 256 != 0) return ENGRAM_EUNSUPPORTED;
  if (T == 0) return ENGRAM_OK;
  if (!partials || ((uintptr_t)partials & 7u)) return ENGRAM_EINVAL;
  return hip_status(launch_gate_parts(hidden, value, (const float2*)partials, token_mask, T, hc, dim, eps,
                                      clamp, out, gate_out, (hipStream_t)stream));
}

int engram_gate(const void* hidden, const void* kv, const void* q_weight,
                const void* k_weight, const uint8_t* token_mask, int64_t T,
                int32_t hc, int32_t dim, float eps, float clamp, void* out,
                float* gate_out, void* stream) {
  int st = check_gate(hidden, kv, q_weight, k_weight, T, hc, dim, out);
  if (st != ENGRAM_OK || T == 0) return st;
  return hip_status(launch_gate(hidden, kv, q_weight, k_weight, token_mask, T, hc,
                                dim, eps, clamp, out, gate_out, (hipStream_t)stream));
}

// Forward workspace: a 64 KiB flag area (used by engram_forward_single_launch;
// zero before the first call, left zero by every call), then staged rows
// [T, K] bf16 | kv [T, N] bf16 | MXFP8 staging, or the single-launch
// scratch, whichever is larger.
constexpr size_t kSyncBytes = kDecodeSyncBytes;

static bool use_decode_path(const engram_forward_args* a, int32_t K, int32_t N) {
  return a->w_format == ENGRAM_W_MXFP8 && decode_forward_supported(a->T, K, N, a->head_dim, a->dim, a->hc);
}

size_t engram_forward_workspace_size(const engram_forward_args* a) {
  if (!a || a->T <= 0 || a->n_cols <= 0 || a->head_dim <= 0 || a->hc <= 0 || a->dim <= 0)
    return 0;
  const int64_t K = (int64_t)a->n_cols * a->head_dim;
  const int64_t N = (int64_t)(a->hc + 1) * a->dim;
  size_t bytes = round_up((size_t)a->T * K * 2) + round_up((size_t)a->T * N * 2);
  if (a->w_format == ENGRAM_W_MXFP8) bytes += mx_stage_bytes(a->T, (int32_t)K);
  if (K <= INT32_MAX && N <= INT32_MAX && use_decode_path(a, (int32_t)K, (int32_t)N))
    bytes = std::max(bytes, decode_forward_scratch_bytes(a->T, (int)K, (int)N, a->dim));
  return kSyncBytes + bytes;
}

// Argument checks shared by the forward entry points, the workspace left
// out; sets K and N.
static int check_forward_args(const engram_forward_args* a, int32_t* K, int32_t* N) {
  if (!a || (a->options & ~ENGRAM_FORWARD_STORE_KV)) return ENGRAM_EINVAL;
  const int64_t K64 = (int64_t)a->n_cols * a->head_dim;
  const int64_t N64 = (int64_t)(a->hc + 1) * a->dim;
  if (K64 > INT32_MAX || N64 > INT32_MAX) return ENGRAM_EUNSUPPORTED;
  *K = (int32_t)K64;
  *N = (int32_t)N64;
  int st = a->table_scales
               ? check_lookup_fp8(a->table, a->table_scales, a->num_rows, a->head_dim, a->hash_ids,
                                  a->ids_stride_t, a->ids_stride_c, a->T, a->n_cols, (void*)16)
               : check_lookup(a->table, a->num_rows, a->head_dim, a->hash_ids, a->ids_stride_t,
                              a->ids_stride_c, a->T, a->n_cols, (void*)16);
  if (st != ENGRAM_OK) return st;
  st = check_gate(a->hidden, (void*)16, a->q_weight, a->k_weight, a->T, a->hc, a->dim, a->out);
  if (st != ENGRAM_OK) return st;
  return check_wkv((void*)16, a->T, *K, a->w, a->w_scales, a->w_format, *N, (void*)16);
}

// The forward entry points' checks, the caller's workspace included.
static int check_forward(const engram_forward_args* a, void* workspace, size_t workspace_bytes, int32_t* K,
                  int32_t* N) {
  int st = check_forward_args(a, K, N);
  if (st != ENGRAM_OK || a->T == 0) return st;
  const size_t need = engram_forward_workspace_size(a);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign)) return ENGRAM_EINVAL;
  return ENGRAM_OK;
}

// engram_forward's launches, given checked arguments and the workspace past
// its flag area (rows | kv | MXFP8 staging; nothing in it needs to start at
// zero: every byte a kernel reads was written earlier in the same call).
static int run_forward(const engram_forward_args* a, int32_t K, int32_t N, uint8_t* ws, hipStream_t s) {
  int st = ENGRAM_OK;
  void* rows = ws;
  void* kv = ws + round_up((size_t)a->T * K * 2);
  void* mx = (uint8_t*)kv + round_up((size_t)a->T * N * 2);
  // Unless ENGRAM_FORWARD_STORE_KV is set, when a tiled GEMM runs and a
  // 256-column tile lies inside one key block (dim % 256 == 0), its epilogue
  // turns key tiles into the gate's partial sums and stores only the value:
  // kv's keys never reach HBM. The value and partials take kv's place in the
  // workspace.
  const bool tiled = a->w_format == ENGRAM_W_BF16 ? !gemv_bf16_supported(a->T, K, N)
                                                 : !gemv_mxfp8_supported(a->T, K);
  const bool epi = !(a->options & ENGRAM_FORWARD_STORE_KV) && tiled && a->dim % 256 == 0;
  uint16_t* value = (uint16_t*)kv;
  float2* part = (float2*)((uint8_t*)kv + round_up((size_t)a->T * a->dim * 2));
  const GateEpi ep = epi ? GateEpi{(const uint16_t*)a->hidden, (const uint16_t*)a->q_weight,
                                   (const uint16_t*)a->k_weight, value, part, a->hc, a->dim}
                         : kPlainStore;
  hipError_t e;
  if (a->w_format == ENGRAM_W_MXFP8 && a->head_dim % 32 == 0) {
    // the gather feeds the quantizer directly: bf16 staged rows never reach HBM
    uint8_t* xq = (uint8_t*)mx;
    uint8_t* xs = xq + round_up((size_t)a->T * K);
    e = launch_gather_quantize(a->table, a->table_scales, a->num_rows, a->head_dim, a->hash_ids,
                               a->ids_stride_t, a->ids_stride_c, a->T, a->n_cols, xq, xs, a->err_flag, s);
    if (e != hipSuccess) return ENGRAM_EHIP;
    e = run_mx_projection(xq, xs, a->T, K, a->w, a->w_scales, N, kv, s, ep);
    if (e != hipSuccess) return ENGRAM_EHIP;
  } else {
    e = a->table_scales
            ? launch_lookup_fp8(a->table, a->table_scales, a->num_rows, a->head_dim, a->hash_ids,
                                a->ids_stride_t, a->ids_stride_c, a->T, a->n_cols, rows, a->err_flag, s)
            : launch_lookup(a->table, a->num_rows, a->head_dim, a->hash_ids, a->ids_stride_t,
                            a->ids_stride_c, a->T, a->n_cols, rows, a->err_flag, s);
    if (e != hipSuccess) return ENGRAM_EHIP;
    st = run_wkv(rows, a->T, K, a->w, a->w_scales, a->w_format, N, kv, mx, s, ep);
    if (st != ENGRAM_OK) return st;
  }
  e = epi ? launch_gate_parts(a->hidden, value, part, a->token_mask, a->T, a->hc, a->dim, a->eps,
                              a->clamp, a->out, a->gate_out, s)
          : launch_gate(a->hidden, kv, a->q_weight, a->k_weight, a->token_mask, a->T, a->hc,
                        a->dim, a->eps, a->clamp, a->out, a->gate_out, s);
  return hip_status(e);
}

int engram_forward(const engram_forward_args* a, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int32_t K = 0, N = 0;
  int st = check_forward(a, workspace, workspace_bytes, &K, &N);
  if (st != ENGRAM_OK || a->T == 0) return st;
  return run_forward(a, K, N, (uint8_t*)workspace + kSyncBytes, (hipStream_t)stream);
}

// ---- engram_forward_noalloc: engram_forward on a fixed device buffer ----
//
// `scratch` is a fixed buffer in device memory (one per GPU the library runs
// on, held until the process ends). Host code never passes its name to a
// kernel: on the host that name is only a stand-in, not a device address.
// The device address is looked up once per device, with that device
// current, and kept; launches take that pointer.

static __device__ __align__(256) uint8_t scratch[ENGRAM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on the first call on
// that device); ENGRAM_EHIP if the runtime cannot give its address.
static int scratch_of_current_device(uint8_t** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ENGRAM_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return ENGRAM_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return ENGRAM_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *p = (uint8_t*)g_scratch_ptr[dev];
  return ENGRAM_OK;
}

int engram_forward_noalloc(const engram_forward_args* a, void* stream) {
  int32_t K = 0, N = 0;
  int st = check_forward_args(a, &K, &N);
  if (st != ENGRAM_OK || a->T == 0) return st;
  // the workspace engram_forward would need, without its flag area (which
  // only engram_forward_single_launch uses)
  const size_t need = engram_forward_workspace_size(a) - kSyncBytes;
  if (need > (size_t)ENGRAM_NOALLOC_SCRATCH_BYTES) return ENGRAM_ENOSPACE;
  uint8_t* p = nullptr;
  st = scratch_of_current_device(&p);
  if (st != ENGRAM_OK) return st;
  return run_forward(a, K, N, p, (hipStream_t)stream);
}

int engram_forward_single_launch(const engram_forward_args* a, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  int32_t K = 0, N = 0;
  int st = check_forward(a, workspace, workspace_bytes, &K, &N);
  if (st != ENGRAM_OK || a->T == 0) return st;
  if (a->table_scales || !use_decode_path(a, K, N)) return ENGRAM_EUNSUPPORTED;
  uint8_t* ws = (uint8_t*)workspace + kSyncBytes;
  return hip_status(launch_decode_forward(a->table, a->num_rows, a->head_dim, a->hash_ids, a->ids_stride_t,
                                          a->ids_stride_c, a->n_cols, a->T, K, a->w, a->w_scales, N,
                                          a->hidden, a->q_weight, a->k_weight, a->token_mask, a->hc,
                                          a->dim, a->eps, a->clamp, a->out, a->gate_out, a->err_flag,
                                          (uint32_t*)workspace, ws, (hipStream_t)stream));
}

// ---- measurement probes ----

size_t engram_probe_out_bytes(void) {
  const int blocks = probe_mfma_blocks() > probe_mem_blocks() ? probe_mfma_blocks() : probe_mem_blocks();
  return (size_t)blocks * probe_threads() * 4;
}

int engram_probe_mfma(int32_t w_format, int32_t iters, float* out, double* flops, void* stream) {
  if (w_format != ENGRAM_W_BF16 && w_format != ENGRAM_W_MXFP8) return ENGRAM_EINVAL;
  if (iters <= 0 || !out || ((uintptr_t)out & 3u)) return ENGRAM_EINVAL;
  const bool fp8 = w_format == ENGRAM_W_MXFP8;
  if (flops)
    *flops = (double)probe_mfma_blocks() * (probe_threads() / 64) * probe_chains() * (double)iters *
             (fp8 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16);
  return hip_status(launch_probe_mfma(fp8, iters, out, (hipStream_t)stream));
}

int engram_probe_read(const void* src, size_t bytes, uint32_t* out, void* stream) {
  if (bytes % 16 != 0 || !out || ((uintptr_t)out & 3u)) return ENGRAM_EINVAL;
  if (bytes == 0) return ENGRAM_OK;
  if (!src || !aligned16(src)) return ENGRAM_EINVAL;
  return hip_status(launch_probe_read(src, (int64_t)(bytes / 16), out, (hipStream_t)stream));
}

int engram_probe_stream(const void* src, void* dst, size_t dst_bytes, int32_t reads_per_write,
                        void* stream) {
  if (dst_bytes % 16 != 0 || reads_per_write < 1 || reads_per_write > 4) return ENGRAM_EINVAL;
  if (dst_bytes == 0) return ENGRAM_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return ENGRAM_EINVAL;
  return hip_status(launch_probe_stream(src, dst, (int64_t)(dst_bytes / 16), reads_per_write,
                                        (hipStream_t)stream));
}

}  // extern "C"
