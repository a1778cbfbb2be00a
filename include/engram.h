/*
 * engram.h -- C ABI of libengram.so, the Engram layer's forward hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow the vLLM API pages:
 *   [P-common]  "vllm.models.deepseek_v4_1.common.engram"
 *   [P-rocm]    "vllm.models.deepseek_v41.amd.engram"
 *   [P-prefetch]"vllm.models.deepseek_v41.nvidia.specialized_decode.engram.prefetch"
 *   [P-gemv]    "vllm.models.deepseek_v41.amd.mono.attention.gemv"
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or keeps them; every call only enqueues kernels on
 *     `stream` (a hipStream_t passed as void*, NULL = the null stream) and
 *     returns without synchronising.
 *   - bf16 tensors are passed as raw 16-bit patterns (void*). Dense tensors
 *     are row-major and contiguous; their base addresses must be 16-byte
 *     aligned (ENGRAM_EINVAL otherwise).
 *   - T == 0 is a valid no-op (ENGRAM_OK, nothing launched), as on [P-common]
 *     where empty batches return before any launch.
 *   - Argument errors are reported synchronously through the return code.
 *     Data-dependent errors (out-of-range hash ids) are reported through an
 *     optional device-side flag the caller reads after synchronising.
 *   - Results are deterministic: no floating-point atomics; every reduction
 *     runs in a fixed order.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENGRAM_ABI_VERSION 5

/* Status codes. */
enum {
  ENGRAM_OK = 0,
  ENGRAM_EINVAL = 1,       /* NULL required pointer, bad size, misalignment */
  ENGRAM_EUNSUPPORTED = 2, /* a valid shape the library has no kernel for */
  ENGRAM_EHIP = 3,         /* a HIP runtime error at launch */
  ENGRAM_ENOSPACE = 4      /* engram_forward_noalloc: the call needs more than
                              ENGRAM_NOALLOC_SCRATCH_BYTES of scratch */
};

/* wkv weight formats. */
enum {
  ENGRAM_W_BF16 = 0,  /* W bf16 [N, K] row-major */
  ENGRAM_W_MXFP8 = 1  /* W e4m3fn codes [N, K] row-major + E8M0 bytes [N/32, K/32] */
};

/* Version of this ABI (ENGRAM_ABI_VERSION). */
int engram_abi_version(void);

/* Static text for a status code. */
const char* engram_status_string(int status);

/*
 * engram_lookup -- the row gather.
 *   [P-common] Engram.prepare_embeddings / ParallelEngramEmbedding.lookup:
 *   ids [T, heads] -> staged rows [T, heads, head_dim] bf16.
 *
 *   rows_out[t, c, :] = table[hash_ids[t * ids_stride_t + c * ids_stride_c], :]
 *
 *   table       bf16 [num_rows, head_dim], all per-column tables back to back
 *               (ids are GLOBAL rows: column offset already added).
 *   hash_ids    int32, element (t, c) at hash_ids[t*ids_stride_t + c*ids_stride_c]
 *               (strides in elements, >= 0; a layer's view of a [T, layers, C]
 *               hash tensor is strided).
 *   rows_out    bf16 [T, n_cols, head_dim] contiguous.
 *   head_dim    multiple of 8 (rows move in 16-byte pieces), <= 1024.
 *   err_flag    optional int32 device flag; an id outside [0, num_rows) yields
 *               a zero row and sets *err_flag = 1 (never cleared by the call).
 */
int engram_lookup(const void* table, int64_t num_rows, int32_t head_dim,
                  const int32_t* hash_ids, int64_t ids_stride_t,
                  int64_t ids_stride_c, int64_t T, int32_t n_cols,
                  void* rows_out, int32_t* err_flag, void* stream);

/*
 * engram_lookup_background -- engram_lookup for a side stream.
 *   [P-common] ParallelEngramEmbedding.lookup: with `background` set the
 *   persistent grid is halved so that the lookup leaves compute units to the
 *   kernels of the main stream; Engram.prepare_embeddings issues the layer's
 *   lookup ahead of its forward. Here the grid is capped at half the compute
 *   units (one workgroup of 256 threads per two CUs; engram_lookup runs up to
 *   8 per CU). Same arguments, results (bit for bit), error flag and errors
 *   as engram_lookup. Enqueue it on a stream other than the one whose work it
 *   should overlap (both at the default priority), and order the consumer
 *   after it with an event.
 */
int engram_lookup_background(const void* table, int64_t num_rows, int32_t head_dim,
                             const int32_t* hash_ids, int64_t ids_stride_t,
                             int64_t ids_stride_c, int64_t T, int32_t n_cols,
                             void* rows_out, int32_t* err_flag, void* stream);

/*
 * Host-resident tables.
 *   [P-common] ParallelEngramEmbedding (docstring: with cpu_offload the
 *   table shard lives in pinned host memory and is read over UVA;
 *   _storage). engram_host_alloc returns page-locked host memory mapped into
 *   the device's address space (hipHostMalloc, mapped and portable):
 *     *host_ptr    the address the CPU writes the table through;
 *     *device_ptr  the address kernels read it through: pass it as `table`
 *                  to engram_lookup, engram_lookup_background or
 *                  engram_forward, whose gathers then read the rows over the
 *                  host link (results bit for bit those of a device table).
 *   The memory is the caller's until engram_host_free(host_ptr); it is not
 *   a device allocation and is never touched by the library otherwise.
 *   engram_host_free first waits for all work on the current device to
 *   finish (hipDeviceSynchronize), so lookups still queued there cannot
 *   read freed memory; work on other devices that reads it must be
 *   finished by the caller. It is not allowed during stream capture.
 *   ENGRAM_EINVAL for bytes == 0 or NULL out-pointers, ENGRAM_EHIP when the
 *   runtime cannot allocate or map it (both out-pointers are then NULL).
 *   engram_host_free(NULL) is a no-op.
 */
int engram_host_alloc(size_t bytes, void** host_ptr, void** device_ptr);
int engram_host_free(void* host_ptr);

/*
 * engram_lookup_fp8 -- the row gather from an fp8 table, dequantized to bf16.
 *   [P-common] ParallelEngramEmbedding (docstring, __init__, lookup): the
 *   table is float8_e4m3fn [rows, dim] with one uint8 ue8m0 scale per row and
 *   32 elements (weight_scale_inv [rows, dim / 32]); rows stay fp8 and are
 *   dequantized on lookup:
 *     rows_out[t, c, j] = bf16_rne(e4m3(codes[id, j]) * 2^(scales[id, j/32] - 127))
 *   with id = hash_ids[t * ids_stride_t + c * ids_stride_c] (scale byte 255
 *   is NaN; products beyond the bf16 range become inf).
 *
 *   table_codes   uint8 e4m3fn codes [num_rows, head_dim], 16-byte aligned.
 *   table_scales  uint8 ue8m0 bytes [num_rows, head_dim / 32].
 *   Other arguments, the error flag and the errors as engram_lookup;
 *   head_dim must be a multiple of 32 (<= 1024), else ENGRAM_EUNSUPPORTED.
 */
int engram_lookup_fp8(const void* table_codes, const uint8_t* table_scales,
                      int64_t num_rows, int32_t head_dim,
                      const int32_t* hash_ids, int64_t ids_stride_t,
                      int64_t ids_stride_c, int64_t T, int32_t n_cols,
                      void* rows_out, int32_t* err_flag, void* stream);

/*
 * engram_mx_quantize -- MXFP8 quantization of bf16 activations.
 *   [P-prefetch] module docstring (the WKV chain quantizes its input to MXFP8)
 *   and [P-gemv] module docstring (tokens' MXFP8 rows). The rule (not on the
 *   pages) is the OCP MX v1.0 conversion: per token and 32-element K block,
 *   X = floor(log2(max|x|)) - 8, scale byte = clamp(X + 127, 0, 254) (0 for an
 *   all-zero block), code = e4m3fn(x / 2^(byte-127)) round-to-nearest-even,
 *   saturating at +-448, sign kept. A block holding an infinity or a NaN gets
 *   scale byte 255 (the E8M0 NaN) and every code 0x7F (the e4m3fn NaN), so
 *   it decodes to NaN.
 *
 *   x   bf16 [T, K];  xq  uint8 e4m3fn codes [T, K];  xs  uint8 E8M0 [T, K/32].
 *   K   multiple of 32.
 */
int engram_mx_quantize(const void* x, int64_t T, int32_t K, uint8_t* xq,
                       uint8_t* xs, void* stream);

/*
 * engram_wkv -- the wkv projection kv = bf16(x . W^T), fp32 accumulation,
 *   round-to-nearest-even to bf16.
 *   [P-common] Engram.__init__ / forward: bias-free linear from
 *   n_hash_cols*head_dim (K) to dim*(hc_mult+1) (N) on the flattened staged
 *   rows; output row [key_0 | ... | key_{hc-1} | value].
 *   [P-gemv] module docstring: the MXFP8 weight is row-major e4m3 [N, K] with
 *   E8M0 scales per 32x32 block [N/32, K/32].
 *
 *   x          bf16 [T, K] (the staged rows [T, C, head_dim] viewed flat).
 *   w          bf16 [N, K] (ENGRAM_W_BF16) or uint8 codes [N, K] (ENGRAM_W_MXFP8).
 *   w_scales   uint8 [N/32, K/32] for MXFP8, NULL for bf16.
 *   kv         bf16 [T, N].
 *   workspace  device scratch of at least engram_wkv_workspace_size() bytes
 *              (NULL allowed when that size is 0). For MXFP8 it holds x's
 *              MXFP8 codes and scales. 256-byte aligned.
 *   Shapes: bf16 needs K % 8 == 0 and N % 4 == 0; MXFP8 needs K % 128 == 0
 *   and N % 32 == 0; both need K <= 2^20 (32-bit buffer offsets). Other
 *   shapes return ENGRAM_EUNSUPPORTED.
 *   Kernels: a tiled GEMM; for T <= 64 a weight-streaming GEMV instead
 *   (MXFP8 with K/128 <= 32; bf16 with K % 32 == 0, K <= 2048, N % 16 == 0
 *   where it beats the GEMM). The two sum in different fp32 orders, so
 *   their kv can differ in the last bit.
 */
size_t engram_wkv_workspace_size(int64_t T, int32_t K, int32_t N,
                                 int32_t w_format);
int engram_wkv(const void* x, int64_t T, int32_t K, const void* w,
               const uint8_t* w_scales, int32_t w_format, int32_t N, void* kv,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * engram_wkv_gate_partials -- the projection fused with the gate's kv-side
 *   sums: [P-rocm] _engram_gate_partials_kernel / _engram_gate_finish_kernel
 *   split the gate into per-shard partial sums and a finish step; here a
 *   shard is a 256-column tile of the projection. kv = bf16(x . W^T) is
 *   computed by the tiled GEMM engram_wkv runs (bit for bit the same where
 *   engram_wkv runs that GEMM), but only the
 *   value block is stored; each key tile (copy h, columns 256i .. 256i+255)
 *   is reduced, per token t, against hidden, q and k:
 *     partials[2*((h*T + t)*(dim/256) + i)]     = sum hidden*q*k*key
 *     partials[2*((h*T + t)*(dim/256) + i) + 1] = sum key^2
 *   over the tile, on the bf16-rounded keys (fp32, fixed order). The keys
 *   never reach memory. engram_forward uses it where it applies and finishes
 *   the gate from the partials (engram_gate_finish).
 *
 *   x, T, K, w, w_scales, w_format: as engram_wkv, with N = (hc+1)*dim.
 *   hidden      bf16 [T, hc, dim];  q_weight, k_weight  bf16 [hc, dim]
 *   value       bf16 [T, dim] (kv's value block)
 *   partials    fp32 [hc, T, dim/256, 2], 8-byte aligned
 *   workspace   engram_wkv_workspace_size(T, K, (hc+1)*dim, w_format) bytes
 *   Errors: ENGRAM_EINVAL for hc or dim <= 0, a NULL or misaligned pointer,
 *   or a short workspace; T = 0 is a no-op. Asynchronous on `stream`.
 *   Shapes: as engram_wkv, plus dim % 256 == 0 and 1 <= hc <= 8; other
 *   shapes return ENGRAM_EUNSUPPORTED. This always runs the tiled GEMM
 *   (engram_wkv may take a GEMV for T <= 64).
 */
int engram_wkv_gate_partials(const void* x, int64_t T, int32_t K, const void* w,
                             const uint8_t* w_scales, int32_t w_format, int32_t hc,
                             int32_t dim, const void* hidden, const void* q_weight,
                             const void* k_weight, void* value, float* partials,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * engram_gate_finish -- the gate and residual update from per-tile partials.
 *   [P-rocm] _engram_gate_finish_kernel: the finish step of the partial /
 *   finish split, here with the partials of engram_wkv_gate_partials (one
 *   shard = one 256-column tile). For every token t and copy h:
 *     dot, ks = sums over the dim/256 tiles i of partials[h, t, i, 0] and
 *               partials[h, t, i, 1]
 *     hs  = sum hidden[t,h,:]^2
 *     g   = sigmoid(sign(d) * sqrt(max(|d|, clamp))),
 *           d = dot * rsqrt(hs/dim + eps) * rsqrt(ks/dim + eps) * rsqrt(dim)
 *     out[t,h,:] = bf16(hidden[t,h,:] + g * value[t,:])
 *   Tokens whose mask byte is 0 pass through: out = hidden bit for bit, g = 0.
 *
 *   hidden      bf16 [T, hc, dim];  value  bf16 [T, dim]
 *   partials    fp32 [hc, T, dim/256, 2] as engram_wkv_gate_partials writes
 *               them, 8-byte aligned
 *   token_mask, out, gate_out  as engram_gate. All sums in fp32 in a fixed
 *   order. Shapes: dim % 256 == 0, dim <= 16384, 1 <= hc <= 8; else
 *   ENGRAM_EUNSUPPORTED.
 */
int engram_gate_finish(const void* hidden, const void* value, const float* partials,
                       const uint8_t* token_mask, int64_t T, int32_t hc, int32_t dim,
                       float eps, float clamp, void* out, float* gate_out, void* stream);

/*
 * engram_gate -- gate and residual update.
 *   [P-rocm] _engram_gate_finish_kernel (single shard) and
 *   _engram_gate_partials_kernel; [P-common] Engram docstring and forward.
 *   For every token t and copy h < hc, over d < dim:
 *     hs  = sum hidden[t,h,d]^2
 *     ks  = sum key[t,h,d]^2                     key = kv[t, h*dim + d]
 *     dot = sum hidden*q[h,d]*k[h,d]*key
 *     g   = sigmoid(sign(dot) * sqrt(max(|dot'|, clamp)))
 *           dot' = dot * rsqrt(hs/dim + eps) * rsqrt(ks/dim + eps) * rsqrt(dim)
 *           (sign negative only when dot' < 0)
 *     out[t,h,d] = bf16(hidden[t,h,d] + g * value[t,d])   value = kv[t, hc*dim + d]
 *   Tokens whose mask byte is 0 pass through: out = hidden bit for bit, g = 0.
 *
 *   hidden      bf16 [T, hc, dim];  kv  bf16 [T, (hc+1)*dim]
 *   q_weight    bf16 [hc, dim];     k_weight  bf16 [hc, dim]
 *   token_mask  optional uint8 [T] (nonzero = active; NULL = all active)
 *   out         bf16 [T, hc, dim], must not overlap hidden or kv
 *   gate_out    optional fp32 [T, hc]
 *   Shapes: dim % 8 == 0, dim <= 16384, 1 <= hc <= 8.
 */
int engram_gate(const void* hidden, const void* kv, const void* q_weight,
                const void* k_weight, const uint8_t* token_mask, int64_t T,
                int32_t hc, int32_t dim, float eps, float clamp, void* out,
                float* gate_out, void* stream);

/*
 * engram_forward -- one Engram layer forward: lookup -> (MXFP8 quantize) ->
 *   wkv -> gate, all on `stream`.
 *   [P-common] Engram.forward: kv = wkv(embed(hash_ids).flatten(-2)), then the
 *   fused gate over [T, hc, dim]; the staged rows and kv live in the caller's
 *   workspace (the pages keep them as persistent buffers: Engram.staged_rows,
 *   EngramPrefetch's per-layer kv buffers).
 *   Field meanings are those of the calls above; K = n_cols*head_dim and
 *   N = (hc+1)*dim.
 *   workspace  engram_forward_workspace_size() bytes, 256-byte aligned; its
 *              first 64 KiB are the flag area of
 *              engram_forward_single_launch (zero before the first call of
 *              that entry point on the workspace; left zero by every call).
 *   err_flag   bit 0: an id outside [0, num_rows) (zero row used); bit 1:
 *              see engram_forward_single_launch. Never cleared by the call.
 */
typedef struct engram_forward_args {
  const void* table;       /* bf16 [num_rows, head_dim] */
  int64_t num_rows;
  const int32_t* hash_ids; /* int32, strided as in engram_lookup */
  int64_t ids_stride_t;
  int64_t ids_stride_c;
  const void* w;           /* wkv weight, see engram_wkv */
  const uint8_t* w_scales; /* MXFP8 only */
  int32_t w_format;
  const void* hidden;      /* bf16 [T, hc, dim] */
  const void* q_weight;    /* bf16 [hc, dim] */
  const void* k_weight;    /* bf16 [hc, dim] */
  const uint8_t* token_mask; /* optional uint8 [T] */
  int64_t T;
  int32_t hc;
  int32_t dim;
  int32_t n_cols;
  int32_t head_dim;
  float eps;
  float clamp;
  void* out;               /* bf16 [T, hc, dim] */
  float* gate_out;         /* optional fp32 [T, hc] */
  int32_t* err_flag;       /* optional int32 device flag, bits above */
  const uint8_t* table_scales; /* NULL: `table` is bf16. Else `table` holds
                                  e4m3 codes and these are its ue8m0 bytes
                                  [num_rows, head_dim / 32], as in
                                  engram_lookup_fp8 (head_dim % 32 == 0) */
  int32_t options;         /* 0, or ENGRAM_FORWARD_STORE_KV; other bits
                              give ENGRAM_EINVAL */
} engram_forward_args;

/*
 * Gate epilogue (the default) and ENGRAM_FORWARD_STORE_KV. Where the
 *   projection runs as a tiled GEMM (T too large for the GEMV of engram_wkv,
 *   or a shape it does not take) and dim % 256 == 0, engram_forward by default has
 *   the GEMM's epilogue reduce each 256-column key tile against hidden, q
 *   and k to the gate's per-tile sums (sum key^2, sum hidden*q*k*key over the
 *   bf16-rounded keys: the partial / finish split of [P-rocm]
 *   _engram_gate_partials_kernel / _engram_gate_finish_kernel at tile
 *   granularity, as engram_wkv_gate_partials computes) and stores only the
 *   value, so the keys never reach HBM; a small finish kernel then forms the
 *   gate and the update. ENGRAM_FORWARD_STORE_KV turns this off: kv is
 *   stored whole and the plain gate kernel reads it back (the composition of
 *   engram_wkv and engram_gate). Elsewhere the option has no effect. The two
 *   routes agree to the rounding of the gate's sums (the same bf16 keys
 *   summed in another order).
 */
#define ENGRAM_FORWARD_STORE_KV 1

size_t engram_forward_workspace_size(const engram_forward_args* a);
int engram_forward(const engram_forward_args* a, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * engram_forward_single_launch -- the same forward for decode batches as ONE
 *   kernel: gather, MXFP8 quantize, weight-streaming GEMV and the gate, the
 *   gate's kv-side sums taken as per-tile partials and finished in-launch,
 *   the split of [P-rocm] _engram_gate_partials_kernel /
 *   _engram_gate_finish_kernel (one shard). Same arguments, workspace size
 *   and results (to rounding of the gate's sums) as engram_forward.
 *   Supported: w_format ENGRAM_W_MXFP8, bf16 table (table_scales NULL),
 *   1 <= T <= 64, K % 1024 == 0, head_dim % 32 == 0, dim % 16 == 0,
 *   T*K <= 128 KiB; else ENGRAM_EUNSUPPORTED.
 *   Its workgroups coordinate through flags in the first 64 KiB of the
 *   workspace:
 *     - those bytes must be zero before the first call on a workspace
 *       (allocate it zeroed); every call returns them to zero;
 *     - calls sharing a workspace must be ordered on one stream;
 *     - flags found raised on entry, or a wait that timed out (the launch
 *       starved of compute units for 200 ms), set bit 1 (value 2) of
 *       *err_flag and the outputs are not valid; zero those 64 KiB again
 *       before the next call.
 *   On MI355X it is slower than engram_forward at the decode sizes measured
 *   (the hand-offs between workgroups cost more than the launch gaps they
 *   remove), so engram_forward does not use it.
 */
int engram_forward_single_launch(const engram_forward_args* a, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * engram_forward_noalloc -- engram_forward for callers that cannot allocate
 *   device memory (code under HIP graph capture, tight serving loops,
 *   harnesses that forbid hipMalloc): the same launches and results, bit for
 *   bit, as engram_forward with a caller workspace, but the scratch (staged
 *   rows, kv or value + gate partials, MXFP8 staging) lives in a fixed
 *   buffer of ENGRAM_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 *   held until the process ends. The call allocates and frees nothing.
 *
 *   Arguments, checks and errors as engram_forward, plus ENGRAM_ENOSPACE
 *   (nothing launched) when engram_forward_workspace_size(a) - 64 KiB
 *   exceeds ENGRAM_NOALLOC_SCRATCH_BYTES: at dim 4096 and K 2048 that is
 *   about 740 tokens; every decode batch (T <= 64) fits.
 *   Every call on one GPU uses that GPU's one buffer and leaves its last
 *   contents there (nothing in it has to start at zero). Calls that overlap
 *   on one GPU (different streams or threads without ordering between them)
 *   race on the buffer and give undefined results: order them on one stream.
 */
#define ENGRAM_NOALLOC_SCRATCH_BYTES (32u << 20)
int engram_forward_noalloc(const engram_forward_args* a, void* stream);

/*
 * Measurement probes. Not steps of the layer: they measure the rates this
 * chip sustains, so that each kernel's achieved rate can be quoted against a
 * measured ceiling as well as against the datasheet peak. Asynchronous on
 * `stream` like the rest; time them with events.
 *
 * engram_probe_out_bytes -- bytes of device memory `out` must hold for
 *   engram_probe_mfma and engram_probe_read (4-byte words: one per thread
 *   of the MFMA probe, 1024 per compute unit; depends on the device's
 *   compute-unit count).
 *
 * engram_probe_mfma -- a register-only loop of independent MFMA chains on
 *   every compute unit: v_mfma_f32_32x32x16_bf16 (ENGRAM_W_BF16, operands
 *   bf16 2^-8) or the scaled v_mfma_scale_f32_32x32x64_f8f6f4 (ENGRAM_W_MXFP8,
 *   e4m3 1.0 with E8M0 scale 2^0), `iters` steps of 8 MFMAs per wave. Each
 *   thread stores the sum of its 128 accumulators to out[thread]: exactly
 *   128 * iters * 2^-12 (bf16) or 128 * 64 * iters (MXFP8) while that is
 *   below 2^24. *flops (host, nullable) receives the flop count launched.
 *   ENGRAM_EINVAL for another format, iters <= 0, or a NULL / misaligned out.
 *
 * engram_probe_read -- streams `bytes` (a multiple of 16) from device memory
 *   `src` (16-byte aligned) in 16-byte pieces: one pass of workgroups that
 *   covers the buffer, each thread issuing its 4 loads before it uses any.
 *   Each wave XORs the words it read into one word of out (wave index
 *   modulo out's words) with an atomic XOR, so, with out zeroed first, the
 *   XOR of all of out's words is the XOR of the buffer.
 *
 * engram_probe_stream -- a streaming read/write at a fixed ratio: dst
 *   (dst_bytes, a multiple of 16) receives, per 16-byte piece d, the XOR of
 *   src pieces j*(dst_bytes/16) + d for j < reads_per_write (1..4; 1 is a
 *   copy), so src holds reads_per_write * dst_bytes; one pass of workgroups,
 *   each thread loading 2 pieces of every read stream before its stores.
 *   Both 16-byte aligned, not overlapping. ENGRAM_EINVAL otherwise;
 *   dst_bytes = 0 is a no-op.
 */
size_t engram_probe_out_bytes(void);
int engram_probe_mfma(int32_t w_format, int32_t iters, float* out, double* flops, void* stream);
int engram_probe_read(const void* src, size_t bytes, uint32_t* out, void* stream);
int engram_probe_stream(const void* src, void* dst, size_t dst_bytes, int32_t reads_per_write,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
