// Single-launch decode forward (T <= 64, MXFP8 wkv): row gather + MXFP8
// quantize + weight-streaming GEMV + gate in one kernel.
//
// What is computed is the Engram forward ("vllm.models.deepseek_v4_1.common.
// engram", Engram.forward): x = flatten(table[hash_ids]), kv = wkv(x) in the
// MXFP8 format of "vllm.models.deepseek_v41.amd.mono.attention.gemv" (module
// docstring), then the gate of "vllm.models.deepseek_v41.amd.engram" split
// the way its _engram_gate_partials_kernel / _engram_gate_finish_kernel pair
// splits it: the kv-side sums (sum key^2 and sum hidden*q*k*key) are
// partials over column tiles, finished after all tiles are in.
//
// Why one launch: at decode the weight stream (42 MB at dim 4096) is the
// only real traffic; with separate gather, GEMV and gate kernels the fixed
// costs (launch, first-byte latency, the gather's dependent loads, the gate's
// reductions) add up to more than the stream itself.
//
// Each workgroup (8 wavefronts) owns rows [16*RT*b, 16*RT*(b+1)) of W and
// all T tokens:
//  1. every thread loads the hash ids of its share of x's 32-element MX
//     blocks, then the table rows, and only then its weight slice. Vector
//     memory returns in issue order per wavefront and the HBM queues fill
//     with the weight stream within a microsecond, so the gather's two
//     dependent loads go first; every workgroup gathers all of x for itself
//     (the rows are shared through L2), which costs some extra L2 hits but
//     no exchange between workgroups;
//  2. the blocks are quantized straight into LDS (codes with 16-byte pieces
//     XOR-swizzled by token, scales), the weights land, the scaled MFMAs run
//     split over k as in the stand-alone decode GEMV, and the 8 partial tiles
//     are summed through LDS in wave order;
//  3. each 16-column tile of keys yields per-token partials (sum
//     key*hidden*q*k, sum key^2) of the bf16-rounded keys, stored contiguously
//     per (copy, token); value tiles are stored as bf16; then the workgroup
//     raises its own flag (release);
//  4. the last F workgroups (by index, so dispatched last) wait until every
//     flag is up and each finishes whole (token, copy) rows: fixed-order sums
//     of the tile partials and of hidden^2 (hidden prefetched before the
//     wait), the gate, out = hidden + g * value. The last finisher lowers the
//     flags again.
//
// The flags and one counter live in the first 64 KiB of the caller's
// workspace: zero before the first call, zero again after every call. Every
// wait is bounded in time; a timeout, or a flag found up on entry, sets bit 1
// of the error flag instead of hanging.
#include <algorithm>
#include <array>
#include <mutex>
#include <unordered_map>

#include "common.h"
#include "mx_rule.h"

namespace engram {

namespace {

constexpr int DF_WAVES = 8;
constexpr int DF_THREADS = DF_WAVES * 64;
constexpr uint64_t kSpinTicks = 20000000ull;   // 200 ms of the 100 MHz real-time counter
constexpr int kMaxBPL = 8;                     // MX blocks of x per thread (T*K <= 128 KiB)
constexpr int kPrefetch = 2;                   // hidden pieces per finisher thread fetched early
constexpr int kRegBudget = 160;                // VGPRs for weights + rows in flight (no spills)
constexpr int SY_FDONE = 0, SY_FLAGS = 64;     // uint32 word offsets in the counter area

struct DecodeArgs {
  const uint4* table; int64_t num_rows; int head_dim;
  const int32_t* ids; int64_t st, sc; int n_cols;
  int T, K, N;
  const uint8_t* w; const uint8_t* ws;
  const uint16_t* hidden; const uint16_t* q; const uint16_t* k; const uint8_t* mask;
  int hc, dim; float eps, clamp, inv_dim, rsqrt_dim;
  uint16_t* out; float* gate_out; int32_t* err;
  uint32_t* sync; uint16_t* value; float2* part;
  int finishers;
};

__device__ __forceinline__ i32x8 cat(const uint4& lo, const uint4& hi) {
  return __builtin_shufflevector(__builtin_bit_cast(i32x4, lo), __builtin_bit_cast(i32x4, hi),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = bf16lo(v.x); f[1] = bf16hi(v.x);
  f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
  f[4] = bf16lo(v.z); f[5] = bf16hi(v.z);
  f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
}

// Wave 0 waits until flags[0, G) are all up (relaxed polls, one acquire at
// the end). The loop control is scalar (ballot, readfirstlane) so all lanes
// stay together. Bounded; returns false on timeout.
__device__ bool wait_all_flags(const uint32_t* flags, int G, int lane) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    bool up = true;
    for (int i = lane; i < G; i += 64)
      up = up && __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    const int all_up = __builtin_amdgcn_readfirstlane(__ballot(!up) == 0ull ? 1 : 0);
    if (all_up) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) return false;
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

// Finish one (token, copy) row: fixed-order sums of the tile partials and of
// hidden^2, the gate, out = hidden + g * value. pre0/pre1 hold this
// thread's hidden pieces j = tid and tid + DF_THREADS when `have_pre`.
__device__ __forceinline__ void finish_row(const DecodeArgs& a, int t, int h, uint4 pre0, uint4 pre1,
                                           bool have_pre, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int dim8 = a.dim / 8;
  const uint4* hrow = reinterpret_cast<const uint4*>(a.hidden + ((int64_t)t * a.hc + h) * a.dim);
  uint4* orow = reinterpret_cast<uint4*>(a.out + ((int64_t)t * a.hc + h) * a.dim);
  // fn(j, hidden piece j) over this thread's pieces j = tid + DF_THREADS*m;
  // the first two come from registers
  // (value selects, not `c ? pre0 : hrow[j]`, which would give pre0 an address)
  auto piece = [&](int j, const uint4& pre) {
    uint4 v;
    if (have_pre) v = pre;
    else v = hrow[j];
    return v;
  };
  auto for_pieces = [&](auto fn) {
    if (tid < dim8) fn(tid, piece(tid, pre0));
    if (tid + DF_THREADS < dim8) fn(tid + DF_THREADS, piece(tid + DF_THREADS, pre1));
    for (int j = tid + DF_THREADS * kPrefetch; j < dim8; j += DF_THREADS) fn(j, hrow[j]);
  };
  if (a.mask && a.mask[t] == 0) {
    for_pieces([&](int j, const uint4& hv) { orow[j] = hv; });
    if (a.gate_out && tid == 0) a.gate_out[(int64_t)t * a.hc + h] = 0.0f;
    return;
  }
  const int tiles = a.dim / 16;
  const float2* prow = a.part + ((int64_t)h * a.T + t) * tiles;
  float dt = 0.f, ks = 0.f, hs = 0.f;
  for (int i = tid; i < tiles; i += DF_THREADS) {
    const float2 p = prow[i];
    dt += p.x;
    ks += p.y;
  }
  for_pieces([&](int, const uint4& hv) {
    float f[8];
    unpack8(hv, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) hs = fmaf(f[e], f[e], hs);
  });
  dt = wave_sum(dt);
  ks = wave_sum(ks);
  hs = wave_sum(hs);
  if (lane == 0) { red[wave * 3 + 0] = dt; red[wave * 3 + 1] = ks; red[wave * 3 + 2] = hs; }
  __syncthreads();
  float s_dt = 0.f, s_ks = 0.f, s_hs = 0.f;
#pragma unroll
  for (int v = 0; v < DF_WAVES; ++v) {   // fixed wave order
    s_dt += red[v * 3 + 0];
    s_ks += red[v * 3 + 1];
    s_hs += red[v * 3 + 2];
  }
  const float hidden_rms = 1.0f / sqrtf(s_hs * a.inv_dim + a.eps);
  const float key_rms = 1.0f / sqrtf(s_ks * a.inv_dim + a.eps);
  const float d = s_dt * hidden_rms * key_rms * a.rsqrt_dim;
  float s = sqrtf(fmaxf(fabsf(d), a.clamp));
  s = d < 0.0f ? -s : s;
  const float g = 1.0f / (1.0f + expf(-s));
  if (a.gate_out && tid == 0) a.gate_out[(int64_t)t * a.hc + h] = g;
  const uint4* vrow = reinterpret_cast<const uint4*>(a.value + (int64_t)t * a.dim);
  for_pieces([&](int j, const uint4& hv) {
    float f[8], v[8];
    unpack8(hv, f);
    unpack8(vrow[j], v);
    uint4 o;
    o.x = pack_bf16x2(fmaf(g, v[0], f[0]), fmaf(g, v[1], f[1]));
    o.y = pack_bf16x2(fmaf(g, v[2], f[2]), fmaf(g, v[3], f[3]));
    o.z = pack_bf16x2(fmaf(g, v[4], f[4]), fmaf(g, v[5], f[5]));
    o.w = pack_bf16x2(fmaf(g, v[6], f[6]), fmaf(g, v[7], f[7]));
    orow[j] = o;
  });
  __syncthreads();   // red is reused by the next row
}

// LDS layout (dynamic): [ x codes T*K (16-byte pieces XOR-swizzled by token),
// aliased by the cross-wave reduction after the MFMAs ] [ x scales T*K/32 ]
// [ hidden slices RT x 16*NT tokens x 16 bf16 ] [ q*k slices RT x 16 fp32 ].
template <int RT, int NT, int SPW, int BPL>
__global__ __launch_bounds__(DF_THREADS) void decode_forward_kernel(DecodeArgs a, int xs_off, int hid_off,
                                                                    int qk_off) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  __shared__ float s_red[3 * DF_WAVES];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, b = blockIdx.x;
  const int n0 = b * 16 * RT;
  const int K = a.K, T = a.T, kb = K / 32;
  const int g = lane >> 4, r = lane & 15;
  const int nsteps = K / 128;
  const int key_cols = a.hc * a.dim;
  const int bpr = a.head_dim / 32;
  const int nblocks = T * a.n_cols * bpr;
  const int F = a.finishers;
  const bool finisher = b >= G - F;
  uint32_t* flags = a.sync + SY_FLAGS;

  // 1. hash ids of this thread's MX blocks q = tid + DF_THREADS*i, then their rows
  int64_t id[BPL];
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int qb = tid + DF_THREADS * i;
    id[i] = -1;
    if (qb < nblocks) {
      const int row = qb / bpr, t = row / a.n_cols, c = row - t * a.n_cols;
      id[i] = a.ids[(int64_t)t * a.st + (int64_t)c * a.sc];
    }
  }
  uint4 rows[BPL][4];
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int qb = tid + DF_THREADS * i;
#pragma unroll
    for (int e = 0; e < 4; ++e) rows[i][e] = make_uint4(0, 0, 0, 0);
    if (qb < nblocks && id[i] >= 0 && id[i] < a.num_rows) {
      const uint4* src = a.table + (id[i] * a.head_dim + (qb % bpr) * 32) / 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) rows[i][e] = src[e];
    }
  }

  // 2. the weight slice: wave w takes k steps [w*SPW, (w+1)*SPW) of every row tile
  uint4 wlo[RT][SPW], whi[RT][SPW];
  int wsc[RT][SPW];
  const int step0 = wave * SPW;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int nrow = n0 + rt * 16;
    const uint8_t* wrow = a.w + (int64_t)(nrow + r) * K;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      wlo[rt][s] = whi[rt][s] = make_uint4(0, 0, 0, 0);
      wsc[rt][s] = 0;
      if (step0 + s < nsteps) {
        const int kbyte = (step0 + s) * 128 + 16 * g;
        wlo[rt][s] = *reinterpret_cast<const uint4*>(wrow + kbyte);
        whi[rt][s] = *reinterpret_cast<const uint4*>(wrow + kbyte + 64);
        wsc[rt][s] = a.ws[(nrow / 32) * kb + (step0 + s) * 4 + g];
      }
    }
  }

  // 3. operands of the epilogue and of the finish (needed after the weights
  // anyway): hidden and q*k slices of this workgroup's key tiles, the
  // finisher's first hidden row, and this workgroup's own flag (down on entry)
  constexpr int HID_PIECES = RT * NT * 16 * 2;             // 16-byte pieces, <= DF_THREADS
  static_assert(HID_PIECES <= DF_THREADS, "one hidden piece per thread");
  uint4 hslice = make_uint4(0, 0, 0, 0);
  if (tid < HID_PIECES) {
    const int rt = tid / (NT * 32), rem = tid - rt * NT * 32, tt = rem >> 1, half = rem & 1;
    const int n = n0 + rt * 16;
    if (tt < T && n < key_cols) {
      const int h = n / a.dim, d = n - h * a.dim + half * 8;
      hslice = *reinterpret_cast<const uint4*>(a.hidden + ((int64_t)tt * a.hc + h) * a.dim + d);
    }
  }
  float qk = 0.f;
  if (tid < RT * 16 && n0 + tid < key_cols) {
    const int n = n0 + tid, h = n / a.dim, d = n - h * a.dim;
    qk = __uint_as_float((uint32_t)a.q[h * a.dim + d] << 16) * __uint_as_float((uint32_t)a.k[h * a.dim + d] << 16);
  }
  static_assert(kPrefetch == 2, "two prefetched pieces: pre0, pre1");
  uint4 pre0 = make_uint4(0, 0, 0, 0), pre1 = make_uint4(0, 0, 0, 0);
  const int first_pair = b - (G - F);
  const bool have_pre = finisher && first_pair < T * a.hc && a.dim / 8 <= DF_THREADS * kPrefetch;
  if (have_pre) {
    const int t = first_pair / a.hc, h = first_pair - t * a.hc;
    const uint4* hrow = reinterpret_cast<const uint4*>(a.hidden + ((int64_t)t * a.hc + h) * a.dim);
    if (tid < a.dim / 8) pre0 = hrow[tid];
    if (tid + DF_THREADS < a.dim / 8) pre1 = hrow[tid + DF_THREADS];
  }
  const uint32_t own_flag = tid == 0 ? __hip_atomic_load(flags + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;

  // 4. quantize this thread's blocks into LDS (the rows were issued first)
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int qb = tid + DF_THREADS * i;
    if (qb < nblocks) {
      if ((id[i] < 0 || id[i] >= a.num_rows) && a.err) atomicOr(a.err, 1);
      uint32_t wv[16], packed[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wv[4 * e + 0] = rows[i][e].x; wv[4 * e + 1] = rows[i][e].y;
        wv[4 * e + 2] = rows[i][e].z; wv[4 * e + 3] = rows[i][e].w;
      }
      const int byte = mx_block(wv, packed);
      const int row = qb / bpr, t = row / a.n_cols, c = row - t * a.n_cols;
      const int kpos = c * a.head_dim + (qb % bpr) * 32;      // byte offset in x's row
      const int piece = kpos >> 4;
      char* xrow = smem + t * K;
      *reinterpret_cast<uint4*>(xrow + ((piece ^ (t & 15)) << 4)) =
          make_uint4(packed[0], packed[1], packed[2], packed[3]);
      *reinterpret_cast<uint4*>(xrow + (((piece + 1) ^ (t & 15)) << 4)) =
          make_uint4(packed[4], packed[5], packed[6], packed[7]);
      smem[xs_off + t * kb + (kpos >> 5)] = (char)byte;
    }
  }
  if (tid < HID_PIECES) reinterpret_cast<uint4*>(smem + hid_off)[tid] = hslice;
  if (tid < RT * 16) reinterpret_cast<float*>(smem + qk_off)[tid] = qk;
  __syncthreads();   // x, hidden and q*k slices in LDS

  // 5. scaled MFMAs: A = 16 W rows, B = 16 tokens (padding tokens read zeros)
  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = j * 16 + r;
    const bool live = t < T;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (step0 + s >= nsteps) break;  // uniform per wave
      const int piece = (step0 + s) * 8 + g;
      uint4 xlo = make_uint4(0, 0, 0, 0), xhi = make_uint4(0, 0, 0, 0);
      int xsc = 0;
      if (live) {
        xlo = *reinterpret_cast<const uint4*>(smem + t * K + ((piece ^ (t & 15)) << 4));
        xhi = *reinterpret_cast<const uint4*>(smem + t * K + (((piece + 4) ^ (t & 15)) << 4));
        xsc = (unsigned char)smem[xs_off + t * kb + (step0 + s) * 4 + g];
      }
      const i32x8 xb = cat(xlo, xhi);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            cat(wlo[rt][s], whi[rt][s]), xb, acc[rt][j], 0, 0, 0, wsc[rt][s], 0, xsc);
    }
  }
  __syncthreads();   // x no longer needed: its LDS becomes the reduction buffer
  f32x4* red = reinterpret_cast<f32x4*>(smem);   // [8][RT*NT][64]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[(wave * RT * NT + rt * NT + j) * 64 + lane] = acc[rt][j];
  __syncthreads();

  // 6. wave v < RT*NT finishes tile pair v = (rt, j): lane l holds rows
  // 4*(l/16)+i of tile rt, token j*16 + l%16
  if (wave < RT * NT) {
    const int rt = wave / NT, j = wave - rt * NT;
    f32x4 sum = red[wave * 64 + lane];
#pragma unroll
    for (int v = 1; v < DF_WAVES; ++v) {
      const f32x4 p = red[(v * RT * NT + wave) * 64 + lane];
      sum[0] += p[0]; sum[1] += p[1]; sum[2] += p[2]; sum[3] += p[3];
    }
    const int t = j * 16 + (lane & 15);
    const int nt0 = n0 + rt * 16;                 // the tile's first column
    const int nr = 4 * (lane >> 4);               // this lane's first row in the tile
    uint32_t kb2[2];
    kb2[0] = pack_bf16x2(sum[0], sum[1]);
    kb2[1] = pack_bf16x2(sum[2], sum[3]);
    if (nt0 < key_cols) {
      // key tile: partial sums from the bf16-rounded keys
      const float key[4] = {bf16lo(kb2[0]), bf16hi(kb2[0]), bf16lo(kb2[1]), bf16hi(kb2[1])};
      const uint16_t* hl = reinterpret_cast<const uint16_t*>(smem + hid_off) + (rt * NT * 16 + t) * 16;
      const float* qk_l = reinterpret_cast<const float*>(smem + qk_off) + rt * 16;
      float dt = 0.f, ks = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float hv = __uint_as_float((uint32_t)hl[nr + i] << 16);
        ks = fmaf(key[i], key[i], ks);
        dt = fmaf(hv * qk_l[nr + i], key[i], dt);
      }
      // lanes l, l^16, l^32, l^48 hold the tile's 16 rows of one token
      dt += __shfl_xor(dt, 16, 64);
      ks += __shfl_xor(ks, 16, 64);
      dt += __shfl_xor(dt, 32, 64);
      ks += __shfl_xor(ks, 32, 64);
      const int h = nt0 / a.dim;
      if (lane < 16 && t < T)
        a.part[((int64_t)h * T + t) * (a.dim / 16) + (nt0 - h * a.dim) / 16] = make_float2(dt, ks);
    } else if (t < T) {
      *reinterpret_cast<uint2*>(a.value + (int64_t)t * a.dim + (nt0 - key_cols) + nr) =
          make_uint2(kb2[0], kb2[1]);
    }
  }

  // 7. publish: every thread's stores have landed, then this workgroup's flag goes up
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    if (own_flag != 0u && a.err) atomicOr(a.err, 2);   // flags not lowered: counter area dirty
    __hip_atomic_store(flags + b, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!finisher) return;

  // 8. finish: wait for every flag, then whole (token, copy) rows
  if (wave == 0) {
    const bool ok = wait_all_flags(flags, G, lane);
    if (!ok && lane == 0 && a.err) atomicOr(a.err, 2);
  }
  __syncthreads();
  for (int p = first_pair, n = 0; p < T * a.hc; p += F, ++n) {
    const int t = p / a.hc, h = p - t * a.hc;
    finish_row(a, t, h, pre0, pre1, have_pre && n == 0, s_red);
  }

  // 9. the last finisher lowers every flag for the next call
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(a.sync + SY_FDONE, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = done == (uint32_t)F - 1 ? 1 : 0;
    if (done >= (uint32_t)F && a.err) atomicOr(a.err, 2);
  }
  __syncthreads();
  if (s_last) {
    for (int i = tid; i < G; i += DF_THREADS)
      __hip_atomic_store(flags + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) __hip_atomic_store(a.sync + SY_FDONE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Raise a kernel's dynamic-LDS limit to what a launch needs (above 64 KiB the
// launch fails without it). Host-side cost matters at decode, so the largest
// value set per (kernel, device) is cached.
hipError_t allow_lds(const void* fn, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static std::unordered_map<const void*, std::array<int, kMaxDev>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = done.find(fn);
  if (it == done.end()) it = done.emplace(fn, std::array<int, kMaxDev>{}).first;
  if (dev < kMaxDev && it->second[dev] >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && dev < kMaxDev) it->second[dev] = bytes;
  return e;
}

template <int RT, int NT, int BPL>
hipError_t launch_rt(const DecodeArgs& a, int spw, hipStream_t s) {
  const int G = a.N / (16 * RT);
  const int red_bytes = DF_WAVES * RT * NT * 64 * 16;
  const int xs_off = (std::max(a.T * a.K, red_bytes) + 255) & ~255;
  const int hid_off = (xs_off + a.T * (a.K / 32) + 255) & ~255;
  const int qk_off = hid_off + RT * NT * 16 * 32;
  const int lds = qk_off + RT * 16 * 4;
  DecodeArgs b = a;
  b.finishers = std::min(G, std::min(a.T * a.hc, 64));
  hipError_t e;
#define DF_CASE(S)                                                                                    \
  case S:                                                                                             \
    if constexpr (RT * S * 8 + BPL * 16 <= kRegBudget) {                                              \
      e = allow_lds((const void*)decode_forward_kernel<RT, NT, S, BPL>, lds);                         \
      if (e != hipSuccess) return e;                                                                  \
      hipLaunchKernelGGL((decode_forward_kernel<RT, NT, S, BPL>), dim3(G), dim3(DF_THREADS), lds, s,  \
                         b, xs_off, hid_off, qk_off);                                                 \
      return hipGetLastError();                                                                       \
    }                                                                                                 \
    return hipErrorInvalidValue;
  switch (spw) {
    DF_CASE(1) DF_CASE(2) DF_CASE(3) DF_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef DF_CASE
}

// Row tiles per workgroup: the largest of 5, 4, 2, 1 that divides N/16, keeps
// RT*NT <= 8 (LDS of the cross-wave sum) and the weight and row registers in
// flight within budget.
template <int NT, int BPL>
hipError_t launch_nt(const DecodeArgs& a, hipStream_t s) {
  const int tiles = a.N / 16;
  const int spw = (a.K / 128 + DF_WAVES - 1) / DF_WAVES;
  auto fits = [&](int rt) { return rt * spw * 8 + BPL * 16 <= kRegBudget; };
  if constexpr (5 * NT <= 8)
    if (tiles % 5 == 0 && fits(5)) return launch_rt<5, NT, BPL>(a, spw, s);
  if constexpr (4 * NT <= 8)
    if (tiles % 4 == 0 && fits(4)) return launch_rt<4, NT, BPL>(a, spw, s);
  if (tiles % 2 == 0 && fits(2)) return launch_rt<2, NT, BPL>(a, spw, s);
  return launch_rt<1, NT, BPL>(a, spw, s);
}

template <int NT>
hipError_t launch_bpl(const DecodeArgs& a, hipStream_t s) {
  const int bpl = (a.T * a.K / 32 + DF_THREADS - 1) / DF_THREADS;
  if (bpl <= 1) return launch_nt<NT, 1>(a, s);
  if (bpl <= 2) return launch_nt<NT, 2>(a, s);
  if (bpl <= 4) return launch_nt<NT, 4>(a, s);
  return launch_nt<NT, 8>(a, s);
}

}  // namespace

bool decode_forward_supported(int64_t T, int K, int N, int head_dim, int dim, int hc) {
  if (T < 1 || T > kGemvMaxT || K % 1024 != 0 || N % 16 != 0 || head_dim % 32 != 0 || dim % 16 != 0 ||
      N != (hc + 1) * dim || N / 16 > kDecodeMaxFlags)
    return false;
  if (T * K / 32 > DF_THREADS * kMaxBPL) return false;        // x fits LDS and registers
  const int spw = (K / 128 + DF_WAVES - 1) / DF_WAVES;
  const int bpl = (int)((T * K / 32 + DF_THREADS - 1) / DF_THREADS);
  const int bpl_t = bpl <= 1 ? 1 : bpl <= 2 ? 2 : bpl <= 4 ? 4 : 8;
  return spw <= 4 && spw * 8 + bpl_t * 16 <= kRegBudget;        // RT = 1 fits
}

size_t decode_forward_scratch_bytes(int64_t T, int K, int N, int dim) {
  (void)K;
  // value [T, dim] bf16 | partials [hc, T, dim/16] float2
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return up((size_t)T * dim * 2) + up((size_t)(N / 16) * T * 8);
}

hipError_t launch_decode_forward(const void* table, int64_t num_rows, int head_dim, const int32_t* ids,
                                 int64_t st, int64_t sc, int n_cols, int64_t T, int K, const void* w,
                                 const uint8_t* w_scales, int N, const void* hidden, const void* q,
                                 const void* k, const uint8_t* mask, int hc, int dim, float eps,
                                 float clamp, void* out, float* gate_out, int32_t* err, uint32_t* sync,
                                 uint8_t* scratch, hipStream_t s) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  DecodeArgs a;
  a.table = (const uint4*)table; a.num_rows = num_rows; a.head_dim = head_dim;
  a.ids = ids; a.st = st; a.sc = sc; a.n_cols = n_cols;
  a.T = (int)T; a.K = K; a.N = N;
  a.w = (const uint8_t*)w; a.ws = w_scales;
  a.hidden = (const uint16_t*)hidden; a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.mask = mask;
  a.hc = hc; a.dim = dim; a.eps = eps; a.clamp = clamp;
  a.inv_dim = 1.0f / (float)dim; a.rsqrt_dim = 1.0f / sqrtf((float)dim);
  a.out = (uint16_t*)out; a.gate_out = gate_out; a.err = err;
  a.sync = sync;
  a.value = (uint16_t*)scratch;
  a.part = (float2*)(scratch + up((size_t)T * dim * 2));
  a.finishers = 1;
  switch ((int)((T + 15) / 16)) {
    case 1: return launch_bpl<1>(a, s);
    case 2: return launch_bpl<2>(a, s);
    case 3: return launch_bpl<3>(a, s);
    case 4: return launch_bpl<4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace engram
