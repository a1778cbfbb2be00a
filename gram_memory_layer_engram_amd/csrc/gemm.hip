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
//  * Both operands are K-contiguous. A = W rows (n), B = x rows (tokens): an
//    accumulator lane then holds 4 consecutive n of one token.
//  * Block tile 256 (n) x 256 (tokens); four waves in 2x2, each 128x128 =
//    4x4 MFMA tiles of 32x32 (256 fp32 accumulators per lane, in AGPRs). That
//    is the largest tile one CU's register file holds, and at K = 2048 the
//    kernel is bound by L2 -> CU operand traffic (one 256x256 tile reads 2 x
//    256 rows per k) and by the clock the chip sustains with MFMA and that
//    traffic both running, not by MFMA issue: the loop is paced for the
//    address unit, not for the matrix cores.
//  * Global -> LDS with buffer_load ... lds (16 bytes per lane, written at
//    LDS base + lane*16): no staging registers, no ds_write, and the buffer
//    descriptor's range check returns zeros past the last row of W or x, so
//    ragged tiles need no branches; a stage that does not exist is loaded
//    from an offset past the range (zeros into a buffer nobody reads), which
//    keeps the loop free of branches. The range check covers the vector
//    offset only, so every DMA offset (row, k slice, piece) is carried in it
//    and the scalar offset is 0 (gemm_dma.h; a host model of those offsets
//    checks each against the range).
//  * bf16: a k slice is 64 elements, so one DMA instruction fetches 8 rows x
//    128 bytes, 8 whole cache lines (with 32-element stages it touched half
//    of 16 lines: 627 -> 564 us for the prefill GEMM, same instructions,
//    same bytes). LDS rows are 128 bytes of 8 pieces, piece p of row r at
//    p ^ ((r >> 1) & 7), conflict-free for the 32-row fragment reads. Each
//    operand's slice is a 32 KiB chunk in a ring of five (160 KiB, all of
//    LDS): during slice d, B of slice d+1 is fetched first (one DMA per 2
//    MFMAs), then A of slice d+2 (one per 4), so every DMA has at least ~38
//    MFMAs before the barrier that needs it (32 already suffice: a
//    three-stage ring times like a four-stage one). The barrier that
//    publishes slice d+1 sits after the first 4 of the last 16 MFMAs of
//    slice d, and the next slice's first fragments are read under the other
//    12.
//  * MXFP8 (K % 256 == 0): the same ring of five 32 KiB chunks, a slice
//    being 128 e4m3 per row (gemm_mx_ring_kernel, described above it).
//    Other K: a plain two-stage kernel with 128-byte k stages (piece p of
//    row r at p ^ ((r >> 1) & 7)).
//  * Epilogue: the bf16 tile is staged in LDS as [token][n] (512-byte rows,
//    16-byte chunks XOR-swizzled by token) and written back as whole rows,
//    16 bytes per lane: 8 full cache lines per store instruction instead of
//    32 partial ones, which halves the epilogue.
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
#include "gemm_dma.h"

namespace engram {

namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BM = 256;      // W rows per block
constexpr int BN = 256;      // tokens per block
constexpr int THREADS = 256;
constexpr int LDS_BYTES = 128 * 1024;            // MXFP8 stages; the epilogue's staging tile (bf16 ring: Q_LDS)
// MXFP8: 128-byte k stages, two of them
constexpr int ROW_BYTES = 128;
constexpr int PIECES = ROW_BYTES / 16;
constexpr int TILE_BYTES = BM * ROW_BYTES;       // 32 KiB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;      // A + B
static_assert(2 * STAGE_BYTES == LDS_BYTES, "LDS budget");
static_assert(BN * 512 == LDS_BYTES, "epilogue staging tile");
// bf16: 64-element k slices (128-byte LDS rows of 8 pieces, piece p of row
// r at p ^ ((r >> 1) & 7)); each operand's slice is a 32 KiB chunk in a ring
// of five
constexpr int Q_ROW = 128;
constexpr int Q_CHUNK = BM * Q_ROW;
constexpr int Q_SLOTS = 5;
constexpr int Q_LDS = Q_SLOTS * Q_CHUNK;         // 160 KiB
constexpr int Q_DMA = Q_CHUNK / (THREADS * 16);  // DMA instructions per wave per chunk
static_assert(Q_DMA == 8 && Q_LDS >= LDS_BYTES, "bf16 ring");
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

// One MXFP8 k stage of both operand tiles, global -> LDS. Wave w issues 8
// DMA instructions per operand; instruction i fills rows 8*(w + 4*i) .. +8.
// `kb` is the stage's byte offset inside a row; `row_bytes` the global row
// pitch.
__device__ __forceinline__ void stage_load(rsrc_t ra, rsrc_t rb, char* lds_stage, int wave, int lane,
                                           uint32_t row_bytes, uint32_t kb) {
  const int sub = lane >> 3, pp = lane & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = wave + 4 * i;
    const int r = blk * 8 + sub;
    const int p = pp ^ ((r >> 1) & 7);
    const uint32_t off = (uint32_t)r * row_bytes + kb + (uint32_t)p * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(lds_stage + blk * 1024), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(lds_stage + TILE_BYTES + blk * 1024), 16, off, 0, 0, 0);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// A bare workgroup barrier: unlike __syncthreads() it does not first wait
// for every outstanding vector load, so later stages keep streaming.
__device__ __forceinline__ void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }

#define SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
constexpr int SG_MFMA = 0x008, SG_VMEM = 0x010, SG_DSR = 0x100;

// 16 bytes of the output tile, stored non-temporal: the kernel never reads
// kv back, and streaming it past the L2 keeps the operand lines there (the
// long-prefill MXFP8 GEMM, 2.2 GiB of kv: 3.15 -> 2.98 ms; the prefill
// shapes unchanged).
__device__ __forceinline__ void store_nt(uint16_t* dst, const uint4& v) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(dst));
}

// Write the block's accumulators: converted with v_cvt_pk_bf16_f32 (one
// instruction per pair instead of a dozen for the bit-level rounding: 644 ->
// 614 us for the prefill GEMM), staged in LDS as [token][n]
// (512-byte rows; 16-byte chunk c of row t at c ^ (t & 31)), then go over
// whole rows. The caller has drained its DMAs; LDS is free after the first
// barrier here. Rows past T are not written.
//  * plain (ep.hidden == nullptr): store the rows into kv [T, N] (N % 4 == 0,
//    so a row's last chunk may be half);
//  * gate epilogue (dim % 256 == 0, so a tile lies inside one key block or
//    the value block): value tiles go to ep.value [T, dim]; key tiles are
//    not stored but reduced, per token, to the gate's two kv-side sums over
//    the tile's 256 columns, sum hidden*q*k*key and sum key^2 of the
//    bf16-rounded keys ("vllm.models.deepseek_v41.amd.engram",
//    _engram_gate_partials_kernel, at tile granularity), into
//    ep.part[(h*T + t) * (dim/256) + tile].
__device__ __forceinline__ void store_tile(f32x16 (&acc)[4][4], char* smem, uint16_t* __restrict__ kv,
                                           int T, int N, int t0, int n0, int wn, int wt, int lane,
                                           int wave, const GateEpi& ep) {
  const int lrow = lane & 31, lhalf = lane >> 5;
  wait_lgkm0();
  bare_barrier();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = wt + j * 32 + lrow;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // accumulator r of lane l: n = 8*(r/4) + 4*(l/32) + r%4, token = l%32
        const int n = wn + i * 32 + 8 * g + 4 * lhalf;
        uint2 o;
        o.x = cvt_pk_bf16(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
        o.y = cvt_pk_bf16(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        *reinterpret_cast<uint2*>(smem + t * 512 + (((n >> 3) ^ (t & 31)) << 4) + (n & 7) * 2) = o;
      }
  }
  wait_lgkm0();
  bare_barrier();
  const int c = lane & 31;
  auto lds_row = [&](int t) { return *reinterpret_cast<const uint4*>(smem + t * 512 + ((c ^ (t & 31)) << 4)); };
  if (!ep.hidden) {
    const int n = n0 + c * 8;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
      const int t = wave * 64 + it * 2 + (lane >> 5);
      const uint4 v = lds_row(t);
      if (t0 + t < T) {
        uint16_t* dst = kv + (int64_t)(t0 + t) * N + n;
        if (n + 8 <= N) store_nt(dst, v);
        else if (n + 4 <= N) *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
      }
    }
    return;
  }
  const int key_cols = ep.hc * ep.dim;
  if (n0 >= key_cols) {
    // value tile
    const int d = n0 - key_cols + c * 8;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
      const int t = wave * 64 + it * 2 + (lane >> 5);
      const uint4 v = lds_row(t);
      if (t0 + t < T) store_nt(ep.value + (int64_t)(t0 + t) * ep.dim + d, v);
    }
    return;
  }
  // key tile of copy h, columns d0 .. d0+255 of that copy. Lane group g =
  // lane/16 of wave w takes rows t = 64w + 4r + g (r = 0..15: the four
  // groups read consecutive rows, which the LDS swizzle keeps on distinct
  // banks); lane c16 = lane%16 takes the 16-byte pieces c16 and 16 + c16 of
  // each row (columns 8*c16.. and 128 + 8*c16..), so a load instruction
  // covers 256 contiguous bytes of four rows.
  const int h = n0 / ep.dim, d0 = n0 - h * ep.dim;
  const int g = lane >> 4, c16 = lane & 15;
  float qk[16];
  {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int d = d0 + half * 128 + c16 * 8;
      const uint4 q8 = *reinterpret_cast<const uint4*>(ep.q + h * ep.dim + d);
      const uint4 k8 = *reinterpret_cast<const uint4*>(ep.k + h * ep.dim + d);
      const uint32_t qw[4] = {q8.x, q8.y, q8.z, q8.w}, kw[4] = {k8.x, k8.y, k8.z, k8.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qk[half * 8 + 2 * e] = bf16lo(qw[e]) * bf16lo(kw[e]);
        qk[half * 8 + 2 * e + 1] = bf16hi(qw[e]) * bf16hi(kw[e]);
      }
    }
  }
  const int tiles = ep.dim / 256, tile = d0 / 256;
  // all 32 hidden pieces of this thread in flight at once (the accumulators
  // are dead, their registers free), then the reductions
  uint4 hid[16][2];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = wave * 64 + 4 * r + g;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      hid[r][half] = make_uint4(0, 0, 0, 0);
      if (t0 + t < T)
        hid[r][half] = *reinterpret_cast<const uint4*>(ep.hidden + ((int64_t)(t0 + t) * ep.hc + h) * ep.dim + d0 +
                                                       half * 128 + c16 * 8);
    }
  }
  // per-lane sums of this lane's 16 columns, one pair per row r
  float dts[16], kss[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = wave * 64 + 4 * r + g;
    float dt = 0.f, ks = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int ch = half * 16 + c16;
      const uint4 kv8 = *reinterpret_cast<const uint4*>(smem + t * 512 + ((ch ^ (t & 31)) << 4));
      const uint4 h8 = hid[r][half];
      const uint32_t kw[4] = {kv8.x, kv8.y, kv8.z, kv8.w}, hw[4] = {h8.x, h8.y, h8.z, h8.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float k0 = bf16lo(kw[e]), k1 = bf16hi(kw[e]);
        ks = fmaf(k0, k0, ks);
        ks = fmaf(k1, k1, ks);
        dt = fmaf(bf16lo(hw[e]) * qk[half * 8 + 2 * e], k0, dt);
        dt = fmaf(bf16hi(hw[e]) * qk[half * 8 + 2 * e + 1], k1, dt);
      }
    }
    dts[r] = dt;
    kss[r] = ks;
  }
  // Sum over the 16 lanes of each group for all 16 rows at once: at each
  // step lane c16 keeps the half of its rows selected by bit w of c16 and
  // adds the partner's (lane c16^w) copy of them, so 15 exchanges per sum;
  // lane c16 ends with row r = c16, in a fixed order. (With 32 lanes per row
  // the exchanges double, 62 shuffles against 30: 633 -> 625 us at the
  // prefill shape; 8 lanes per row, 14 shuffles but 128-byte row pieces per
  // load, measured 642 us.)
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) {
    const bool upper = (c16 & w) != 0;
#pragma unroll
    for (int i = 0; i < w; ++i) {
      const float rd = __shfl_xor(upper ? dts[i] : dts[i + w], w, 64);
      const float rk = __shfl_xor(upper ? kss[i] : kss[i + w], w, 64);
      dts[i] = (upper ? dts[i + w] : dts[i]) + rd;
      kss[i] = (upper ? kss[i + w] : kss[i]) + rk;
    }
  }
  const int t = wave * 64 + 4 * c16 + g;
  if (t0 + t < T) ep.part[((int64_t)h * T + t0 + t) * tiles + tile] = make_float2(dts[0], kss[0]);
}

// bf16 wkv GEMM (see the file comment). KTAIL: K % 64 != 0, the last slice's
// pieces past the row end are loaded from past the range (zeros).
template <bool KTAIL>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint16_t* __restrict__ x, int T, int K, const uint16_t* __restrict__ w,
                      int N, uint16_t* __restrict__ kv, int tiles_n, int tiles_t, GateEpi ep) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int tn, tt;
  tile_of(blockIdx.x, tiles_n, tiles_t, tn, tt);
  const int n0 = tn * BM, t0 = tt * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = (wave >> 1) * 128, wt = (wave & 1) * 128;
  const uint32_t row_bytes = (uint32_t)K * 2u;
  const rsrc_t ra = make_rsrc(w + (int64_t)n0 * K, (uint32_t)min(BM, N - n0) * row_bytes);
  const rsrc_t rb = make_rsrc(x + (int64_t)t0 * K, (uint32_t)min(BN, T - t0) * row_bytes);
  const uint32_t oob = (uint32_t)BM * row_bytes;   // at or past both ranges
  const int nk = (K + 63) / 64;

  // DMA i (0..7) of a chunk: LDS rows 8*(wave + 4i) .. +8 (gemm_dma.h). The
  // whole offset, row step and k offset included, is the range-checked
  // vector offset; the scalar offset stays 0.
  const dma::Lane dl = dma::lane_of(wave, lane, row_bytes);
  auto dma = [&](int slot_ofs, int op, uint32_t kofs, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op ? rb : ra, (lds_ptr_t)(smem + slot_ofs + (wave + 4 * i) * 1024),
                                             16, dma::voffset(dl, i, kofs, row_bytes, oob, KTAIL), 0, 0, 0);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int lrow = lane & 31, lhalf = lane >> 5;
  const int fsw = (lrow >> 1) & 7;
  bf16x8_t a[2][4], b[2][4];
  // fragment f (0..3: b0..b3, 4..7: a0..a3) of sub-step kk (0..3) into register set c
  auto frag = [&](int sa, int sb, int kk, int c, int f) {
    const int i = f & 3;
    const int row = (f < 4 ? wt : wn) + i * 32 + lrow;
    const int piece = (2 * kk + lhalf) ^ fsw;
    const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(smem + (f < 4 ? sb : sa) + row * Q_ROW + piece * 16);
    if (f < 4) b[c][i] = v; else a[c][i] = v;
  };
  auto mfma_row = [&](int c, int i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
  };

  // prologue: A0 -> slot 0, B0 -> slot 1, A1 -> slot 2
#pragma unroll
  for (int i = 0; i < Q_DMA; ++i) dma(0, 0, 0u, i);
#pragma unroll
  for (int i = 0; i < Q_DMA; ++i) dma(Q_CHUNK, 1, 0u, i);
#pragma unroll
  for (int i = 0; i < Q_DMA; ++i) dma(2 * Q_CHUNK, 0, nk > 1 ? (uint32_t)Q_ROW : oob, i);
  wait_vm<Q_DMA>();
  bare_barrier();
#pragma unroll
  for (int f = 0; f < 8; ++f) frag(0, Q_CHUNK, 0, 0, f);

  // Chunk c (A_d = 2d, B_d = 2d+1) lives in ring slot c % 5. While slice d
  // is computed, B_{d+1} (slot (2d+3) % 5) and A_{d+2} (slot (2d+4) % 5) are
  // fetched into the slots of A_{d-1} and B_{d-1}, freed by the previous
  // slice's barrier. The slot offsets are computed per slice (an unrolled
  // ring makes every fragment address loop-invariant: 232 spilled VGPRs).
  int base = 0;   // (2d) % 5
  for (int d = 0; d < nk; ++d) {
    {
      auto slot = [&](int m) { const int v = base + m; return (v >= Q_SLOTS ? v - Q_SLOTS : v) * Q_CHUNK; };
      const int sa = slot(0), sb = slot(1), sa1 = slot(2), sb1 = slot(3), sa2 = slot(4);
      const uint32_t kb1 = d + 1 < nk ? (uint32_t)(d + 1) * Q_ROW : oob;
      const uint32_t ka2 = d + 2 < nk ? (uint32_t)(d + 2) * Q_ROW : oob;
      // sub-step 0: MFMAs on set 0; sub-step 1's fragments into set 1; B_{d+1}, two DMAs per quarter
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        dma(sb1, 1, kb1, 2 * q);
        dma(sb1, 1, kb1, 2 * q + 1);
        frag(sa, sb, 1, 1, 2 * q);
        frag(sa, sb, 1, 1, 2 * q + 1);
        mfma_row(0, q);
        SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_DSR, 1); SGB(SG_MFMA, 1);
        SGB(SG_VMEM, 1); SGB(SG_MFMA, 1); SGB(SG_DSR, 1); SGB(SG_MFMA, 1);
      }
      // sub-steps 1 and 2: A_{d+2}, one DMA per quarter
#pragma unroll
      for (int kk = 1; kk < 3; ++kk) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __builtin_amdgcn_sched_barrier(0);
          dma(sa2, 0, ka2, (kk - 1) * 4 + q);
          frag(sa, sb, kk + 1, (kk + 1) & 1, 2 * q);
          frag(sa, sb, kk + 1, (kk + 1) & 1, 2 * q + 1);
          mfma_row(kk & 1, q);
          SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_MFMA, 1); SGB(SG_DSR, 1);
          SGB(SG_MFMA, 1); SGB(SG_DSR, 1); SGB(SG_MFMA, 1);
        }
      }
      // sub-step 3, first quarter, then publish slice d+1: each wave waits
      // for its own DMAs of A_{d+1} and B_{d+1} (only A_{d+2}'s 8 may still
      // fly) and for its LDS reads of slice d, then the barrier
      __builtin_amdgcn_sched_barrier(0);
      mfma_row(1, 0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<Q_DMA>();
      wait_lgkm0();
      bare_barrier();
      // quarters 1-3: slice d+1's sub-step-0 fragments into set 0 (3 + 3 + 2)
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        const int f0 = q == 1 ? 0 : (q == 2 ? 3 : 6), nf = q == 3 ? 2 : 3;
#pragma unroll
        for (int f = 0; f < nf; ++f) frag(sa1, sb1, 0, 0, f0 + f);
        mfma_row(1, q);
        if (q < 3) {
          SGB(SG_MFMA, 1); SGB(SG_DSR, 1); SGB(SG_MFMA, 1); SGB(SG_DSR, 1);
          SGB(SG_MFMA, 1); SGB(SG_DSR, 1); SGB(SG_MFMA, 1);
        } else {
          SGB(SG_MFMA, 1); SGB(SG_DSR, 1); SGB(SG_MFMA, 1); SGB(SG_DSR, 1); SGB(SG_MFMA, 2);
        }
      }
    }
    base = base + 2 >= Q_SLOTS ? base + 2 - Q_SLOTS : base + 2;
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();   // the zero-fill DMAs of the last slices land before LDS is reused
  store_tile(acc, smem, kv, T, N, t0, n0, wn, wt, lane, wave, ep);
}

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mxfp8_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int T, int K,
                       const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, int N,
                       uint16_t* __restrict__ kv, int tiles_n, int tiles_t, GateEpi ep) {
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

  stage_load(ra, rb, smem, wave, lane, row_bytes, 0);
  scale_load(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE_BYTES;
    uint32_t csa[4], csb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { csa[i] = sa[i]; csb[i] = sb[i]; }
    if (kt + 1 < nk) {
      stage_load(ra, rb, smem + ((kt + 1) & 1) * STAGE_BYTES, wave, lane, row_bytes,
                 (uint32_t)(kt + 1) * 128u);
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

  store_tile(acc, smem, kv, T, N, t0, n0, wn, wt, lane, wave, ep);
}

constexpr int S_ROW = 128;                      // MXFP8 ring: 128-byte slices (two k steps)

// MXFP8 GEMM on the bf16 kernel's ring (K % 256 == 0). A slice is 128
// e4m3 per row, two MFMA k steps ("stages", 16 MFMAs per wave each), so a
// DMA instruction fetches 8 rows x 128 bytes, 8 whole cache lines. Each
// operand's slice is a 32 KiB chunk in a ring of five (all 160 KiB of LDS),
// chunk c in slot c % 5 with A_d = chunk 2d and B_d = chunk 2d+1. During
// slice d, B_{d+1} goes out in stage 0 (two DMAs per quarter) and A_{d+2} in
// stage 1 (3, 3, 2), into the slots of A_{d-1} and B_{d-1}; the barrier that
// publishes slice d+1 sits after three of stage 1's four MFMA row blocks.
// A's DMAs thus get more than a slice of lead (two 64 KiB slice buffers
// gave every DMA about 37% of one: long-prefill GEMM 3.32 -> 3.16 ms).
// With LDS full, the E8M0 bytes are read from memory into registers, one
// group of four stages (8 bytes per row) ahead, issued at the start of a
// group's first slice, before its DMAs, so the barrier's wait covers them.
// Lane (row l%32, group g = l/32) reads, for stage h, pieces 4h+g and
// 4h+2+g of its row and passes the E8M0 byte of k block 2*stage + g. The
// fragments stream one A row block ahead (two register sets); B and the
// next stage's first A block are read under a stage's last four MFMAs.
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mx_ring_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int T, int K,
                         const uint8_t* __restrict__ w, const uint8_t* __restrict__ ws, int N,
                         uint16_t* __restrict__ kv, int tiles_n, int tiles_t, GateEpi ep) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int tn, tt;
  tile_of(blockIdx.x, tiles_n, tiles_t, tn, tt);
  const int n0 = tn * BM, t0 = tt * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = (wave >> 1) * 128, wt = (wave & 1) * 128;
  const uint32_t row_bytes = (uint32_t)K;
  const rsrc_t ra = make_rsrc(w + (int64_t)n0 * K, (uint32_t)min(BM, N - n0) * row_bytes);
  const rsrc_t rb = make_rsrc(xq + (int64_t)t0 * K, (uint32_t)min(BN, T - t0) * row_bytes);
  const uint32_t oob = (uint32_t)BM * row_bytes;   // at or past both ranges
  const int ns = K / 128;                           // slices, even
  const int kb = K / 32;                            // scale bytes per row, a multiple of 8
  const int lrow = lane & 31, lg = lane >> 5;

  const dma::Lane dl = dma::lane_of(wave, lane, row_bytes);
  auto dma = [&](int slot_ofs, int op, uint32_t kofs, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op ? rb : ra, (lds_ptr_t)(smem + slot_ofs + (wave + 4 * i) * 1024),
                                             16, dma::voffset(dl, i, kofs, row_bytes, oob, false), 0, 0, 0);
  };

  // The 8 scale bytes of stages s4 .. s4+3 (s4 % 4 == 0) of each row, as
  // range-checked vector loads: a scalar load would be waited for by the
  // next fragment read's lgkmcnt(0). Token rows past T read zeros.
  const rsrc_t rsa = make_rsrc(ws, (uint32_t)(N / 32) * (uint32_t)kb);
  const rsrc_t rsb = make_rsrc(xs + (int64_t)t0 * kb, (uint32_t)min(BN, T - t0) * (uint32_t)kb);
  uint32_t arow[4], brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    arow[i] = (uint32_t)min((n0 + wn + i * 32) / 32, N / 32 - 1) * (uint32_t)kb;
    brow[i] = (uint32_t)(wt + i * 32 + lrow) * (uint32_t)kb;
  }
  auto scales8 = [&](int s4, u32x2 (&a8)[4], u32x2 (&b8)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a8[i] = __builtin_amdgcn_raw_buffer_load_b64(rsa, arow[i] + 2u * (uint32_t)s4, 0, 0);
      b8[i] = __builtin_amdgcn_raw_buffer_load_b64(rsb, brow[i] + 2u * (uint32_t)s4, 0, 0);
    }
  };
  const uint32_t lsh = (uint32_t)lg * 8u;
  auto pick = [&](const u32x2& v, int u) {   // u static: byte 2u + lg
    return (int)(((u < 2 ? v.x : v.y) >> ((uint32_t)(16 * (u & 1)) + lsh)) & 0xffu);
  };
  auto frag = [&](int slot_ofs, int half, int row) {
    const char* base = smem + slot_ofs + row * S_ROW;
    const int sw = (row >> 1) & 7;
    const i32x4 lo = *reinterpret_cast<const i32x4*>(base + (((4 * half + lg) ^ sw) << 4));
    const i32x4 hi = *reinterpret_cast<const i32x4*>(base + (((4 * half + 2 + lg) ^ sw) << 4));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  i32x8 a0, a1, b[4], nb[4];
  int sa[4], sb[4];
  auto mfma_row = [&](const i32x8& a, int i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[j], acc[i][j], 0, 0, 0, sa[i], 0,
                                                                 sb[j]);
  };

  // prologue: the first group's scale bytes, then A_0 -> slot 0, B_0 -> slot
  // 1, A_1 -> slot 2; wait for all but A_1's 8 DMAs
  u32x2 sa8[4], sb8[4], na8[4], nb8[4];
  scales8(0, sa8, sb8);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < Q_DMA; ++i) dma(0, 0, 0u, i);
#pragma unroll
  for (int i = 0; i < Q_DMA; ++i) dma(Q_CHUNK, 1, 0u, i);
#pragma unroll
  for (int i = 0; i < Q_DMA; ++i) dma(2 * Q_CHUNK, 0, ns > 1 ? (uint32_t)S_ROW : oob, i);
  wait_vm<Q_DMA>();
  // a use here keeps the first group's scale loads ahead of the DMAs (left
  // to itself, the compiler sinks them to the loop, and the waits it then
  // places at the loop head drain every slice's DMAs)
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(sa8[i]), "+v"(sb8[i]));
  bare_barrier();
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = frag(Q_CHUNK, 0, wt + j * 32 + lrow);
  a0 = frag(0, 0, wn + lrow);

  int base = 0;   // (2d) % 5
  // one slice; PAR = d % 2 (the slice's place in its group of two)
  auto slice = [&](int d, auto par) {
    constexpr int PAR = decltype(par)::value;
    auto slot = [&](int m) { const int v = base + m; return (v >= Q_SLOTS ? v - Q_SLOTS : v) * Q_CHUNK; };
    const int s_a = slot(0), s_b = slot(1), s_a1 = slot(2), s_b1 = slot(3), s_a2 = slot(4);
    const uint32_t kb1 = d + 1 < ns ? (uint32_t)(d + 1) * S_ROW : oob;
    const uint32_t ka2 = d + 2 < ns ? (uint32_t)(d + 2) * S_ROW : oob;
    if (PAR == 0) scales8(min(2 * d + 4, 2 * ns - 4), na8, nb8);   // the last group reloads itself, unused
    // stage 0: B_{d+1}, two DMAs per quarter
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = pick(sa8[i], 2 * PAR);
      sb[i] = pick(sb8[i], 2 * PAR);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_barrier(0);
      dma(s_b1, 1, kb1, 2 * q);
      dma(s_b1, 1, kb1, 2 * q + 1);
      if (q < 3) {
        if (q & 1) a0 = frag(s_a, 0, wn + (q + 1) * 32 + lrow);
        else a1 = frag(s_a, 0, wn + (q + 1) * 32 + lrow);
        mfma_row((q & 1) ? a1 : a0, q);
        SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_DSR, 1); SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_DSR, 1);
        SGB(SG_MFMA, 2);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) nb[j] = frag(s_b, 1, wt + j * 32 + lrow);
        a0 = frag(s_a, 1, wn + lrow);
        mfma_row(a1, 3);
        SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_DSR, 4); SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_DSR, 3);
        SGB(SG_MFMA, 1); SGB(SG_DSR, 3); SGB(SG_MFMA, 1);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = nb[j];
    // stage 1: A_{d+2}, 3 + 3 + 2 DMAs; the barrier after the third row block
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = pick(sa8[i], 2 * PAR + 1);
      sb[i] = pick(sb8[i], 2 * PAR + 1);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      __builtin_amdgcn_sched_barrier(0);
      const int nd = q < 2 ? 3 : 2, d0 = 3 * q;
#pragma unroll
      for (int k = 0; k < nd; ++k) dma(s_a2, 0, ka2, d0 + k);
      if (q & 1) a0 = frag(s_a, 1, wn + (q + 1) * 32 + lrow);
      else a1 = frag(s_a, 1, wn + (q + 1) * 32 + lrow);
      mfma_row((q & 1) ? a1 : a0, q);
      if (nd == 3) {
        SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_DSR, 1); SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_DSR, 1);
        SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_MFMA, 1);
      } else {
        SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_DSR, 1); SGB(SG_MFMA, 1); SGB(SG_VMEM, 1); SGB(SG_DSR, 1);
        SGB(SG_MFMA, 2);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<Q_DMA>();   // all but A_{d+2}'s 8: B_{d+1}, A_{d+1} and the scale loads are in
    wait_lgkm0();
    bare_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) nb[j] = frag(s_b1, 0, wt + j * 32 + lrow);
    a0 = frag(s_a1, 0, wn + lrow);
    mfma_row(a1, 3);
    SGB(SG_MFMA, 1); SGB(SG_DSR, 4); SGB(SG_MFMA, 1); SGB(SG_DSR, 3); SGB(SG_MFMA, 1); SGB(SG_DSR, 3);
    SGB(SG_MFMA, 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = nb[j];
    if (PAR == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa8[i] = na8[i];
        sb8[i] = nb8[i];
      }
    }
    base = base + 2 >= Q_SLOTS ? base + 2 - Q_SLOTS : base + 2;
  };
  for (int d = 0; d < ns; d += 2) {
    slice(d, std::integral_constant<int, 0>{});
    slice(d + 1, std::integral_constant<int, 1>{});
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();   // the zero-fill DMAs of the last slices land before LDS is reused
  store_tile(acc, smem, kv, T, N, t0, n0, wn, wt, lane, wave, ep);
}

hipError_t set_lds(const void* fn, int bytes = LDS_BYTES) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

}  // namespace

hipError_t launch_gemm_bf16(const void* x, int64_t T, int K, const void* w, int N, void* kv,
                            hipStream_t s, const GateEpi& ep) {
  const int tiles_n = (N + BM - 1) / BM;
  const int tiles_t = (int)((T + BN - 1) / BN);
  const dim3 grid(tiles_n * tiles_t), block(THREADS);
  hipError_t e;
  if (K % 64 == 0) {
    if ((e = set_lds((const void*)gemm_bf16_kernel<false>, Q_LDS)) != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_bf16_kernel<false>, grid, block, Q_LDS, s, (const uint16_t*)x, (int)T, K,
                       (const uint16_t*)w, N, (uint16_t*)kv, tiles_n, tiles_t, ep);
  } else {
    if ((e = set_lds((const void*)gemm_bf16_kernel<true>, Q_LDS)) != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_bf16_kernel<true>, grid, block, Q_LDS, s, (const uint16_t*)x, (int)T, K,
                       (const uint16_t*)w, N, (uint16_t*)kv, tiles_n, tiles_t, ep);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_mxfp8(const uint8_t* xq, const uint8_t* xs, int64_t T, int K, const uint8_t* w,
                             const uint8_t* ws, int N, void* kv, hipStream_t s, const GateEpi& ep) {
  const int tiles_n = (N + BM - 1) / BM;
  const int tiles_t = (int)((T + BN - 1) / BN);
  if (K % 256 == 0 && N % 32 == 0) {
    hipError_t e = set_lds((const void*)gemm_mx_ring_kernel, Q_LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_mx_ring_kernel, dim3(tiles_n * tiles_t), dim3(THREADS), Q_LDS, s, xq, xs, (int)T,
                       K, w, ws, N, (uint16_t*)kv, tiles_n, tiles_t, ep);
    return hipGetLastError();
  }
  hipError_t e = set_lds((const void*)gemm_mxfp8_kernel);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_mxfp8_kernel, dim3(tiles_n * tiles_t), dim3(THREADS), LDS_BYTES, s, xq, xs,
                     (int)T, K, w, ws, N, (uint16_t*)kv, tiles_n, tiles_t, ep);
  return hipGetLastError();
}

}  // namespace engram
