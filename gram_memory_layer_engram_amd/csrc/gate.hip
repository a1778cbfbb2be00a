// Gate and residual update: out = hidden + sigmoid(signed-sqrt(d)) * value.
//
// Math: "vllm.models.deepseek_v41.amd.engram", _engram_gate_finish_kernel
// (one shard) together with _engram_gate_partials_kernel, which shows the two
// kv-side sums: sum key^2 and sum hidden*q*k*key over dim; the hidden-side
// sum is sum hidden^2. Per token and copy h:
//   d = dot * rsqrt(hs/dim + eps) * rsqrt(ks/dim + eps) * rsqrt(dim)
//   g = sigmoid(sqrt(max(|d|, clamp)) carrying the sign of d, negative only
//       when d < 0)
//   out = bf16(hidden + g * value); masked tokens copy hidden, g = 0
// ("vllm.models.deepseek_v4_1.common.engram", Engram.forward docstring:
// masked positions pass through untouched).
//
// After the prefill GEMM's gate epilogue the kv-side sums arrive as
// per-tile partials and only the value row is read (launch_gate_parts).
//
// Layout on MI355X: for large T one workgroup per token serves all hc copies,
// so the value row (the last dim-wide block of the kv row) is read once per
// token instead of once per copy; for small T the copies are split over
// workgroups to keep enough of them in flight. Every thread owns CH 16-byte
// pieces of each row; the 3*hc sums are reduced inside each 64-lane wavefront with cross-lane
// shuffles, then across wavefronts through LDS in fixed wave order, so the
// result does not depend on scheduling.
#include "common.h"

namespace engram {

namespace {

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = bf16lo(v.x); f[1] = bf16hi(v.x);
  f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
  f[4] = bf16lo(v.z); f[5] = bf16hi(v.z);
  f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// HC copies per workgroup, CH pieces (8 bf16 each) per thread per row, BS
// threads. A token's hc_total copies are served by hc_total/HC workgroups
// (blockIdx.y picks the group): all of them in one workgroup when T is large
// (the value row is read once per token), one copy per workgroup when T is
// small (more workgroups in flight; the value row then comes from L2).
// PARTS: the kv-side sums arrive as per-256-column-tile partials from the
// prefill GEMM's epilogue (part [hc, T, tiles]) and `kv` is the value
// [T, dim] alone; only the hidden side is summed here.
template <int HC, int CH, int BS, bool PARTS>
__global__ __launch_bounds__(BS) void gate_kernel(
    const uint4* __restrict__ hidden, const uint4* __restrict__ kv,
    const uint4* __restrict__ qw, const uint4* __restrict__ kw,
    const float2* __restrict__ part, int tiles, int T,
    const uint8_t* __restrict__ mask, int hc_total, int dim8, float inv_dim,
    float rsqrt_dim, float eps, float clamp, uint4* __restrict__ out,
    float* __restrict__ gate_out) {
  constexpr int NW = BS / 64;
  constexpr bool KEEP = HC * CH <= 16;  // keep hidden in registers
  __shared__ float red[NW][3 * HC];
  __shared__ float gates[HC];

  const int64_t t = blockIdx.x;
  const int h0 = blockIdx.y * HC;
  const int tid = threadIdx.x;
  const uint4* hrow = hidden + (t * hc_total + h0) * dim8;
  const uint4* kvrow = PARTS ? nullptr : kv + t * (hc_total + 1) * dim8 + h0 * dim8;
  const uint4* vrow = PARTS ? kv + t * dim8 : kv + t * (hc_total + 1) * dim8 + hc_total * dim8;
  qw += h0 * dim8;
  kw += h0 * dim8;
  uint4* orow = out + (t * hc_total + h0) * dim8;
  float* gout = gate_out ? gate_out + t * hc_total + h0 : nullptr;

  if (mask && mask[t] == 0) {
    // Masked token: the gate is shut and the position passes through.
#pragma unroll
    for (int h = 0; h < HC; ++h)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int j = tid + c * BS;
        if (j < dim8) orow[h * dim8 + j] = hrow[h * dim8 + j];
      }
    if (gout && tid < HC) gout[tid] = 0.0f;
    return;
  }

  float hs[HC], ks[HC], dt[HC];
#pragma unroll
  for (int h = 0; h < HC; ++h) hs[h] = ks[h] = dt[h] = 0.0f;

  uint4 hreg[KEEP ? HC : 1][CH];
  uint4 vreg[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j = tid + c * BS;
    vreg[c] = j < dim8 ? vrow[j] : make_uint4(0, 0, 0, 0);
  }
  if constexpr (PARTS) {
    if (tid < tiles) {
#pragma unroll
      for (int h = 0; h < HC; ++h) {
        const float2 p = part[((int64_t)(h0 + h) * T + t) * tiles + tid];
        dt[h] = p.x;
        ks[h] = p.y;
      }
    }
  }

#pragma unroll
  for (int h = 0; h < HC; ++h) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int j = tid + c * BS;
      if (j < dim8) {
        const uint4 hv = hrow[h * dim8 + j];
        if constexpr (KEEP) hreg[h][c] = hv;
        float a[8];
        unpack8(hv, a);
#pragma unroll
        for (int e = 0; e < 8; ++e) hs[h] = fmaf(a[e], a[e], hs[h]);
        if constexpr (!PARTS) {
          const uint4 kv8 = kvrow[h * dim8 + j];
          const uint4 q8 = qw[h * dim8 + j];
          const uint4 k8 = kw[h * dim8 + j];
          float b[8], qf[8], kf[8];
          unpack8(kv8, b);
          unpack8(q8, qf);
          unpack8(k8, kf);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            ks[h] = fmaf(b[e], b[e], ks[h]);
            dt[h] = fmaf(a[e] * qf[e] * kf[e], b[e], dt[h]);
          }
        }
      }
    }
  }

  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    const float s0 = wave_sum(hs[h]);
    const float s1 = wave_sum(ks[h]);
    const float s2 = wave_sum(dt[h]);
    if (lane == 0) {
      red[wave][3 * h + 0] = s0;
      red[wave][3 * h + 1] = s1;
      red[wave][3 * h + 2] = s2;
    }
  }
  __syncthreads();
  if (tid < HC) {
    const int h = tid;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {  // fixed wave order
      s0 += red[w][3 * h + 0];
      s1 += red[w][3 * h + 1];
      s2 += red[w][3 * h + 2];
    }
    const float hidden_rms = 1.0f / sqrtf(s0 * inv_dim + eps);
    const float key_rms = 1.0f / sqrtf(s1 * inv_dim + eps);
    const float d = s2 * hidden_rms * key_rms * rsqrt_dim;
    float s = sqrtf(fmaxf(fabsf(d), clamp));
    s = d < 0.0f ? -s : s;
    const float g = 1.0f / (1.0f + expf(-s));
    gates[h] = g;
    if (gout) gout[h] = g;
  }
  __syncthreads();

#pragma unroll
  for (int h = 0; h < HC; ++h) {
    const float g = gates[h];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int j = tid + c * BS;
      if (j < dim8) {
        uint4 hv;
        if constexpr (KEEP) hv = hreg[h][c];
        else hv = hrow[h * dim8 + j];
        float a[8], v[8];
        unpack8(hv, a);
        unpack8(vreg[c], v);
        uint4 o;
        o.x = cvt_pk_bf16(fmaf(g, v[0], a[0]), fmaf(g, v[1], a[1]));
        o.y = cvt_pk_bf16(fmaf(g, v[2], a[2]), fmaf(g, v[3], a[3]));
        o.z = cvt_pk_bf16(fmaf(g, v[4], a[4]), fmaf(g, v[5], a[5]));
        o.w = cvt_pk_bf16(fmaf(g, v[6], a[6]), fmaf(g, v[7], a[7]));
        orow[h * dim8 + j] = o;
      }
    }
  }
}

// The same gate when each thread owns exactly one 16-byte piece of every row
// (BS == dim/8): no bounds tests, so every load of the workgroup -- the mask
// byte, the value, the hidden and key rows, q, k or the partials -- is issued
// before the first wait. (Behind per-piece bounds tests the compiler waits
// after each group of four loads: eight dependent round trips per token.)
// A masked token still reads its rows and then copies hidden.
template <int HC, int BS, bool PARTS>
__global__ __launch_bounds__(BS) void gate_exact_kernel(
    const uint4* __restrict__ hidden, const uint4* __restrict__ kv,
    const uint4* __restrict__ qw, const uint4* __restrict__ kw,
    const float2* __restrict__ part, int tiles, int T,
    const uint8_t* __restrict__ mask, int hc_total, float inv_dim,
    float rsqrt_dim, float eps, float clamp, uint4* __restrict__ out,
    float* __restrict__ gate_out) {
  constexpr int NW = BS / 64, dim8 = BS;
  __shared__ float red[NW][3 * HC];
  __shared__ float gates[HC];

  const int64_t t = blockIdx.x;
  const int h0 = blockIdx.y * HC;
  const int tid = threadIdx.x;
  const uint4* hrow = hidden + (t * hc_total + h0) * dim8;
  const uint4* kvrow = PARTS ? nullptr : kv + t * (hc_total + 1) * dim8 + h0 * dim8;
  const uint4* vrow = PARTS ? kv + t * dim8 : kv + t * (hc_total + 1) * dim8 + hc_total * dim8;
  uint4* orow = out + (t * hc_total + h0) * dim8;

  const uint4 vv = vrow[tid];
  uint4 hv[HC], k8[HC], qv[HC], kwv[HC];
  float2 p[HC];
#pragma unroll
  for (int h = 0; h < HC; ++h) hv[h] = hrow[h * dim8 + tid];
  if constexpr (!PARTS) {
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      k8[h] = kvrow[h * dim8 + tid];
      qv[h] = qw[(h0 + h) * dim8 + tid];
      kwv[h] = kw[(h0 + h) * dim8 + tid];
    }
  } else {
    const int i = tid < tiles ? tid : 0;
#pragma unroll
    for (int h = 0; h < HC; ++h) p[h] = part[((int64_t)(h0 + h) * T + t) * tiles + i];
  }
  // the mask byte last (without a mask, hidden's first byte, ignored)
  const uint8_t mbyte = *(mask ? mask + t : reinterpret_cast<const uint8_t*>(hrow));
  __builtin_amdgcn_sched_barrier(0);

  float hs[HC], ks[HC], dt[HC];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    float a[8];
    unpack8(hv[h], a);
    hs[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) hs[h] = fmaf(a[e], a[e], hs[h]);
    if constexpr (!PARTS) {
      float b[8], qf[8], kf[8];
      unpack8(k8[h], b);
      unpack8(qv[h], qf);
      unpack8(kwv[h], kf);
      ks[h] = dt[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ks[h] = fmaf(b[e], b[e], ks[h]);
        dt[h] = fmaf(a[e] * qf[e] * kf[e], b[e], dt[h]);
      }
    } else {
      dt[h] = tid < tiles ? p[h].x : 0.f;
      ks[h] = tid < tiles ? p[h].y : 0.f;
    }
  }

  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    const float s0 = wave_sum(hs[h]);
    const float s1 = wave_sum(ks[h]);
    const float s2 = wave_sum(dt[h]);
    if (lane == 0) {
      red[wave][3 * h + 0] = s0;
      red[wave][3 * h + 1] = s1;
      red[wave][3 * h + 2] = s2;
    }
  }
  __syncthreads();
  const bool active = mask == nullptr || mbyte != 0;
  if (tid < HC) {
    const int h = tid;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {  // fixed wave order
      s0 += red[w][3 * h + 0];
      s1 += red[w][3 * h + 1];
      s2 += red[w][3 * h + 2];
    }
    const float hidden_rms = 1.0f / sqrtf(s0 * inv_dim + eps);
    const float key_rms = 1.0f / sqrtf(s1 * inv_dim + eps);
    const float d = s2 * hidden_rms * key_rms * rsqrt_dim;
    float s = sqrtf(fmaxf(fabsf(d), clamp));
    s = d < 0.0f ? -s : s;
    const float g = 1.0f / (1.0f + expf(-s));
    gates[h] = g;
    if (gate_out) gate_out[t * hc_total + h0 + h] = active ? g : 0.0f;
  }
  __syncthreads();

  float v[8];
  unpack8(vv, v);
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    const float g = gates[h];
    float a[8];
    unpack8(hv[h], a);
    uint4 o;
    o.x = cvt_pk_bf16(fmaf(g, v[0], a[0]), fmaf(g, v[1], a[1]));
    o.y = cvt_pk_bf16(fmaf(g, v[2], a[2]), fmaf(g, v[3], a[3]));
    o.z = cvt_pk_bf16(fmaf(g, v[4], a[4]), fmaf(g, v[5], a[5]));
    o.w = cvt_pk_bf16(fmaf(g, v[6], a[6]), fmaf(g, v[7], a[7]));
    if (!active) o = hv[h];   // masked: hidden, bit for bit
    orow[h * dim8 + tid] = o;
  }
}

struct GateCall {
  const void* hidden; const void* kv; const void* q; const void* k;
  const float2* part; int tiles;
  const uint8_t* mask; int64_t T; int hc_total; int dim; float eps, clamp;
  void* out; float* gate_out;
};

template <int HC, int CH, int BS, bool PARTS>
hipError_t launch_t(const GateCall& g, hipStream_t s) {
  hipLaunchKernelGGL((gate_kernel<HC, CH, BS, PARTS>), dim3((unsigned)g.T, g.hc_total / HC), dim3(BS), 0, s,
                     (const uint4*)g.hidden, (const uint4*)g.kv, (const uint4*)g.q, (const uint4*)g.k,
                     g.part, g.tiles, (int)g.T, g.mask, g.hc_total, g.dim / 8, 1.0f / (float)g.dim,
                     1.0f / sqrtf((float)g.dim), g.eps, g.clamp, (uint4*)g.out, g.gate_out);
  return hipGetLastError();
}

template <int HC, int BS, bool PARTS>
hipError_t launch_exact(const GateCall& g, hipStream_t s) {
  hipLaunchKernelGGL((gate_exact_kernel<HC, BS, PARTS>), dim3((unsigned)g.T, g.hc_total / HC), dim3(BS), 0, s,
                     (const uint4*)g.hidden, (const uint4*)g.kv, (const uint4*)g.q, (const uint4*)g.k,
                     g.part, g.tiles, (int)g.T, g.mask, g.hc_total, 1.0f / (float)g.dim,
                     1.0f / sqrtf((float)g.dim), g.eps, g.clamp, (uint4*)g.out, g.gate_out);
  return hipGetLastError();
}

template <int HC, bool PARTS>
hipError_t launch_hc(const GateCall& g, hipStream_t s) {
  const int dim8 = g.dim / 8;
  // one piece per thread when dim/8 is a multiple of 128 up to 1024 and the
  // rows of HC copies fit in registers (4*HC + 1 pieces, or HC + 1 with
  // partials, under the 128 VGPRs of a 1024-thread workgroup)
  if constexpr (PARTS || 4 * HC + 1 <= 24) {
    switch (dim8) {
      case 128: return launch_exact<HC, 128, PARTS>(g, s);
      case 256: return launch_exact<HC, 256, PARTS>(g, s);
      case 384: return launch_exact<HC, 384, PARTS>(g, s);
      case 512: return launch_exact<HC, 512, PARTS>(g, s);
      case 640: return launch_exact<HC, 640, PARTS>(g, s);
      case 768: return launch_exact<HC, 768, PARTS>(g, s);
      case 896: return launch_exact<HC, 896, PARTS>(g, s);
      case 1024: return launch_exact<HC, 1024, PARTS>(g, s);
      default: break;
    }
  }
  if (dim8 <= 64) return launch_t<HC, 1, 64, PARTS>(g, s);
  if (dim8 <= 128) return launch_t<HC, 1, 128, PARTS>(g, s);
  const int ch = (dim8 + 255) / 256;
  switch (ch) {
    case 1: return launch_t<HC, 1, 256, PARTS>(g, s);
    case 2: return launch_t<HC, 2, 256, PARTS>(g, s);
    case 3: return launch_t<HC, 3, 256, PARTS>(g, s);
    case 4: return launch_t<HC, 4, 256, PARTS>(g, s);
    case 5: return launch_t<HC, 5, 256, PARTS>(g, s);
    case 6: return launch_t<HC, 6, 256, PARTS>(g, s);
    case 7: return launch_t<HC, 7, 256, PARTS>(g, s);
    case 8: return launch_t<HC, 8, 256, PARTS>(g, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool PARTS>
hipError_t dispatch(const GateCall& g, hipStream_t s) {
  // Few tokens: one copy per workgroup, so T*hc workgroups share the work.
  if (g.T * 2 < dev_info().num_cus && g.hc_total > 1) return launch_hc<1, PARTS>(g, s);
  switch (g.hc_total) {
    case 1: return launch_hc<1, PARTS>(g, s);
    case 2: return launch_hc<2, PARTS>(g, s);
    case 3: return launch_hc<3, PARTS>(g, s);
    case 4: return launch_hc<4, PARTS>(g, s);
    case 5: return launch_hc<5, PARTS>(g, s);
    case 6: return launch_hc<6, PARTS>(g, s);
    case 7: return launch_hc<7, PARTS>(g, s);
    case 8: return launch_hc<8, PARTS>(g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gate(const void* hidden, const void* kv, const void* q,
                       const void* k, const uint8_t* mask, int64_t T, int hc,
                       int dim, float eps, float clamp, void* out,
                       float* gate_out, hipStream_t s) {
  const GateCall g{hidden, kv, q, k, nullptr, 0, mask, T, hc, dim, eps, clamp, out, gate_out};
  return dispatch<false>(g, s);
}

hipError_t launch_gate_parts(const void* hidden, const void* value, const float2* part,
                             const uint8_t* mask, int64_t T, int hc, int dim, float eps,
                             float clamp, void* out, float* gate_out, hipStream_t s) {
  const GateCall g{hidden, value, hidden, hidden, part, dim / 256, mask, T, hc, dim, eps, clamp, out, gate_out};
  return dispatch<true>(g, s);
}

}  // namespace engram
