// Router: logits = W_r x in fp32, softmax over all experts in fp32, top-K
// (by logit, equal logits: lower expert index first), renormalised weights (model API page,
// build_moe_config; the gate kept in fp32 per the model-coverage page,
// "Train", and 'mlp.gate' in _keep_in_fp32_modules_strict).
//
// bf16 activations: the fp32 router weight is split once per call into three
// bf16 terms hi + mid + lo that sum to it exactly (Henry, Tang & Heinecke,
// "Leveraging the bfloat16 Artificial Intelligence Datatype for
// Higher-Precision Computations", ARITH 2019). Each product x*term is exact
// in fp32, so bf16 MFMA with fp32 accumulation gives the fp32 router at
// matrix-core rate instead of the vector-FMA rate.
//
// The same kernel also builds the per-block expert histogram that the
// stable counting sort scans (block b covers tokens [32b, 32b + 32)).
#include "common.h"

namespace hi3 {

// --------------------------------------------------------------- weight split

__global__ __launch_bounds__(256) void split_router_kernel(const float *__restrict__ wr,
                                                           uint16_t *__restrict__ ws,
                                                           int E, int Epad, int H) {
  const int64_t n = static_cast<int64_t>(Epad) * H;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int e = static_cast<int>(i / H);
  const float v = e < E ? wr[i] : 0.0f;
  // Truncating to the top 8 significand bits leaves an exact remainder.
  const uint32_t hi = __float_as_uint(v) & 0xFFFF0000u;
  const float r1 = v - __uint_as_float(hi);
  const uint32_t mid = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mid);
  ws[i] = static_cast<uint16_t>(hi >> 16);
  ws[n + i] = static_cast<uint16_t>(mid >> 16);
  ws[2 * n + i] = f32_to_bf16(r2);  // at most 8 significant bits: exact
}

hipError_t launch_split_router(const float *w_router, uint16_t *wsplit, int E, int Epad,
                               int H, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(Epad) * H;
  hipLaunchKernelGGL(split_router_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, w_router, wsplit, E, Epad, H);
  return hipGetLastError();
}

// --------------------------------------------------------------- selection

struct RouterShared {
  float logit[kRouterTB][kMaxE + 1];
  uint64_t selmask[kRouterTB];
};

// Softmax over all experts, top-K, renormalisation for the token in
// LDS row rr; one wavefront, lane = expert. Writes the routes and the
// selection bitmask.
__device__ void select_row(const RouterArgs &a, RouterShared &sh, int rr, int lane,
                           int64_t t) {
  const bool is_pad = a.pad && a.pad[t];
  if (is_pad) {
    if (lane < a.K) {
      a.idx[t * a.K + lane] = -1;
      a.wts[t * a.K + lane] = 0.0f;
    }
    if (lane == 0) sh.selmask[rr] = 0;
    return;
  }
  const bool live = lane < a.E;
  const float l = live ? sh.logit[rr][lane] : -INFINITY;
  const float m = wave_max(l);
  const float ex = live ? expf(l - m) : 0.0f;
  const float z = wave_sum_uniform(ex);
  const float p = ex / z;
  // Top-K is taken on the logits: softmax is strictly increasing, so this is
  // the exact order of the probabilities, and it does not depend on which
  // small probabilities underflow in fp32. Equal logits: lower index first.
  bool avail = live;
  int my_e = -1;
  float my_p = 0.0f;
  float s = 0.0f;
  uint64_t mask = 0;
  for (int k = 0; k < a.K; ++k) {
    float bv = avail ? l : -INFINITY;
    int be = avail ? lane : 0x7fffffff;
    wave_argmax(bv, be);
    const float pb = __shfl(p, be, kWave);
    if (lane == k) {
      my_e = be;
      my_p = pb;
    }
    if (lane == be) avail = false;
    s += pb;  // in k order
    mask |= 1ull << be;
  }
  if (lane < a.K) {
    a.idx[t * a.K + lane] = my_e;
    a.wts[t * a.K + lane] = my_p / s;
  }
  if (lane == 0) sh.selmask[rr] = mask;
}

// Per-block histogram of selected experts and count of real rows.
__device__ void block_histogram(const RouterArgs &a, RouterShared &sh, int64_t t0) {
  const int tid = threadIdx.x;
  if (tid < a.E) {
    int c = 0;
    for (int rr = 0; rr < kRouterTB; ++rr) c += static_cast<int>((sh.selmask[rr] >> tid) & 1u);
    a.blkcnt[static_cast<int64_t>(blockIdx.x) * a.E + tid] = c;
  }
  if (tid == 64) {
    int c = 0;
    for (int rr = 0; rr < kRouterTB; ++rr) {
      const int64_t t = t0 + rr;
      c += (t < a.T && !(a.pad && a.pad[t])) ? 1 : 0;
    }
    a.blkval[blockIdx.x] = c;
  }
}

// --------------------------------------------------------------- bf16 router

// 256 threads = 4 waves; block covers 32 tokens; wave w accumulates the
// 64-wide k chunks c = w, w+4, ... of all 32 tokens x Epad experts with
// v_mfma_f32_32x32x16_bf16, then the 4 partial logit tiles are summed in a
// fixed order in LDS.
//
// MFMA operand layout used here (32x32x16): lane l supplies row (l % 32) of
// A and column (l % 32) of B, and 8 consecutive k values; lanes 0-31 and
// 32-63 cover two disjoint k groups. Any k assignment is valid as long as A
// and B agree, so within a 64-wide chunk lane half g takes k in
// [32g, 32g + 32) and MFMA q uses its elements [8q, 8q + 8): each lane reads
// 64 contiguous bytes per operand row. Result element v of lane l is
// row 8*(v/4) + 4*(l/32) + v%4, column l%32.
template <int NS>
__global__ __launch_bounds__(256) void router_bf16_kernel(RouterArgs a) {
  __shared__ float part[4][kRouterTB][NS * 32 + 1];
  __shared__ RouterShared sh;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 31;
  const int g = lane >> 5;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouterTB;
  const int64_t t = t0 + r;
  const bool row_ok = t < a.T && !(a.pad && a.pad[t]);
  const uint16_t *x = static_cast<const uint16_t *>(a.x);
  const uint16_t *xrow = x + (row_ok ? t : 0) * static_cast<int64_t>(a.H);
  const int64_t plane = static_cast<int64_t>(a.Epad) * a.H;

  f32x16_t acc_hi[NS], acc_lo[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      acc_hi[n][v] = 0.0f;
      acc_lo[n][v] = 0.0f;
    }

  const int nchunks = a.H / 64;
  for (int c = wave; c < nchunks; c += 4) {
    const int k0 = c * 64 + g * 32;
    u32x4_t av[4];
    if (row_ok) {
      const u32x4_t *p = reinterpret_cast<const u32x4_t *>(xrow + k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) av[q] = p[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) av[q] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int n = 0; n < NS; ++n) {
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) {
        const u32x4_t *p = reinterpret_cast<const u32x4_t *>(
            a.wsplit + sp * plane + static_cast<int64_t>(n * 32 + r) * a.H + k0);
        u32x4_t bv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) bv[q] = p[q];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x8_t A = __builtin_bit_cast(bf16x8_t, av[q]);
          const bf16x8_t B = __builtin_bit_cast(bf16x8_t, bv[q]);
          if (sp == 0)
            acc_hi[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc_hi[n], 0, 0, 0);
          else
            acc_lo[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc_lo[n], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NS; ++n)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      part[wave][(v >> 2) * 8 + g * 4 + (v & 3)][n * 32 + r] = acc_hi[n][v] + acc_lo[n][v];
  __syncthreads();
  for (int i = threadIdx.x; i < kRouterTB * a.E; i += blockDim.x) {
    const int rr = i / a.E, e = i % a.E;
    sh.logit[rr][e] = ((part[0][rr][e] + part[1][rr][e]) + part[2][rr][e]) + part[3][rr][e];
  }
  __syncthreads();
  for (int rr = wave; rr < kRouterTB; rr += 4) {
    const int64_t tt = t0 + rr;
    if (tt >= a.T) {
      if (lane == 0) sh.selmask[rr] = 0;
      continue;
    }
    select_row(a, sh, rr, lane, tt);
  }
  __syncthreads();
  block_histogram(a, sh, t0);
}

// --------------------------------------------------------------- fp32 router

// fp32 activations: plain fp32 FMA dot products (lane = expert, one token
// per wave at a time); used for the small fp32 layers.
__global__ __launch_bounds__(256) void router_f32_kernel(RouterArgs a) {
  __shared__ RouterShared sh;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouterTB;
  const float *x = static_cast<const float *>(a.x);
  for (int rr = wave; rr < kRouterTB; rr += 4) {
    const int64_t t = t0 + rr;
    if (t >= a.T || (a.pad && a.pad[t])) continue;
    if (lane < a.E) {
      const float *xr = x + t * a.H;
      const float *wrow = a.w_router + static_cast<int64_t>(lane) * a.H;
      float acc = 0.0f;
      for (int h = 0; h < a.H; ++h) acc = fmaf(xr[h], wrow[h], acc);
      sh.logit[rr][lane] = acc;
    }
  }
  __syncthreads();
  for (int rr = wave; rr < kRouterTB; rr += 4) {
    const int64_t tt = t0 + rr;
    if (tt >= a.T) {
      if (lane == 0) sh.selmask[rr] = 0;
      continue;
    }
    select_row(a, sh, rr, lane, tt);
  }
  __syncthreads();
  block_histogram(a, sh, t0);
}

hipError_t launch_router(const RouterArgs &a, int dtype, hipStream_t s) {
  const int nb = static_cast<int>((a.T + kRouterTB - 1) / kRouterTB);
  if (dtype == kF32) {
    hipLaunchKernelGGL(router_f32_kernel, dim3(nb), dim3(256), 0, s, a);
  } else if (a.Epad <= 32) {
    hipLaunchKernelGGL(router_bf16_kernel<1>, dim3(nb), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(router_bf16_kernel<2>, dim3(nb), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// --------------------------------------------------------------- histogram

// Histogram of given routes (dispatch without the router): same blocking and
// the same selection-bitmask rule as the router's fused histogram. Ids outside
// [0, E) are ignored.
__global__ __launch_bounds__(256) void histogram_kernel(const int32_t *__restrict__ idx,
                                                        const uint8_t *__restrict__ pad,
                                                        int64_t T, int E, int K,
                                                        int32_t *__restrict__ blkcnt,
                                                        int32_t *__restrict__ blkval) {
  __shared__ uint64_t selmask[kRouterTB];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouterTB;
  const int tid = threadIdx.x;
  if (tid < kRouterTB) {
    const int64_t t = t0 + tid;
    uint64_t m = 0;
    if (t < T && !(pad && pad[t])) {
      for (int k = 0; k < K; ++k) {
        const int e = idx[t * K + k];
        if (e >= 0 && e < E) m |= 1ull << e;
      }
    }
    selmask[tid] = m;
  }
  __syncthreads();
  if (tid < E) {
    int c = 0;
    for (int rr = 0; rr < kRouterTB; ++rr) c += static_cast<int>((selmask[rr] >> tid) & 1u);
    blkcnt[static_cast<int64_t>(blockIdx.x) * E + tid] = c;
  }
  if (tid == 64) {
    int c = 0;
    for (int rr = 0; rr < kRouterTB; ++rr) {
      const int64_t t = t0 + rr;
      c += (t < T && !(pad && pad[t])) ? 1 : 0;
    }
    blkval[blockIdx.x] = c;
  }
}

hipError_t launch_histogram(const int32_t *idx, const uint8_t *pad, int64_t T, int E,
                            int K, int32_t *blkcnt, int32_t *blkval, hipStream_t s) {
  const int nb = static_cast<int>((T + kRouterTB - 1) / kRouterTB);
  hipLaunchKernelGGL(histogram_kernel, dim3(nb), dim3(256), 0, s, idx, pad, T, E, K,
                     blkcnt, blkval);
  return hipGetLastError();
}

}  // namespace hi3
