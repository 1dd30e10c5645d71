// Router: logits = W_r x in fp32, softmax over all experts in fp32, top-K
// (by logit, equal logits: lower expert index first), renormalised weights (model API page,
// build_moe_config; the gate kept in fp32 per the model-coverage page,
// "Train", and 'mlp.gate' in _keep_in_fp32_modules_strict).
//
// bf16 activations: the fp32 router weight is split once per call into three
// bf16 terms hi + mid + lo that sum to it exactly (Henry, Tang & Heinecke,
// "Leveraging the bfloat16 Artificial Intelligence Datatype for
// Higher-Precision Computations", ARITH 2019), stored in MFMA-fragment order
// so every fragment load is one contiguous 1 KiB per wave. Each product
// x*term is exact in fp32, so bf16 MFMA with fp32 accumulation gives the fp32
// router at matrix-core rate instead of the vector-FMA rate.
//
// The selection kernel also builds the per-block expert histogram that the
// stable counting sort scans (block b covers tokens [32b, 32b + 32)).
#include <algorithm>

#include "common.h"

namespace hi3 {

// --------------------------------------------------------------- weight split

// Output layout ("fragment order"): for split term sp, 32-expert column
// tile n, 64-wide k chunk c and MFMA step q, the 64 lanes' 8-element pieces
// lie next to each other (lane = 32 g + r holds expert 32 n + r, k =
// 64 c + 32 g + 8 q + [0, 8)), so the router reads each B fragment as one
// contiguous 1 KiB block.
__device__ __forceinline__ int64_t wsplit_index(int sp, int e, int h, int ns, int nchunks) {
  const int n = e >> 5, r = e & 31;
  const int c = h >> 6, w = h & 63;
  const int g = w >> 5, q = (w & 31) >> 3, j = w & 7;
  const int lane = g * 32 + r;
  return ((((static_cast<int64_t>(sp) * ns + n) * nchunks + c) * 4 + q) * 64 + lane) * 8 + j;
}

__global__ __launch_bounds__(256) void split_router_kernel(const float *__restrict__ wr,
                                                           uint16_t *__restrict__ ws,
                                                           int E, int Epad, int H) {
  const int64_t n = static_cast<int64_t>(Epad) * H;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int e = static_cast<int>(i / H);
  const int h = static_cast<int>(i % H);
  const float v = e < E ? wr[i] : 0.0f;
  // Truncating to the top 8 significand bits leaves an exact remainder.
  const uint32_t hi = __float_as_uint(v) & 0xFFFF0000u;
  const float r1 = v - __uint_as_float(hi);
  const uint32_t mid = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mid);
  const int ns = Epad / 32, nchunks = H / 64;
  ws[wsplit_index(0, e, h, ns, nchunks)] = static_cast<uint16_t>(hi >> 16);
  ws[wsplit_index(1, e, h, ns, nchunks)] = static_cast<uint16_t>(mid >> 16);
  ws[wsplit_index(2, e, h, ns, nchunks)] = f32_to_bf16(r2);  // at most 8 significant bits: exact
}


// --------------------------------------------------------------- selection

// Softmax over all experts, top-K and renormalisation for 32 tokens per
// block: 8 waves, one token per wave at a time, lane = expert; then the
// block's expert histogram and real-row count.
// The token's logits are the slice partials summed in slice order. Every
// lane reads all of the token's logits from the other lanes (readlane, in
// expert order) to get the maximum and its own rank in the selection order
// (larger logit first, lower index first on equal logits; softmax is
// strictly increasing, so this is the order of the probabilities, and fp32
// underflow of small probabilities cannot change it). Z sums exp(l - max) in
// ascending expert order, the selected p = exp(l - max) / Z are summed in
// selection order, and each is divided by that sum.
// partial: [slices][T][E] fp32. EC = 64: E is 64 (no per-expert guards);
// EC = 0: any E <= 64.
#ifndef HI3_SEL_THREADS
#define HI3_SEL_THREADS 1024
#endif
// threads of the selection kernel (kRouterTB / (threads / 64) tokens per wave)
constexpr int kSelThreads = HI3_SEL_THREADS;
struct SelectShared {
  float psel[kRouterTB][kMaxE];
  int esel[kRouterTB][kMaxE];
  uint64_t selmask[kRouterTB];
};

__device__ __forceinline__ float nan_as_neg_inf(float v) { return v != v ? -INFINITY : v; }

// Orders this wave's LDS writes before its following LDS reads: LDS
// operations of one wave complete in order, so waiting for the wave's own
// LDS counter is enough (a memory fence would also wait for the wave's
// global stores).
__device__ __forceinline__ void wave_lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int EC>
__global__ __launch_bounds__(kSelThreads) void router_select_kernel(RouterArgs a,
                                                                   const float *partial,
                                                            int slices) {
  __shared__ SelectShared sh;
  const int E = EC > 0 ? EC : a.E;
  const int K = a.K;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouterTB;

  // logits of the wave's tokens: lane e sums partial[ks][t][e] over the
  // slices in slice order (one coalesced 256-byte row per slice); all of the
  // wave's loads are issued before the first sum
  constexpr int TPW = kRouterTB / (kSelThreads / 64);  // tokens per wave
  float lsum[TPW];
  {
    float v[TPW][kRouterMaxSlices];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int64_t t = t0 + wave + (kSelThreads / 64) * j;
      const int64_t tc = t < a.T ? t : a.T - 1;
      const int ec = lane < E ? lane : E - 1;
#pragma unroll
      for (int ks = 0; ks < kRouterMaxSlices; ++ks)
        if (ks < slices) v[j][ks] = partial[(static_cast<int64_t>(ks) * a.T + tc) * E + ec];
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      float l = 0.0f;
#pragma unroll
      for (int ks = 0; ks < kRouterMaxSlices; ++ks)
        if (ks < slices) l += v[j][ks];
      lsum[j] = l;
    }
  }

#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int rr = wave + (kSelThreads / 64) * j;
    const int64_t t = t0 + rr;
    if (t >= a.T) {
      if (lane == 0) sh.selmask[rr] = 0;
      continue;
    }
    if (a.pad && a.pad[t]) {
      if (lane < K) {
        a.idx[t * K + lane] = -1;
        a.wts[t * K + lane] = 0.0f;
      }
      if (lane == 0) sh.selmask[rr] = 0;
      continue;
    }
    // A NaN logit counts as -infinity: the order (larger first, lower index
    // on equal values) is then total, the ranks of the E lanes are a
    // permutation, and exactly K experts are selected whatever the inputs.
    // Every lane walks the row's logits in expert order (readlane: no
    // memory round trips) for the maximum, its own rank in the selection
    // order and the softmax denominator, summed in ascending expert order.
    const bool live = lane < E;
    const float l = live ? nan_as_neg_inf(lsum[j]) : -INFINITY;
    float m = -INFINITY;
    int rank = 0;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      if (EC == 0 && e >= E) continue;  // (wave-uniform)
      const float ve = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), e));
      m = fmaxf(m, ve);
      rank += (ve > l || (ve == l && e < lane)) ? 1 : 0;
    }
    const float ex = live ? expf(l - m) : 0.0f;
    float z = 0.0f;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      if (EC == 0 && e >= E) continue;
      z += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), e));
    }
    const float p = ex / z;
    const bool sel = live && rank < K;
    if (sel) {
      sh.psel[rr][rank] = p;
      sh.esel[rr][rank] = lane;
    }
    const uint64_t mask = __ballot(sel);
    wave_lds_sync();
    // the selected probabilities summed in selection order
    float ssum = 0.0f;
    for (int k = 0; k < K; ++k) ssum += sh.psel[rr][k];
    if (lane < K) {
      a.idx[t * K + lane] = sh.esel[rr][lane];
      a.wts[t * K + lane] = sh.psel[rr][lane] / ssum;
    }
    if (lane == 0) sh.selmask[rr] = mask;
  }
  __syncthreads();

  const int tid = threadIdx.x;
  if (tid < E) {
    int c = 0;
    for (int rr = 0; rr < kRouterTB; ++rr) c += static_cast<int>((sh.selmask[rr] >> tid) & 1u);
    a.blkcnt[static_cast<int64_t>(blockIdx.x) * E + tid] = c;
  }
  if (tid >= 64 && tid < 64 + kRouterTB) {
    const int rr = tid - 64;
    const int64_t t = t0 + rr;
    const bool ok = t < a.T && !(a.pad && a.pad[t]);
    const uint64_t bal = __ballot(ok);
    if (rr == 0) a.blkval[blockIdx.x] = __popcll(bal);
  }
}

// --------------------------------------------------------------- bf16 router

// Partial logits of kRouterMT tokens over one slice of the hidden
// dimension. Grid: x = blocks of kRouterMT tokens, y = k slices (ranges of
// 64-wide chunks). 256 threads = 4 waves; wave w takes the chunks
// first + w, first + w + 4, ... of the slice for all kRouterMT / 32 token
// tiles, so each router-weight fragment it loads (and splits) serves every
// token tile of the block. The 4 waves' sums are added in a fixed order in
// LDS and written to partial[slice][t][e].
//
// MFMA operand layout (v_mfma_f32_32x32x16_bf16): lane l supplies row
// (l % 32) of A and column (l % 32) of B, and 8 consecutive k values; lanes
// 0-31 and 32-63 cover two disjoint k groups. Any k assignment is valid as
// long as A and B agree: within a 64-wide chunk lane half g takes k in
// [32g, 32g + 32) and step q uses its elements [8q, 8q + 8), so each lane
// reads 64 contiguous bytes of x and 128 of the weight row per chunk.
// Result element v of lane l is token 8 (v / 4) + 4 (l / 32) + v % 4 of the
// tile and expert l % 32 of the column tile. The three terms of a weight go
// into the same accumulator, hi first; the next chunk's operands are loaded
// while the current chunk is multiplied.
template <int NS>
__global__ __launch_bounds__(256) void router_logits_kernel(RouterArgs a, float *partial,
                                                            int chunks_per_slice) {
  constexpr int TT = kRouterMT / 32;  // token tiles per block
  __shared__ float part[4][kRouterMT][NS * 32 + 1];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 31;
  const int g = lane >> 5;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouterMT;
  const uint16_t *x = static_cast<const uint16_t *>(a.x);
  const int nchunks = a.H / 64;

  const uint16_t *xrow[TT];
  bool row_ok[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int64_t t = t0 + tt * 32 + r;
    row_ok[tt] = t < a.T && !(a.pad && a.pad[t]);
    xrow[tt] = x + (row_ok[tt] ? t : 0) * static_cast<int64_t>(a.H);
  }

  f32x16_t acc[TT][NS];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int n = 0; n < NS; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[tt][n][v] = 0.0f;

  const int c_first = blockIdx.y * chunks_per_slice;
  const int c_end = min(nchunks, c_first + chunks_per_slice);
  // operands of one chunk: the split weights' fragments and the token rows
  u32x4_t wv[NS][3][4];
  u32x4_t xv[TT][4];
  auto load = [&](int c) __attribute__((always_inline)) {
    const int k0 = c * 64 + g * 32;
#pragma unroll
    for (int n = 0; n < NS; ++n)
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) {
        // fragment order: the 4 steps' 1 KiB blocks of (sp, n, c) are adjacent
        const u32x4_t *p = reinterpret_cast<const u32x4_t *>(a.wsplit) +
                           (((static_cast<int64_t>(sp) * NS + n) * nchunks + c) * 4) * 64 + lane;
#pragma unroll
        for (int q = 0; q < 4; ++q) wv[n][sp][q] = p[q * 64];
      }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const u32x4_t *p = reinterpret_cast<const u32x4_t *>(xrow[tt] + k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[tt][q] = row_ok[tt] ? p[q] : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  int c = c_first + wave;
  if (c < c_end) load(c);
  for (; c < c_end; c += 4) {
    // keep this chunk's operands, then request the next chunk's before the
    // MFMAs
    u32x4_t bw[NS][3][4];
    u32x4_t av[TT][4];
#pragma unroll
    for (int n = 0; n < NS; ++n)
#pragma unroll
      for (int sp = 0; sp < 3; ++sp)
#pragma unroll
        for (int q = 0; q < 4; ++q) bw[n][sp][q] = wv[n][sp][q];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int q = 0; q < 4; ++q) av[tt][q] = xv[tt][q];
    if (c + 4 < c_end) load(c + 4);
    // consecutive MFMAs update different accumulators (TT x NS of them)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int sp = 0; sp < 3; ++sp)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int n = 0; n < NS; ++n)
            acc[tt][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, av[tt][q]),
                __builtin_bit_cast(bf16x8_t, bw[n][sp][q]), acc[tt][n], 0, 0, 0);
  }
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int n = 0; n < NS; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        part[wave][tt * 32 + (v >> 2) * 8 + g * 4 + (v & 3)][n * 32 + r] = acc[tt][n][v];
  __syncthreads();
  float *out = partial + static_cast<int64_t>(blockIdx.y) * a.E * a.T;
  for (int i = threadIdx.x; i < kRouterMT * a.E; i += blockDim.x) {
    const int rr = i / a.E, e = i % a.E;
    const int64_t t = t0 + rr;
    if (t < a.T)
      out[t * a.E + e] = ((part[0][rr][e] + part[1][rr][e]) + part[2][rr][e]) + part[3][rr][e];
  }
}

int router_slices(int64_t T, int H) {
  const int nb = static_cast<int>((T + kRouterMT - 1) / kRouterMT);
  // one block per CU (the block's LDS allows no second one): at most 256
  // blocks, so none waits for a second round; at least 4 chunks (one per
  // wave) per slice
  const int max_slices = std::max(1, std::min(kRouterMaxSlices, H / 256));
  const int want = 256 / nb;
  return std::max(1, std::min(max_slices, want));
}

// --------------------------------------------------------------- fp32 router

// fp32 activations: plain fp32 FMA dot products (lane = expert, one token
// per wave at a time), written as a single slice of partial logits for the
// selection kernel; used for the small fp32 layers.
__global__ __launch_bounds__(256) void router_f32_kernel(RouterArgs a, float *partial) {
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
      partial[t * a.E + lane] = acc;
    }
  }
}

hipError_t launch_router(const RouterArgs &a, int dtype, float *partial, hipStream_t s) {
  const int nb = static_cast<int>((a.T + kRouterTB - 1) / kRouterTB);
  int slices = 1;
  if (dtype == kF32) {
    hipLaunchKernelGGL(router_f32_kernel, dim3(nb), dim3(256), 0, s, a, partial);
  } else {
    const int64_t nw = static_cast<int64_t>(a.Epad) * a.H;
    hipLaunchKernelGGL(split_router_kernel, dim3(static_cast<unsigned>((nw + 255) / 256)),
                       dim3(256), 0, s, a.w_router, a.wsplit, a.E, a.Epad, a.H);
    slices = router_slices(a.T, a.H);
    const int cps = (a.H / 64 + slices - 1) / slices;
    const dim3 grid(static_cast<unsigned>((a.T + kRouterMT - 1) / kRouterMT), slices);
    if (a.Epad <= 32)
      hipLaunchKernelGGL(router_logits_kernel<1>, grid, dim3(256), 0, s, a, partial, cps);
    else
      hipLaunchKernelGGL(router_logits_kernel<2>, grid, dim3(256), 0, s, a, partial, cps);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.E == kMaxE)
    hipLaunchKernelGGL(router_select_kernel<kMaxE>, dim3(nb), dim3(kSelThreads), 0, s, a, partial,
                       slices);
  else
    hipLaunchKernelGGL(router_select_kernel<0>, dim3(nb), dim3(kSelThreads), 0, s, a, partial,
                       slices);
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
