// Router: logits = W_r x in fp32, softmax over all experts in fp32, top-K
// (by logit, equal logits: lower expert index first), renormalised weights (model API page,
// build_moe_config; the gate kept in fp32 per the model-coverage page,
// "Train", and 'mlp.gate' in _keep_in_fp32_modules_strict).
//
// bf16 activations: each fp32 router weight is split, in registers, into
// three bf16 terms hi + mid + lo that sum to it exactly (Henry, Tang &
// Heinecke, "Leveraging the bfloat16 Artificial Intelligence Datatype for
// Higher-Precision Computations", ARITH 2019). Each product x * term is exact
// in fp32, so bf16 MFMA with fp32 accumulation gives the fp32 router at
// matrix-core rate instead of the vector-FMA rate. When the layer runs inside
// its decoder block, the block's RMSNorm (layers API page, HunyuanRMSNorm;
// model API page, HunyuanImage3Block: post_attention_layernorm ahead of the
// experts) is computed by the same kernel, which writes the normalised rows
// once for the expert GEMMs and multiplies them in place.
//
// The selection kernel also builds the per-block expert histogram that the
// stable counting sort scans (block b covers tokens [32b, 32b + 32)).
#include <algorithm>

#include "common.h"

namespace hi3 {

// --------------------------------------------------------------- selection

// Softmax over all experts, top-K and renormalisation for 32 tokens per
// block: one wave per token at a time, lane = expert; then the block's
// expert histogram and real-row count.
// Every lane reads all of the token's logits from the other lanes
// (readlane, in expert order) to get the maximum and its own rank in the
// selection order (larger logit first, lower index first on equal logits;
// softmax is strictly increasing, so this is the order of the
// probabilities, and fp32 underflow of small probabilities cannot change
// it). Z sums exp(l - max) in ascending expert order, the selected
// p = exp(l - max) / Z are summed in selection order, and each is divided by
// that sum.
// The token's logits are the slice partials summed in slice order.
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
  float row[kSelThreads / 64][kMaxE];  // one token's values, broadcast to its wave
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
  // slices in slice order (one coalesced row per slice); all of the wave's
  // loads are issued before the first sum
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
    // Every lane reads the row's logits (written to LDS once, read back as
    // broadcasts) in expert order for the maximum, its own rank in the
    // selection order and the softmax denominator, summed in ascending
    // expert order (every lane forms the same sum).
    const bool live = lane < E;
    const float l = live ? nan_as_neg_inf(lsum[j]) : -INFINITY;
    const f32x4_t *rowv = reinterpret_cast<const f32x4_t *>(sh.row[wave]);
    sh.row[wave][lane] = l;
    wave_lds_sync();
    float m = -INFINITY;
    int rank = 0;
#pragma unroll
    for (int e4 = 0; e4 < kMaxE / 4; ++e4) {
      const f32x4_t v4 = rowv[e4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = 4 * e4 + u;
        if (EC == 0 && e >= E) continue;
        const float ve = v4[u];
        m = fmaxf(m, ve);
        rank += (ve > l || (ve == l && e < lane)) ? 1 : 0;
      }
    }
    const float ex = live ? expf(l - m) : 0.0f;
    wave_lds_sync();  // every lane has read the logits before they are overwritten
    sh.row[wave][lane] = ex;
    wave_lds_sync();
    float z = 0.0f;
#pragma unroll
    for (int e4 = 0; e4 < kMaxE / 4; ++e4) {
      const f32x4_t v4 = rowv[e4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (EC == 0 && 4 * e4 + u >= E) continue;
        z += v4[u];
      }
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

// The three bf16 terms of an fp32 value: hi is v with its low 16 bits
// cleared (exact), mid the same of the remainder, lo the rest (at most 8
// significant bits, so its bf16 rounding is exact): hi + mid + lo == v.
__device__ __forceinline__ void split3(float v, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
  const uint32_t h = __float_as_uint(v) & 0xFFFF0000u;
  const float r1 = v - __uint_as_float(h);
  const uint32_t m = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(m);
  hi = h >> 16;
  mid = m >> 16;
  lo = f32_to_bf16(r2);
}

// The router weight split once per call into its three bf16 terms (hi, mid,
// lo; experts past E as zero rows), each stored in the logit kernel's
// fragment order: the 8 terms that lane (r, g) multiplies in step q of chunk
// c of expert tile y form the 16-byte piece
//   ((((y * nchunks + c) * 3 + term) * 2 + g) * 4 + q) * 32 + r,
// so each of the logit kernel's weight loads reads two contiguous 512-byte
// runs, and no block splits the weight again.
__global__ __launch_bounds__(256) void router_split_kernel(const float *__restrict__ w, int E,
                                                           int Epad, int H,
                                                           u32x4_t *__restrict__ wsplit) {
  const int64_t n = static_cast<int64_t>(Epad) * H / 8;  // groups of 8 weights
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int nch = H / 64;
  const int r = static_cast<int>(i % 32);
  int64_t rest = i / 32;
  const int q = static_cast<int>(rest % 4);
  rest /= 4;
  const int g = static_cast<int>(rest % 2);
  rest /= 2;
  const int c = static_cast<int>(rest % nch);
  const int y = static_cast<int>(rest / nch);
  const int e = y * 32 + r;
  const int k = 64 * c + 32 * g + 8 * q;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  if (e < E) {
    const f32x4_t *src = reinterpret_cast<const f32x4_t *>(w + static_cast<int64_t>(e) * H + k);
    const f32x4_t a0 = src[0], a1 = src[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a0[j];
      v[4 + j] = a1[j];
    }
  }
  u32x4_t th, tm, tl;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t h0, m0, l0, h1, m1, l1;
    split3(v[2 * p], h0, m0, l0);
    split3(v[2 * p + 1], h1, m1, l1);
    th[p] = h0 | (h1 << 16);
    tm[p] = m0 | (m1 << 16);
    tl[p] = l0 | (l1 << 16);
  }
  const int64_t base = ((((static_cast<int64_t>(y) * nch + c) * 3) * 2 + g) * 4 + q) * 32 + r;
  constexpr int64_t TERM = 2 * 4 * 32;  // pieces between the terms of one chunk
  wsplit[base] = th;
  wsplit[base + TERM] = tm;
  wsplit[base + 2 * TERM] = tl;
}

// Partial logits of kRouterMT = 128 tokens x 64 experts over one slice of the
// hidden dimension (blockIdx.y; 64-wide chunks [y cps, (y + 1) cps)). The
// router weight is the same for every block of tokens, so the blocks take
// 128 tokens each (fewer weight reads per token) and split the hidden
// dimension for parallelism; the selection kernel adds the slices in order.
// 8 waves: wave w owns tokens 32 (w % 4) .. + 31 and experts 32 (w / 4) ..
// + 31, so every (token, expert) of the block is summed by one wave; the
// four waves of an expert tile read the same weight pieces (L1). Each wave
// loads the next chunk's operands while it multiplies the current one.
// With NORM the rows are normalised on the fly with their r (computed by
// row_rms_kernel): n = bf16(x r), xn = bf16(w n), and the first expert
// tile's waves write xn (the expert GEMMs' input; every chunk of every real
// row is written by exactly one wave).
//
// MFMA operand layout (v_mfma_f32_32x32x16_bf16, A = the rows, B = the
// weight terms): lane l supplies token l % 32 of A and expert l % 32 of B,
// each with 8 consecutive k values; any k assignment is valid as long as A
// and B agree: in chunk c lane half g takes k in 64 c + 32 g + [0, 32) and
// step q its elements [8 q, 8 q + 8), so each lane reads 64 contiguous bytes
// of its row per chunk, and the weight's terms come in the fragment order of
// router_split_kernel. The three terms of a weight go into the same
// accumulator, hi first. Result element v of lane l is token
// 8 (v / 4) + 4 (l / 32) + v % 4 and expert l % 32 of the wave's tile.
// Padding rows are not read (their partial logits are 0, never used) and get
// no normalised row.
struct RouterSliceArgs {
  const uint16_t *x;
  const u32x4_t *wsplit;   // the weight's three bf16 terms in fragment order
  const uint16_t *norm_w;  // [H] (NORM)
  const float *rrow;       // [T] r of each real row (NORM)
  uint16_t *xn;            // [T, H] (NORM)
  const uint8_t *pad;
  int64_t T;
  int H, E;
  int cps;                 // chunks per slice
  float *partial;          // [slices][T][E]
};

template <bool NORM>
__global__ __launch_bounds__(512) void router_slice_kernel(RouterSliceArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, g = lane >> 5;
  const int tt = wave & 3, y = wave >> 2;
  if (y * 32 >= a.E) return;  // E <= 32: one expert tile (no barrier below)
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouterMT + tt * 32 + r;
  const bool tok = t < a.T && !(a.pad && a.pad[t]);
  const int H = a.H;
  const int nchunks = H / 64;
  const int c_lo = blockIdx.y * a.cps;
  const int c_hi = min(nchunks, c_lo + a.cps);
  const u32x4_t *xr = reinterpret_cast<const u32x4_t *>(a.x + (tok ? t : 0) * H) + 4 * g;
  // this lane's weight pieces: (chunk c, term sp, step q) at
  // wt[(c * 3 + sp) * 256 + q * 32]
  const u32x4_t *wt = a.wsplit + (static_cast<int64_t>(y) * nchunks * 3 * 2 + g) * 128 + r;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  float rt = 1.0f;
  const u32x4_t *nwr = nullptr;
  u32x4_t *xno = nullptr;
  if constexpr (NORM) {
    rt = tok ? a.rrow[t] : 1.0f;
    nwr = reinterpret_cast<const u32x4_t *>(a.norm_w) + 4 * g;
    xno = reinterpret_cast<u32x4_t *>(a.xn + (tok ? t : 0) * H) + 4 * g;
  }
  const bool write_xn = NORM && tok && y == 0;

  // four accumulators, chunk c into acc[(c - c_lo) % 4], added in a fixed
  // order at the end: each fp32 sum runs over at most a quarter of the
  // slice's products (large slices, when T is large, keep the rounding of
  // the logits as small as small slices do)
  f32x16_t acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[u][v] = 0.0f;
  u32x4_t xv[4], wv[3][4];
  auto load = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[q] = tok ? xr[8 * c + q] : zero4;
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
#pragma unroll
      for (int q = 0; q < 4; ++q) wv[sp][q] = wt[(static_cast<int64_t>(c) * 3 + sp) * 256 + q * 32];
  };
  // one chunk: multiply the operands loaded for it (after starting the next
  // chunk's loads) into accumulator ac
  auto chunk = [&](int c, f32x16_t &ac) __attribute__((always_inline)) {
    u32x4_t av[4], bw[3][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) av[q] = xv[q];
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
#pragma unroll
      for (int q = 0; q < 4; ++q) bw[sp][q] = wv[sp][q];
    if (c + 1 < c_hi) load(c + 1);
    if constexpr (NORM) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        av[q] = norm_chunk<kBF16>(av[q], nwr[8 * c + q], rt);
        if (write_xn) xno[8 * c + q] = av[q];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, av[q]);
#pragma unroll
      for (int sp = 0; sp < 3; ++sp)
        ac = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, __builtin_bit_cast(bf16x8_t, bw[sp][q]),
                                                     ac, 0, 0, 0);
    }
  };
  if (c_lo < c_hi) load(c_lo);
  for (int c = c_lo; c < c_hi; c += 4) {
    chunk(c, acc[0]);
    if (c + 1 < c_hi) chunk(c + 1, acc[1]);
    if (c + 2 < c_hi) chunk(c + 2, acc[2]);
    if (c + 3 < c_hi) chunk(c + 3, acc[3]);
  }
  float *out = a.partial + static_cast<int64_t>(blockIdx.y) * a.T * a.E;
  const int e = y * 32 + r;
  if (e < a.E) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t tv = static_cast<int64_t>(blockIdx.x) * kRouterMT + tt * 32 + (v >> 2) * 8 +
                         g * 4 + (v & 3);
      if (tv < a.T) out[tv * a.E + e] = ((acc[0][v] + acc[1][v]) + acc[2][v]) + acc[3][v];
    }
  }
}

// r = 1 / sqrt(mean(x^2) + eps) of every real row, exactly as the RMSNorm
// kernel forms it (fp64 sum of the squares, the same butterfly order, one
// rounding of the mean, r evaluated in fp64 and rounded once to fp32): one
// wave per row, four rows per block, the row read once. Padding rows get
// none.
__global__ __launch_bounds__(256) void row_rms_kernel(const uint16_t *__restrict__ x,
                                                      const uint8_t *__restrict__ pad,
                                                      int64_t T, int H, float eps,
                                                      float *__restrict__ rrow) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T || (pad && pad[t])) return;
  const int nc = H / 8;  // 16-byte chunks
  const u32x4_t *xr = reinterpret_cast<const u32x4_t *>(x + t * H);
  double ss = 0.0;
  // (eight loads in flight per lane at a time)
  for (int i0 = 0; i0 < nc; i0 += 8 * 64) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + 64 * u + lane;
      v[u] = i < nc ? xr[i] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) ss += chunk_sq<kBF16>(v[u]);
  }
  const float rv = rms_finish(ss, H, eps);
  if (lane == 0) rrow[t] = rv;
}

int router_slices(int64_t T, int H) {
  const int nb = static_cast<int>((T + kRouterMT - 1) / kRouterMT);
  // one round of blocks (at most 256, one per CU), at least one chunk per
  // slice
  return std::max(1, std::min(std::min(kRouterMaxSlices, H / 64), 256 / nb));
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
    if (a.norm_w) return hipErrorInvalidValue;  // fp32 layers normalise in their own kernel
    hipLaunchKernelGGL(router_f32_kernel, dim3(nb), dim3(256), 0, s, a, partial);
  } else {
    const int Epad = (a.E + 31) / 32 * 32;
    const int64_t n = static_cast<int64_t>(Epad) * a.H / 8;
    hipLaunchKernelGGL(router_split_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, s, a.w_router, a.E, Epad, a.H,
                       static_cast<u32x4_t *>(a.wsplit));
    if (a.norm_w)
      hipLaunchKernelGGL(row_rms_kernel, dim3(static_cast<unsigned>((a.T + 3) / 4)), dim3(256), 0,
                         s, static_cast<const uint16_t *>(a.x), a.pad, a.T, a.H, a.eps, a.rrow);
    slices = router_slices(a.T, a.H);
    const int nchunks = a.H / 64;
    const int cps = (nchunks + slices - 1) / slices;
    slices = (nchunks + cps - 1) / cps;  // no empty slice
    RouterSliceArgs ra{static_cast<const uint16_t *>(a.x), static_cast<const u32x4_t *>(a.wsplit),
                       static_cast<const uint16_t *>(a.norm_w), a.rrow,
                       static_cast<uint16_t *>(a.xn), a.pad, a.T, a.H, a.E, cps, partial};
    const dim3 grid(static_cast<unsigned>((a.T + kRouterMT - 1) / kRouterMT),
                    static_cast<unsigned>(slices));
    if (a.norm_w)
      hipLaunchKernelGGL(router_slice_kernel<true>, grid, dim3(512), 0, s, ra);
    else
      hipLaunchKernelGGL(router_slice_kernel<false>, grid, dim3(512), 0, s, ra);
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
