// Router: logits = W_r x in fp32, softmax over all experts in fp32, top-K
// (by logit, equal logits: lower expert index first), renormalised weights (model API page,
// build_moe_config; the gate kept in fp32 per the model-coverage page,
// "Train", and 'mlp.gate' in _keep_in_fp32_modules_strict).
//
// bf16 activations: each fp32 router weight is split, as the logit kernel
// stages it in LDS, into three bf16 terms hi + mid + lo that sum to it
// exactly (Henry, Tang & Heinecke, "Leveraging the bfloat16 Artificial
// Intelligence Datatype for Higher-Precision Computations", ARITH 2019). Each product x * term is exact
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
#include <type_traits>

#include "common.h"

namespace hi3 {

// Register sets of the logit kernel's load pipeline (chunks loaded ahead).
#ifndef HI3_ROUTER_LOAD_SETS
#define HI3_ROUTER_LOAD_SETS 2
#endif
constexpr int kRouterLoadSets = HI3_ROUTER_LOAD_SETS;
static_assert(kRouterLoadSets >= 2 && kRouterLoadSets <= 4, "router load sets");

// --------------------------------------------------------------- selection

// Softmax over all experts, top-K and renormalisation for 32 tokens per
// block: one wave per token at a time, lane = expert; then the block's
// expert histogram and real-row count.
// Every lane ranks its expert in the selection order (larger logit first,
// lower index first on equal logits; softmax is strictly increasing, so
// this is the order of the probabilities, and fp32 underflow of small
// probabilities cannot change it) by comparing selection keys. Z sums
// exp(l - max) in ascending expert order, the selected p = exp(l - max) / Z
// are summed in selection order, and each is divided by that sum.
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
  uint64_t key[kSelThreads / 64][kMaxE];  // one token's selection keys, likewise
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
    // Each lane's selection key orders the lanes in that order as unsigned
    // 64-bit integers: the logit's bits made monotonic (with -0 read as +0,
    // an equal value), then 63 - lane (the lower index first on equal
    // logits); lanes past E get key 0, below every live key. Every lane
    // reads all keys (written to LDS once, read back as broadcasts) and
    // counts those above its own: its rank. The maximum is the logit of the
    // rank-0 lane. The softmax denominator is summed in ascending expert
    // order from the broadcast values (every lane forms the same sum).
    const bool live = lane < E;
    const float l = live ? nan_as_neg_inf(lsum[j]) : -INFINITY;
    const uint32_t lb = __float_as_uint(l + 0.0f);
    const uint32_t mono = (lb & 0x80000000u) ? ~lb : (lb | 0x80000000u);
    const uint64_t key =
        live ? (static_cast<uint64_t>(mono) << 6) | static_cast<uint64_t>(63 - lane) : 0ull;
    typedef uint64_t u64x2_t __attribute__((ext_vector_type(2)));
    const u64x2_t *keyv = reinterpret_cast<const u64x2_t *>(sh.key[wave]);
    sh.key[wave][lane] = key;
    wave_lds_sync();
    int rank = 0;
#pragma unroll
    for (int e2 = 0; e2 < kMaxE / 2; ++e2) {
      const u64x2_t k2 = keyv[e2];
      rank += k2[0] > key ? 1 : 0;
      rank += k2[1] > key ? 1 : 0;
    }
    const uint64_t first = __ballot(live && rank == 0);  // exactly one lane
    const float m = __int_as_float(
        __builtin_amdgcn_readlane(__float_as_int(l), static_cast<int>(__builtin_ctzll(first))));
    const float ex = live ? expf(l - m) : 0.0f;
    const f32x4_t *rowv = reinterpret_cast<const f32x4_t *>(sh.row[wave]);
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

// The three bf16 terms of two fp32 values, packed in pairs (value 0 in the
// low half): hi is v with its low 16 bits cleared (exact), mid the same of
// the remainder, lo the rest, which has at most 8 significant bits and so
// is a bf16 value itself (for |v| above 2^-110, below which lo may lose
// bits of the fp32 subnormal range): hi + mid + lo == v, and each term is
// the top half of an fp32 word, taken by a byte permute.
__device__ __forceinline__ void split3x2(float v0, float v1, uint32_t &hi, uint32_t &mid,
                                         uint32_t &lo) {
  constexpr uint32_t kTop = 0xFFFF0000u;
  constexpr uint32_t kTops = 0x07060302u;  // bytes 2, 3 of the second operand, then of the first
  const uint32_t u0 = __float_as_uint(v0), u1 = __float_as_uint(v1);
  const float r0 = v0 - __uint_as_float(u0 & kTop), r1 = v1 - __uint_as_float(u1 & kTop);
  const uint32_t q0 = __float_as_uint(r0), q1 = __float_as_uint(r1);
  const float s0 = r0 - __uint_as_float(q0 & kTop), s1 = r1 - __uint_as_float(q1 & kTop);
  hi = __builtin_amdgcn_perm(u1, u0, kTops);
  mid = __builtin_amdgcn_perm(q1, q0, kTops);
  lo = __builtin_amdgcn_perm(__float_as_uint(s1), __float_as_uint(s0), kTops);
}

// Partial logits of kRouterMT = 128 tokens x 64 experts over one slice of the
// hidden dimension (blockIdx.y; 64-wide chunks [y cps, (y + 1) cps)). The
// router weight is the same for every block of tokens, so the blocks take
// 128 tokens each (fewer weight reads per token) and split the hidden
// dimension for parallelism; the selection kernel adds the slices in order.
//
// Each chunk is staged in LDS by all 256 threads with coalesced 16-byte
// loads: the 128 token rows (normalised on the way with NORM), and the 64
// expert rows of the fp32 weight, split on the way into their three bf16
// terms. The loads run kRouterLoadSets chunks ahead of the multiplication
// (that many register sets, two LDS buffers, one barrier per chunk). With
// NORM the rows are normalised with their r (computed by row_rms_kernel):
// n = bf16(x r), xn = bf16(w n); the staging threads also write xn (the
// expert GEMMs' input): every element of every real row is written once.
//
// 4 waves: wave w multiplies tokens 64 (w % 2) .. + 63 (two 32-token tiles)
// by experts 32 (w / 2) .. + 31.
// MFMA operand layout (v_mfma_f32_32x32x16_bf16, A = the rows, B = the
// weight terms): lane l supplies token l % 32 of A and expert l % 32 of B,
// each with 8 consecutive k values; any k assignment is valid as long as A
// and B agree: in chunk c lane half g takes k in 64 c + 32 g + [0, 32) and
// step q its elements [8 q, 8 q + 8). The three terms of a weight go into
// the same accumulator, hi first; chunk c goes into accumulator
// (c - first chunk) % 2, and the two are added at the end (each fp32 sum
// runs over at most half of the slice's products; with two blocks per CU
// in a round, a slice holds at most 64 / (round / token blocks) chunks). Result
// element v of lane l is token 8 (v / 4) + 4 (l / 32) + v % 4 and expert
// l % 32 of the tile. x's padding rows are not read (their partial logits
// are never used) and get no normalised row.
struct RouterSliceArgs {
  const uint16_t *x;
  const float *w;          // [E, H] fp32 router weight
  const uint16_t *norm_w;  // [H] (NORM)
  const float *rrow;       // [T] r of each real row (NORM)
  uint16_t *xn;            // [T, H] (NORM)
  const uint8_t *pad;
  int64_t T;
  int H, E;
  int cps;                 // chunks per slice
  float *partial;          // [slices][T][E]
};

// Workgroup barrier for LDS data only: waits for this wave's LDS operations
// (lgkmcnt(0)) but not for its global loads, which may stay in flight
// across it (__syncthreads() would also drain them).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// LDS position (16-byte units) of 16-byte piece c (0..7) of row `row` of a
// staged chunk (128 bytes per row): piece c is stored at c ^ ((row / 2) % 8),
// so the 16 rows of one fragment read fall in 16 distinct bank groups.
__device__ __forceinline__ int rl_pos(int row, int c) { return row * 8 + (c ^ ((row >> 1) & 7)); }

// f(integral_constant<S>, i + S) for S = 0 .. N - 1
template <int N, int S = 0, typename F>
__device__ __forceinline__ void unroll_steps(F &&f, int i) {
  if constexpr (S < N) {
    f(std::integral_constant<int, S>{}, i + S);
    unroll_steps<N, S + 1>(f, i);
  }
}

// The same for the steps i + S < n, each guard inside the previous one.
template <int N, int S = 0, typename F>
__device__ __forceinline__ void tail_steps(F &&f, int i, int n) {
  if constexpr (S < N) {
    if (i + S < n) {
      f(std::integral_constant<int, S>{}, i + S);
      tail_steps<N, S + 1>(f, i, n);
    }
  }
}

struct RouterStage {
  u32x4_t x[kRouterMT * 8];  // the chunk of the block's token rows
  u32x4_t w[3][kMaxE * 8];   // the chunk of the weight's hi, mid and lo terms
};

template <bool NORM>
__global__ __launch_bounds__(256, 2) void router_slice_kernel(RouterSliceArgs a) {
  __shared__ RouterStage st[2];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 31, g = lane >> 5;
  const int tb = wave & 1, y = wave >> 1;
  const int64_t T0 = static_cast<int64_t>(blockIdx.x) * kRouterMT;
  const int H = a.H;
  const int nchunks = H / 64;
  const int c_lo = blockIdx.y * a.cps;
  const int c_hi = min(nchunks, c_lo + a.cps);

  // staging: piece p = tid + 256 u (u = 0..3) of the token rows (row p / 8,
  // 16 bytes at 8 (p % 8) elements) and of the weight (expert p / 16, 4
  // floats at 4 (p % 16))
  // (row r0 + 32 u of the block and expert e0 + 16 u)
  const int xp = tid & 7, wp = tid & 15;
  const int r0 = tid >> 3, e0 = tid >> 4;
  const int64_t xstep = int64_t{32} * H / 8;
  // The loads are not predicated (a divergent branch around each would make
  // the compiler drain every load in flight before the first use of any):
  // a padding row or a row past T reads the router weight's first row
  // instead (x's padding rows are never read), an expert past E reads
  // expert 0. Their values are staged as they are: an output element
  // depends on its own row and expert only, and the partial logits of
  // those rows and experts are never stored or used.
  const f32x4_t *wsrc = reinterpret_cast<const f32x4_t *>(a.w) + wp;
  u32x4_t *xdst = NORM ? reinterpret_cast<u32x4_t *>(a.xn + (T0 + r0) * H) + xp : nullptr;
  uint32_t xok = 0;           // bit u: row u is real
  const u32x4_t *xsrc[4];
  int32_t woff[4];            // 16-byte units
  float rr[NORM ? 4 : 1];
  // (the padding flags and the rows' r are read for a clamped row, all
  // loads before the first use)
  uint8_t pv[4] = {0, 0, 0, 0};
  if (a.pad) {
#pragma unroll
    for (int u = 0; u < 4; ++u) pv[u] = a.pad[min(T0 + r0 + 32 * u, a.T - 1)];
  }
  if constexpr (NORM) {
#pragma unroll
    for (int u = 0; u < 4; ++u) rr[u] = a.rrow[min(T0 + r0 + 32 * u, a.T - 1)];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t t = T0 + r0 + 32 * u;
    const bool ok = t < a.T && !pv[u];
    const bool eok = e0 + 16 * u < a.E;
    xok |= ok ? 1u << u : 0u;
    xsrc[u] = (ok ? reinterpret_cast<const u32x4_t *>(a.x + t * H)
                  : reinterpret_cast<const u32x4_t *>(a.w)) + xp;
    woff[u] = eok ? (e0 + 16 * u) * (H / 4) : 0;
  }
  const u32x4_t *nwsrc = NORM ? reinterpret_cast<const u32x4_t *>(a.norm_w) + xp : nullptr;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  // NS register sets of staged pieces: chunk c_lo + i goes to set i % NS
  constexpr int NS = kRouterLoadSets;
  u32x4_t xs[NS][4];
  f32x4_t ws[NS][4];
  u32x4_t nws[NS];
#pragma unroll
  for (int b = 0; b < NS; ++b) nws[b] = zero4;
  auto load = [&](auto S, int c) __attribute__((always_inline)) {
    constexpr int b = decltype(S)::value;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xs[b][u] = xsrc[u][8 * c];
      ws[b][u] = wsrc[woff[u] + 16 * c];
    }
    if constexpr (NORM) nws[b] = nwsrc[8 * c];
  };
  // (wr: also write the normalised rows; false when the chunk is a repeat)
  auto store = [&](auto S, RouterStage &sg, int c, bool wr) __attribute__((always_inline)) {
    constexpr int b = decltype(S)::value;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = r0 + 32 * u;
      u32x4_t v = xs[b][u];
      if constexpr (NORM) {
        v = norm_chunk<kBF16>(v, nws[b], rr[u]);
        if (((xok >> u) & 1u) && wr) xdst[u * xstep + 8 * c] = v;
      }
      sg.x[rl_pos(row, xp)] = v;
      // the weight's three terms: 4 bf16 each, the half of a 16-byte piece
      const int e = e0 + 16 * u;
      uint32_t h0, m0, l0, h1, m1, l1;
      split3x2(ws[b][u][0], ws[b][u][1], h0, m0, l0);
      split3x2(ws[b][u][2], ws[b][u][3], h1, m1, l1);
      const int pos = rl_pos(e, wp >> 1);
      const int half = wp & 1;
      reinterpret_cast<u32x2_t *>(&sg.w[0][pos])[half] = u32x2_t{h0, h1};
      reinterpret_cast<u32x2_t *>(&sg.w[1][pos])[half] = u32x2_t{m0, m1};
      reinterpret_cast<u32x2_t *>(&sg.w[2][pos])[half] = u32x2_t{l0, l1};
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][u][v] = 0.0f;
  // multiply the staged chunk in sg into accumulator u of both token tiles
  auto compute = [&](const RouterStage &sg, auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value & 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cc = 4 * g + q;
      const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, sg.x[rl_pos(64 * tb + r, cc)]);
      const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, sg.x[rl_pos(64 * tb + 32 + r, cc)]);
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) {
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, sg.w[sp][rl_pos(32 * y + r, cc)]);
        acc[0][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc[0][u], 0, 0, 0);
        acc[1][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc[1][u], 0, 0, 0);
      }
    }
  };
  // Chunk c_lo + i is loaded into register set i % NS, staged in LDS
  // buffer i % 2 and multiplied into accumulator i % 2. Step i loads chunk
  // i + NS into the set staged in step i - 1, multiplies chunk i and stages
  // chunk i + 1: the loads of chunks i + 1 .. i + NS may be in flight during
  // the multiplication, and those of NS - 1 chunks stay in flight past the
  // staging. Past the slice's last chunk the loads and the staging
  // repeat it (into a set and a buffer that are not read again) instead of
  // being skipped: with no branch around them, the compiler's waits for a
  // set are exactly the loads issued before it (a load that might have been
  // skipped makes it wait for every load in flight). For the same reason
  // the steps run in whole periods of lcm(NS, 2) steps and the remaining
  // steps nest their guards.
  const int n = c_hi - c_lo;
  constexpr int P = NS % 2 == 0 ? NS : 2 * NS;
  auto step = [&](auto Sv, int i) __attribute__((always_inline)) {
    constexpr int sp = decltype(Sv)::value;  // i % P
    constexpr int u = sp & 1;
    // (the scheduling barriers keep the loads ahead of the multiplication
    // and of the staging, whose waits then leave them in flight)
    load(std::integral_constant<int, sp % NS>{}, c_lo + min(i + NS, n - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(st[u], std::integral_constant<int, u>{});
    __builtin_amdgcn_sched_barrier(0);
    store(std::integral_constant<int, (sp + 1) % NS>{}, st[1 - u], c_lo + min(i + 1, n - 1),
          i + 1 < n);
    lds_barrier();
  };
  int i = 0;
  if (n > 0) {
    unroll_steps<NS>([&](auto B, int b) __attribute__((always_inline)) { load(B, c_lo + min(b, n - 1)); },
                     0);
    store(std::integral_constant<int, 0>{}, st[0], c_lo, true);
    __syncthreads();
    for (; i + P <= n; i += P) unroll_steps<P>(step, i);
    tail_steps<P - 1>(step, i, n);
  }
  float *out = a.partial + static_cast<int64_t>(blockIdx.y) * a.T * a.E;
  const int e = y * 32 + r;
  if (e < a.E) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t tv = T0 + 64 * tb + 32 * i + (v >> 2) * 8 + g * 4 + (v & 3);
        if (tv < a.T)
          out[tv * a.E + e] = acc[i][0][v] + acc[i][1][v];
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
  // one round of blocks (at most kRouterRound), at least one chunk per slice
  return std::max(1, std::min(std::min(kRouterMaxSlices, H / 64), kRouterRound / nb));
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
    if (a.norm_w)
      hipLaunchKernelGGL(row_rms_kernel, dim3(static_cast<unsigned>((a.T + 3) / 4)), dim3(256), 0,
                         s, static_cast<const uint16_t *>(a.x), a.pad, a.T, a.H, a.eps, a.rrow);
    slices = router_slices(a.T, a.H);
    const int nchunks = a.H / 64;
    const int cps = (nchunks + slices - 1) / slices;
    slices = (nchunks + cps - 1) / cps;  // no empty slice
    RouterSliceArgs ra{static_cast<const uint16_t *>(a.x), a.w_router,
                       static_cast<const uint16_t *>(a.norm_w), a.rrow,
                       static_cast<uint16_t *>(a.xn), a.pad, a.T, a.H, a.E, cps, partial};
    const dim3 grid(static_cast<unsigned>((a.T + kRouterMT - 1) / kRouterMT),
                    static_cast<unsigned>(slices));
    if (a.norm_w)
      hipLaunchKernelGGL(router_slice_kernel<true>, grid, dim3(256), 0, s, ra);
    else
      hipLaunchKernelGGL(router_slice_kernel<false>, grid, dim3(256), 0, s, ra);
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
