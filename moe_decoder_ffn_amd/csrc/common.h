// Internal definitions shared by the HIP kernels and the host side of the
// C ABI: vector types, bf16 helpers, wavefront reductions, tile constants and
// the workspace plan.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hi3 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kWave = 64;
constexpr int kMaxE = 64;

// Router / dispatch token blocking: one selection block handles kRouterTB
// tokens, and the per-block expert histograms that the stable counting sort
// scans use the same blocking.
#ifndef HI3_ROUTER_TB
#define HI3_ROUTER_TB 32
#endif
constexpr int kRouterTB = HI3_ROUTER_TB;
static_assert(kRouterTB >= 1 && kRouterTB <= 64, "token block: one wave's lanes");
// The bf16 router: tokens per block of its logit kernel, and at most this
// many slices of the hidden dimension.
constexpr int kRouterMT = 128;
constexpr int kRouterMaxSlices = 16;
// Logit blocks per round of the GPU (two 4-wave blocks per CU).
#ifndef HI3_ROUTER_ROUND
#define HI3_ROUTER_ROUND 512
#endif
constexpr int kRouterRound = HI3_ROUTER_ROUND;
// Rows per partial sum of the RMSNorm weight gradient (block backward).
constexpr int kNormBwdRows = 64;

// bf16 grouped GEMM tiles: rows x 256 weight rows x k step, LDS stages.
// The row-tile list holds tiles of HI3_GEMM_BM rows (the up/gate tile); the
// down projection runs each listed tile as HI3_GEMM_DOWN_SPLIT blocks.
#ifndef HI3_GEMM_BM
#define HI3_GEMM_BM 256
#endif
#ifndef HI3_GEMM_BK
#define HI3_GEMM_BK 64
#endif
#ifndef HI3_GEMM_STAGES
#define HI3_GEMM_STAGES 2
#endif
#ifndef HI3_GEMM_DOWN_SPLIT
#define HI3_GEMM_DOWN_SPLIT 1
#endif
#ifndef HI3_GEMM_DOWN_STAGES
#define HI3_GEMM_DOWN_STAGES 2
#endif
#ifndef HI3_GEMM_WN
#define HI3_GEMM_WN 4
#endif
constexpr int kGemmBM = HI3_GEMM_BM;
constexpr int kGemmBN = 256;
constexpr int kGemmBK = HI3_GEMM_BK;
constexpr int kGemmStages = HI3_GEMM_STAGES;
// Streaming configuration for small batches (few rows per expert, the
// weights dominate the traffic): 64-row tiles for both projections with a
// 4-stage ring (the whole 160 KiB of LDS), so more weight bytes are in flight
// per CU. Chosen per call when T * K / E is at most kGemmStreamMaxRows.
#ifndef HI3_GEMM_STREAM_MAX_ROWS
#define HI3_GEMM_STREAM_MAX_ROWS 112
#endif
#ifndef HI3_GEMM_STREAM_STAGES
#define HI3_GEMM_STREAM_STAGES 4
#endif
#ifndef HI3_GEMM_STREAM_BK
#define HI3_GEMM_STREAM_BK 64
#endif
constexpr int kGemmStreamBM = 64;
constexpr int kGemmStreamStages = HI3_GEMM_STREAM_STAGES;
constexpr int kGemmStreamBK = HI3_GEMM_STREAM_BK;
constexpr int kGemmStreamMaxRows = HI3_GEMM_STREAM_MAX_ROWS;
constexpr int kGemmDownSplit = HI3_GEMM_DOWN_SPLIT;
constexpr int kGemmDownStages = HI3_GEMM_DOWN_STAGES;
static_assert(kGemmBM % kGemmDownSplit == 0, "down tile rows");
constexpr int kGemmWN = HI3_GEMM_WN;  // waves along the columns (2 along the rows)
// Row tiles of at most a quarter of the tile rows run a quarter-height body.
#ifndef HI3_GEMM_QUARTER_BODY
#define HI3_GEMM_QUARTER_BODY 1
#endif
// Grouped GEMM job list (modes 0-3): column tiles per chunk (each chunk
// takes every row tile of its group before the next chunk).
#ifndef HI3_GEMM_COL_CHUNK
#define HI3_GEMM_COL_CHUNK 4
#endif
// hi3_moe_forward_overlap runs the shared expert's GEMMs on the caller's side
// stream alongside the routing (when every row is real).
#ifndef HI3_OVERLAP_SHARED
#define HI3_OVERLAP_SHARED 1
#endif
// GEMMs whose B operand is a weight (8-wave blocks, 2-stage ring: the
// forward and the backward's dx GEMM): a third LDS stage for the weights,
// whose copies then run two steps ahead.
#ifndef HI3_GEMM_DEEP_B
#define HI3_GEMM_DEEP_B 1
#endif
// Backward GEMMs: the gradient through the down projection (mode 2) runs each
// listed row tile as HI3_DGRAD_DOWN_SPLIT blocks; the gradient through
// [up; gate] (mode 3) and the weight gradients (mode 4) use the given k step
// and stage counts.
#ifndef HI3_DGRAD_DOWN_SPLIT
#define HI3_DGRAD_DOWN_SPLIT 1
#endif
#ifndef HI3_DGRAD_DOWN_STAGES
#define HI3_DGRAD_DOWN_STAGES 2
#endif
#ifndef HI3_DGRAD_UP_BK
#define HI3_DGRAD_UP_BK 64
#endif
#ifndef HI3_DGRAD_UP_STAGES
#define HI3_DGRAD_UP_STAGES 2
#endif
#ifndef HI3_WGRAD_BK
#define HI3_WGRAD_BK 32
#endif
#ifndef HI3_WGRAD_STAGES
#define HI3_WGRAD_STAGES 3
#endif
// Modes 1, 3 and 4 write their tile through the LDS ring (1) or directly
// from the accumulators (0).
#ifndef HI3_GEMM_STAGED_STORE
#define HI3_GEMM_STAGED_STORE 1
#endif
constexpr bool kGemmStagedStore = HI3_GEMM_STAGED_STORE != 0;
constexpr bool kGemmDeepB = HI3_GEMM_DEEP_B != 0;
constexpr bool kOverlapShared = HI3_OVERLAP_SHARED != 0;
constexpr int kGemmColChunk = HI3_GEMM_COL_CHUNK;
constexpr bool kGemmQuarterBody = HI3_GEMM_QUARTER_BODY != 0;
constexpr int kDgradDownSplit = HI3_DGRAD_DOWN_SPLIT;
// k step of the dh GEMM and the blocks per CU its registers allow
#ifndef HI3_DGRAD_DOWN_BK
#define HI3_DGRAD_DOWN_BK 64
#endif
#ifndef HI3_DGRAD_DOWN_OCC
#define HI3_DGRAD_DOWN_OCC 1
#endif
constexpr int kDgradDownBK = HI3_DGRAD_DOWN_BK;
// the third weight stage for the dh GEMM too (on 256-row tiles, 2 stages)
#ifndef HI3_DGRAD_DOWN_DEEP_B
#define HI3_DGRAD_DOWN_DEEP_B 0
#endif
constexpr bool kDgradDownDeepB = HI3_DGRAD_DOWN_DEEP_B != 0;
constexpr int kDgradDownOcc = HI3_DGRAD_DOWN_OCC;
constexpr int kDgradDownStages = HI3_DGRAD_DOWN_STAGES;
// Rows per wave in flight in the mode-2 epilogue (its u, g, h reads).
#ifndef HI3_DGRAD_EPI_ROWS
#define HI3_DGRAD_EPI_ROWS 4
#endif
constexpr int kDgradEpilogueRows = HI3_DGRAD_EPI_ROWS;
constexpr int kDgradUpBK = HI3_DGRAD_UP_BK;
constexpr int kDgradUpStages = HI3_DGRAD_UP_STAGES;
// Weight-gradient output tile rows: 256 (8 waves, one block per CU) or 128
// (4 waves, two blocks per CU, so one block's prologue and epilogue overlap
// the other's main loop).
// Weight-gradient tile order: groups of this many row tiles, walked down
// the rows first.
#ifndef HI3_WGRAD_GROUP_ROWS
#define HI3_WGRAD_GROUP_ROWS 8
#endif
#ifndef HI3_WGRAD_BM
#define HI3_WGRAD_BM 128
#endif
constexpr int kWgradBM = HI3_WGRAD_BM;
constexpr int kWgradGroupRows = HI3_WGRAD_GROUP_ROWS;
// waves along the output columns (2 along the rows): 128-row tiles run 4 or
// 8 waves
#ifndef HI3_WGRAD_WN
#define HI3_WGRAD_WN 4
#endif
constexpr int kWgradWN = kWgradBM == 256 ? kGemmWN : HI3_WGRAD_WN;
constexpr int kWgradBK = HI3_WGRAD_BK;
constexpr int kWgradStages = HI3_WGRAD_STAGES;
static_assert(kGemmBM % kDgradDownSplit == 0 && (kGemmBM / kDgradDownSplit) % 64 == 0,
              "dgrad tile rows");
// fp32 grouped GEMM tile.
constexpr int kGemmF32BM = 64;
constexpr int kGemmF32BN = 64;

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) |
         (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ---------------------------------------------------------------- RMSNorm steps

// The block's RMSNorm in front of the layer (layers API page,
// HunyuanRMSNorm), step by step to the rounding: the squares of one 16-byte
// chunk summed in fp64 (chunk_sq); n = dtype(x * r), xn = dtype(w * n) for
// the elements of one chunk (norm_chunk).
template <int DT>
__device__ __forceinline__ void unpack16(const u32x4_t &v, float *f) {
  if (DT == kBF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(v[e] << 16);
      f[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
  }
}

// n = dtype(x * r), xn = dtype(w * n) for the elements of one chunk.
template <int DT>
__device__ __forceinline__ u32x4_t norm_chunk(const u32x4_t &xv, const u32x4_t &wv, float r) {
  constexpr int PER = DT == kBF16 ? 8 : 4;
  float f[PER], w[PER];
  unpack16<DT>(xv, f);
  unpack16<DT>(wv, w);
  u32x4_t o;
  if (DT == kBF16) {
    uint16_t q[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float n = bf16_to_f32(f32_to_bf16(f[e] * r));
      q[e] = f32_to_bf16(w[e] * n);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = static_cast<uint32_t>(q[2 * e]) | (static_cast<uint32_t>(q[2 * e + 1]) << 16);
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = __float_as_uint(w[e] * (f[e] * r));
  }
  return o;
}

template <int DT>
__device__ __forceinline__ double chunk_sq(const u32x4_t &v) {
  constexpr int PER = DT == kBF16 ? 8 : 4;
  float f[PER];
  unpack16<DT>(v, f);
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < PER; ++e) ss += static_cast<double>(f[e]) * static_cast<double>(f[e]);
  return ss;
}

// The wave's partial sums of squares (lane l holding the chunks l, l + 64,
// ... of the row, each summed in order) added in a fixed butterfly order,
// m = the mean rounded to fp32, d = m + eps in fp32, r = 1 / sqrt(d)
// evaluated in fp64 and rounded once to fp32; every lane returns the same r.
__device__ __forceinline__ float rms_finish(double ss, int H, float eps) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float m = static_cast<float>(ss / static_cast<double>(H));
  const float d = m + eps;
  return static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
}

// ---------------------------------------------------------------- waves

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Butterfly sum, then lane 0's value broadcast so every lane holds the same
// bits.
__device__ __forceinline__ float wave_sum_uniform(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return __shfl(v, 0, kWave);
}

// Largest value over the wave; equal values resolve to the lowest index.
// Every lane ends with the same (v, i).
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, kWave);
    int oi = __shfl_xor(i, o, kWave);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ int wave_uniform(int v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// ---------------------------------------------------------------- plan

// Number of hidden-dimension slices the bf16 router splits the logits over.
int router_slices(int64_t T, int H);

// Byte offsets of every buffer inside the caller's workspace. Buffers that
// depend on the expert sizes come last, so the route/dispatch layout
// (I = Is = 0) is a prefix of the forward layout.
struct Plan {
  int64_t T;
  int H, E, K, I, Is, dtype;
  int NB;         // token blocks of kRouterTB rows
  int BM;         // grouped-GEMM tile rows (per dtype)
  int max_tiles;  // upper bound on grouped-GEMM row tiles
  size_t rpart;   // [slices][T][E] fp32: router partial logits
  size_t idx;     // [T*K] int32 routes when the caller passes none
  size_t wts;     // [T*K] fp32
  size_t blkcnt;  // [NB][E] int32 per-block expert histogram
  size_t blkval;  // [NB] int32 real rows per block
  size_t eoff;    // [E+1] int32 expert offsets
  size_t counts;  // [E] int32
  size_t misc;    // [16] int32: [0] real rows
  size_t gto;     // [E+2] int32 first row tile of each group (E = shared)
  size_t tiles;   // [max_tiles] int4: group, first row, rows, 0
  size_t perm;    // [T*K] int32 slot -> token
  size_t slotof;  // [T*K] int32 (token, k) -> slot
  size_t vtok;    // [T] int32 real-row index -> token
  size_t vidx;    // [T] int32 token -> real-row index (-1 padding)
  size_t xn;      // [T,H] dtype: rows after the block's RMSNorm (norm + residual entry)
  size_t rnorm;   // [T] fp32: the RMSNorm's r of each row (norm + residual entry)
  size_t h;       // [T*K, I] dtype: SwiGLU activations of routed rows
  size_t hs;      // [T, Is] dtype: SwiGLU activations of the shared expert
  size_t y;       // [T*K, H] fp32: routed expert outputs by slot
  size_t ys;      // [T, H] fp32: shared expert outputs by real-row index
  // backward only (the forward's y / ys hold dx by slot / by real row)
  size_t ug;      // [T*K, 2I] fp32: u and g of the routed rows
  size_t ugs;     // [T, 2Is] fp32: u and g of the shared expert
  size_t xs;      // [T*K, H] dtype: x by slot
  size_t dys;     // [T*K, H] dtype: w * dout by slot
  size_t xv;      // [T, H] dtype: x by real-row index (padding only)
  size_t doutv;   // [T, H] dtype: dout by real-row index (padding only)
  size_t dd;      // [T*K, 2I] dtype: [du; dg] of the routed rows
  size_t dds;     // [T, 2Is] dtype: [du; dg] of the shared expert
  size_t apart;   // [T*K, P] fp32: partial sums of dh * h
  size_t dls;     // [T*K] fp32: logit gradient by slot
  size_t wslot;   // [T*K] fp32: routing weight by slot
  size_t dwrpart; // [max_tiles, H] fp32: router weight gradient per row tile
  size_t dxn;     // [T, H] fp32: dL/dxn (block backward)
  size_t rrow;    // [T] fp32: RMSNorm r per row (block backward)
  size_t nwpart;  // [ceil(T / kNormBwdRows), H] fp32: norm weight gradient partials
  size_t zrow;    // 512 bytes of zeros
  int P;
  size_t total;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Partial sums of dh * h per routed row (bf16: one per 128 columns, written
// by the mode-2 GEMM or by the recompute's SwiGLU backward epilogue).
inline int apart_cols(int I, int dtype) {
  return dtype == kBF16 ? (I + kGemmBN / 2 - 1) / (kGemmBN / 2)
                        : (I + kGemmF32BN - 1) / kGemmF32BN;
}


inline Plan make_plan(int64_t T, int H, int E, int K, int I, int Is, int dtype,
                      bool backward = false) {
  Plan p{};
  p.T = T; p.H = H; p.E = E; p.K = K; p.I = I; p.Is = Is; p.dtype = dtype;
  p.NB = static_cast<int>((T + kRouterTB - 1) / kRouterTB);
  if (dtype != kBF16)
    p.BM = kGemmF32BM;
  else
    p.BM = T * K <= static_cast<int64_t>(kGemmStreamMaxRows) * E ? kGemmStreamBM : kGemmBM;
  const int64_t TK = T * K;
  p.max_tiles = static_cast<int>((TK + p.BM - 1) / p.BM + E + (T + p.BM - 1) / p.BM);
  const size_t es = dtype == kBF16 ? 2 : 4;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  p.rpart = take(static_cast<size_t>(dtype == kBF16 ? router_slices(T, H) : 1) * T * E * 4);
  p.idx = take(TK * 4);
  p.wts = take(TK * 4);
  p.blkcnt = take(static_cast<size_t>(p.NB) * E * 4);
  p.blkval = take(static_cast<size_t>(p.NB) * 4);
  p.eoff = take((E + 1) * 4);
  p.counts = take(E * 4);
  p.misc = take(16 * 4);
  p.gto = take((E + 2) * 4);
  p.tiles = take(static_cast<size_t>(p.max_tiles) * 16);
  p.perm = take(TK * 4);
  p.slotof = take(TK * 4);
  p.vtok = take(T * 4);
  p.vidx = take(T * 4);
  if (I > 0) {
    p.xn = take(T * H * es);
    p.rnorm = take(T * 4);
    p.h = take(TK * I * es);
    p.hs = take(T * Is * es);
    p.y = take(TK * H * 4);
    p.ys = take(T * H * 4);
  }
  if (backward && I > 0) {
    p.P = apart_cols(I, dtype);
    p.ug = take(TK * 2 * I * 4);
    p.ugs = take(T * 2 * Is * 4);
    p.xs = take(TK * H * es);
    p.dys = take(TK * H * es);
    p.xv = take(T * H * es);
    p.doutv = take(T * H * es);
    p.dd = take(TK * 2 * I * es);
    p.dds = take(T * 2 * Is * es);
    p.apart = take(TK * p.P * 4);
    p.dls = take(TK * 4);
    p.wslot = take(TK * 4);
    p.dwrpart = take(static_cast<size_t>(p.max_tiles) * H * 4);
    p.dxn = take(T * H * 4);
    p.rrow = take(T * 4);
    p.nwpart = take(static_cast<size_t>((T + kNormBwdRows - 1) / kNormBwdRows) * H * 4);
    p.zrow = take(512);
  }
  p.total = o;
  return p;
}

// ---------------------------------------------------------------- launches

struct RouterArgs {
  const void *x;
  const float *w_router;
  const void *norm_w;  // bf16 layers: the block's RMSNorm weight [H], or null (x feeds
                       // the router as it is)
  float eps;
  void *xn;            // with norm_w: [T, H] normalised rows out (the experts' input)
  float *rrow;         // with norm_w: [T] fp32 scratch (r of each row)
  const uint8_t *pad;
  int64_t T;
  int H, E, K;
  int32_t *idx;
  float *wts;
  int32_t *blkcnt;
  int32_t *blkval;
};

struct ScanArgs {
  const int32_t *blkcnt;
  const int32_t *blkval;
  int NB, E, BM;
  int32_t *eoff;
  int32_t *counts_out;  // nullable (caller's expert_counts)
  int32_t *counts;      // workspace copy
  int32_t *misc;
  int32_t *gto;
  int4 *tiles;
  // when set, the shared group gets no row tiles here (its GEMMs run as
  // dense launches, launch_gemm_dense)
  int no_shared;
};

struct ScatterArgs {
  const int32_t *idx;
  const uint8_t *pad;
  int64_t T;
  int E, K;
  int32_t *perm;
  int32_t *slotof;
  int32_t *vtok;   // nullable
  int32_t *vidx;   // nullable
};

// One class of grouped-GEMM problems: the E routed experts (class 0) or the
// shared expert (class 1). Modes (gemm.hip):
//   0 [up; gate] + SwiGLU, 1 down projection: A [rows, Kd] and B [N, Kd],
//     both k-contiguous;
//   2 gradient through the down projection (dh = W2^T dy, SwiGLU backward in
//     the epilogue), 3 gradient through [up; gate] (dx = W13^T [du; dg]):
//     A k-contiguous, B k-major ([Kd, N], row stride ldb);
//   4 weight gradients C[m, n] = sum_k A[k, m] B[k, n] over the group's rows:
//     A k-major ([rows, M], row stride lda), B k-major ([rows, N], ldb).
struct GemmClass {
  const void *A;        // left operand, row stride lda elements
  int64_t lda;
  const int32_t *arow;  // nullable: row map (tile row index -> A row), modes 0-3
  const void *B;        // per group: [N, Kd] (modes 0, 1) or [Kd, N] (2, 3), row-major
  int64_t strideB;      // elements between consecutive experts' B
  void *C;              // output rows, row stride ldc elements
  int64_t ldc;
  int N;                // projection outputs (2*I for [up; gate], H for down)
  int Kd;               // reduction length (modes 0-3)
  int64_t ldb;          // B row stride, k-major B (modes 2-4)
  int M;                // mode 4: output rows (A columns)
  int64_t strideC;      // mode 4: elements between consecutive experts' C
  float *ug;            // mode 0: when set, u and g are also stored here (fp32,
                        // [rows, N] with u in the first N/2 columns); mode 2: read
                        // (when null, mode 2 stores dh itself, fp32, to C)
  const void *hsave;    // mode 2: SwiGLU activations [rows, N] (layer dtype)
  float *apart;         // modes 2, 0 with dh_in (nullable): per-row partial sums of
                        // dh * h, one per 128 columns
  int apart_ld;         // partial sums per row
  const float *rowscale;  // mode 2 (nullable): dh = rowscale[row] * (B^T A row)
  // mode 0, bf16 (the backward's recompute after mode 2 ran without ug): when
  // set, the epilogue also runs the SwiGLU backward from the accumulators' u
  // and g: dh_in [rows, N/2] fp32 in, [du; dg] [rows, N] (layer dtype, du
  // first) to dd_out, and the partial sums of dh * h per 128 columns to apart
  const float *dh_in;
  void *dd_out;
};

struct GemmArgs {
  GemmClass cls[2];
  const int4 *tiles;
  const int32_t *gto;
  int E;
  int NTn;    // column tiles of the widest class
  int split;     // blocks per listed row tile; set by the launcher
  int sub_rows;  // rows per block when split > 1 (block p takes rows [p sub_rows, ...))
  // mode 4: group g < E reduces over rows [goff[g], goff[g] + gcnt[g]) of A
  // and B; the shared group over rows [0, *nreal). Rows past the group's end
  // are read from zrow (zeros, at least 512 bytes).
  const int32_t *goff;
  const int32_t *gcnt;
  const int32_t *nreal;
  const void *zrow;
  int wg_shared_blocks;  // set by the launcher
  int dense_rows;        // dense launches: the rows of class 1 (no tile list)
};

struct CombineArgs {
  const float *y;
  const float *ys;
  const int32_t *slotof;
  const int32_t *vidx;
  const float *wts;
  const uint8_t *pad;
  int64_t T;
  int H, K;
  void *out;
  const void *resid;  // [T,H] dtype residual added before the rounding, or null
};

struct NormArgs {
  const void *x;       // [T,H] dtype
  const void *weight;  // [H] dtype
  const uint8_t *pad;  // [T] or null
  int64_t T;
  int H;
  float eps;
  void *xn;            // [T,H] dtype
};
hipError_t launch_rmsnorm(const NormArgs &a, int dtype, hipStream_t s);

// Backward of the block's RMSNorm plus its residual: per real row, r as the
// forward computes it, dx = r w g - r^3 x (sum x w g) / H, dh = dout + dx
// (rounded once to the layer dtype); dweight = sum over rows of g n.
struct NormBwdArgs {
  const void *x;       // [T,H] dtype: the block input h
  const void *weight;  // [H] dtype
  const uint8_t *pad;  // [T] or null
  int64_t T;
  int H;
  float eps;
  const float *g;      // [T,H] fp32: dL/dxn
  const void *dout;    // [T,H] dtype: dL/dout (the residual's share)
  void *dh;            // [T,H] dtype out, nullable
  float *r;            // [T] fp32 scratch: r of each real row
  float *part;         // [ceil(T / kNormBwdRows), H] fp32 scratch
  void *dweight;       // [H] dtype out, nullable
};
hipError_t launch_rmsnorm_backward(const NormBwdArgs &a, int dtype, hipStream_t s);

// partial: [slices][T][E] fp32 scratch (one slice for fp32 layers).
hipError_t launch_router(const RouterArgs &a, int dtype, float *partial, hipStream_t s);
hipError_t launch_histogram(const int32_t *idx, const uint8_t *pad, int64_t T, int E,
                            int K, int32_t *blkcnt, int32_t *blkval, hipStream_t s);
// Expert offsets, counts and row tiles (a) and, with c, the slots of every
// pair (one block per kRouterTB tokens); without c only the former.
hipError_t launch_dispatch(const ScanArgs &a, const ScatterArgs *c, hipStream_t s);
hipError_t launch_gather(const void *x, int64_t row_bytes, const int32_t *slotof,
                         const uint8_t *pad, int64_t T, int K, void *xs, hipStream_t s);
// tile_rows: rows per listed row tile (the plan's BM); it selects the bf16
// configuration (kGemmStreamBM: streaming tiles, else the default tiles).
hipError_t launch_gemm_upgate(const GemmArgs &a, int max_tiles, int tile_rows, int dtype,
                              hipStream_t s);
hipError_t launch_gemm_down(const GemmArgs &a, int max_tiles, int tile_rows, int dtype,
                            hipStream_t s);
// The shared expert alone over rows 0 .. rows-1 of its A operand (every row
// real), with no tile list: a.cls[1] describes it; mode 0 ([up; gate] +
// SwiGLU) or 1 (down), bf16, the default tiles.
hipError_t launch_gemm_dense(const GemmArgs &a, int rows, int mode, hipStream_t s);
hipError_t launch_combine(const CombineArgs &a, int dtype, hipStream_t s);

// ---------------------------------------------------------------- backward

hipError_t launch_gemm_dgrad_down(const GemmArgs &a, int max_tiles, int tile_rows, int dtype,
                                  hipStream_t s);
hipError_t launch_gemm_dgrad_up_gate(const GemmArgs &a, int max_tiles, int tile_rows,
                                     int dtype, hipStream_t s);
hipError_t launch_gemm_wgrad(const GemmArgs &a, int E, int dtype, hipStream_t s);

struct BwdGatherArgs {
  const void *x;
  const void *dout;
  const float *wts;
  const int32_t *slotof;
  const int32_t *vidx;
  const uint8_t *pad;
  int64_t T;
  int H, K;
  void *xs;     // [T*K, H]: x by slot
  void *dys;    // [T*K, H]: w * dout by slot
  float *wslot; // [T*K]: w by slot
  void *xv;     // nullable, [T, H]: x by real-row index
  void *doutv;  // nullable, [T, H]: dout by real-row index
};
hipError_t launch_bwd_gather(const BwdGatherArgs &a, int dtype, hipStream_t s);

struct BwdCombineArgs {
  const float *dxs;      // [T*K, H] by slot
  const float *dxsh;     // [T, H] by real-row index
  const float *apart;    // [T*K, P]
  int P;
  const int32_t *slotof;
  const int32_t *idx;
  const int32_t *vidx;
  const float *wts;
  const float *w_router;  // [E, H]
  const uint8_t *pad;
  int64_t T;
  int H, K;
  float *dls;            // [T*K] logit gradient by slot
  void *dx;              // nullable
  float *dx_f32;         // nullable: dx kept in fp32 (by token) instead of dx
};
hipError_t launch_bwd_combine(const BwdCombineArgs &a, int dtype, hipStream_t s);

// part: [max_tiles, H] fp32 scratch (per row tile of the grouped GEMMs' list).
hipError_t launch_dw_router(const float *dls, const void *xs, const int4 *tiles,
                            const int32_t *gto, int max_tiles, int E, int H, int dtype,
                            float *part, float *dwr, hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);

// ---------------------------------------------------------------- entry points

// hi3_moe_forward on a workspace the caller of this function provides (the
// no-allocation entry point's static scratch); with validate_only the
// arguments are checked exactly as the forward checks them and nothing is
// enqueued.
int forward_single_stream(const void *x, const float *w_router, const void *w_up_gate,
                          const void *w_down, const void *w_shared_up_gate,
                          const void *w_shared_down, const uint8_t *pad_mask, int64_t T,
                          int32_t H, int32_t E, int32_t K, int32_t I, int32_t I_shared,
                          int32_t dtype, void *out, int32_t *topk_idx, float *topk_w,
                          int32_t *expert_counts, void *workspace, size_t workspace_bytes,
                          void *hip_stream, bool validate_only);

}  // namespace hi3
