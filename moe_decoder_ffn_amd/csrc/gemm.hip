// Grouped GEMMs of the experts.
//
//   [up; gate] projection with the SwiGLU epilogue: for every group (routed
//   expert e, or the shared expert) and each of its rows x,
//       h = SiLU(g) * u,  [u; g] = W13 x,  W13 [2I, H] with the up rows first
//   (layers API page, HunyuanSharedMLP: gate_and_up_proj holds [up; gate]);
//   h is stored in the layer dtype.
//   down projection: y = W2 h with W2 [H, I] (down_proj), y stored in fp32.
//
// Both operands are k-contiguous (activations [rows, k], weights [out, in]),
// so every MFMA operand fragment is one 16-byte LDS read.
//
// Work list: the row tiles of all groups (written on the device by the scan
// kernel, expert-major, the shared expert last) times the column tiles. The
// grid is sized for the largest possible tile count; surplus blocks exit.
// Schedule: hardware block b runs on XCD b % 8; each XCD is given one
// contiguous range of the work list, and inside a group the row tiles are
// the fastest index, so the blocks that share one weight slice run at the
// same time on the same XCD and its L2 serves the repeats.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace hi3 {

struct TileJob {
  int g;     // group: expert id, or E for the shared expert
  int row0;  // first row of the tile in the group's row space
  int rows;  // rows in the tile (<= BM)
  int nt;    // column tile
  int cls;   // 0 routed, 1 shared
};

// ntile_cols(c): column tiles of class c.
template <int MODE, int BN>
__device__ __forceinline__ int class_col_tiles(const GemmClass &c) {
  return MODE == 0 ? (c.N / 2 + BN / 2 - 1) / (BN / 2) : (c.N + BN - 1) / BN;
}

template <int MODE, int BN>
__device__ __forceinline__ bool resolve_job(const GemmArgs &a, TileJob &j) {
  const int ntiles = a.gto[a.E + 1];
  const int W = ntiles * a.NTn;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = (W + 7) >> 3;
  if (slot >= per) return false;
  const int L = xcd * per + slot;
  if (L >= W) return false;
  // group: the largest g with gto[g] * NTn <= L (empty groups have empty ranges)
  int lo = 0, hi = a.E;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.gto[mid] * a.NTn <= L) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int first = a.gto[g];
  const int cnt = a.gto[g + 1] - first;
  const int off = L - first * a.NTn;
  const int nt = off / cnt;
  const int mt = first + off % cnt;
  const int4 tile = a.tiles[mt];
  j.g = tile.x;
  j.row0 = tile.y;
  j.rows = tile.z;
  j.nt = nt;
  j.cls = tile.x == a.E ? 1 : 0;
  const GemmClass &c = j.cls ? a.cls[1] : a.cls[0];
  return nt < class_col_tiles<MODE, BN>(c);
}

// --------------------------------------------------------------- bf16 MFMA

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS copy of 16 bytes per lane; lane i writes
// lds_base + 16 i (lds_base must be the same for the whole wave).
// Written as the same three instructions the compiler emits for this copy
// (M0 = LDS base, one wait state, global_load_lds_dwordx4); the copy has no
// register result. It is issued this way because the compiler cannot tell
// which LDS stage an in-flight copy writes and would otherwise drain every
// copy (vmcnt(0)) before each LDS read; the kernel instead waits for exactly
// the stage it reads next (wait_vmem) and then synchronises the workgroup.
__device__ __forceinline__ void lds_dma16(const void *g, u32x4_t *lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t *)(lds_base))));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS layout of one operand stage: BK-wide k slices, CPR 16-byte chunks per
// row. The LDS serves 16 lanes x 16 bytes per cycle from 64 banks (256
// bytes), and an MFMA fragment read has 16 consecutive rows at one logical
// chunk; chunk c of row r is stored at position c ^ ((r / RPW) % CPR), where
// RPW rows fill one 256-byte bank window, so those 16 rows land in 16
// distinct 16-byte bank groups.
template <int BK>
struct LdsLayout {
  static constexpr int RB = BK * 2;        // bytes per row
  static constexpr int CPR = RB / 16;      // chunks per row
  static constexpr int RPW = 256 / RB;     // rows per 256-byte bank window
  static constexpr int RPC = 1024 / RB;    // rows per 1 KiB copy instruction
  __device__ static __forceinline__ int swz(int row) { return (row / RPW) % CPR; }
  __device__ static __forceinline__ int pos(int row, int chunk) {
    return row * CPR + (chunk ^ swz(row));
  }
};

// Workgroup barrier without a memory fence: __syncthreads() would also wait
// for every copy still in flight (the fence drains vmcnt), which would stop
// later stages from overlapping. Each wave has already waited for its own
// copies of the stage read next, and its LDS reads of the current stage have
// returned (the MFMAs consumed them). The signal fences and scheduling
// barriers keep the compiler from moving memory operations across it.
__device__ __forceinline__ void barrier_no_fence() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int S, int NST>
struct StageRing {
  static constexpr int prev = (S + NST - 1) % NST;
};

// Block: 2 x WN waves (the row half wm, the column group wn); tile BM rows x
// 256 weight rows (down: 256 output columns; [up; gate]: 128 up rows + the
// matching 128 gate rows); k step BK; NST-stage ring of LDS buffers filled by
// direct global -> LDS copies: while stage k is multiplied, the copies of
// the next NST - 1 stages are in flight. Each stage lives in its own LDS
// arrays. With WN = 4 (512 threads) two waves share each SIMD, so one
// wave's LDS waits overlap the other's MFMAs.
// Wave (wm, wn) owns rows [BM/2 wm, BM/2 (wm + 1)) and NI 32-row weight
// sub-tiles; with [up; gate] the first NI/2 are up rows and the last NI/2
// the gate rows of the same columns, so each lane holds u and g of the same
// (row, column) for the SwiGLU epilogue.
// The MFMA is issued as C^T = W x^T (v_mfma_f32_32x32x16_bf16 with the
// weight fragment first): result element v of lane l is token l % 32 and
// weight column 8 (v / 4) + 4 (l / 32) + v % 4 of the 32 x 32 sub-tile, so
// every lane holds runs of 4 adjacent output columns and stores them with
// one 8-byte (bf16) or 16-byte (fp32) write.
template <int MODE, int BM, int BK, int NST, int WN>
__global__ __launch_bounds__(128 * WN) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int BN = kGemmBN;
  using L = LdsLayout<BK>;
  constexpr int NW = 2 * WN;                // waves: 2 along rows x WN along columns
  constexpr int A_CP = BM / L::RPC / NW;    // copies per wave per stage
  constexpr int B_CP = BN / L::RPC / NW;
  constexpr int CPW = A_CP + B_CP;
  constexpr int MI = BM / 64;               // 32-row sub-tiles per wave
  constexpr int NI = BN / WN / 32;          // 32-column sub-tiles per wave
  constexpr int AE = BM * L::CPR, BE = BN * L::CPR;
  static_assert(BN == 256 && (BM == 128 || BM == 256) && (BK == 32 || BK == 64), "tile");
  static_assert(NST == 2 || NST == 3, "stages");
  static_assert(A_CP >= 1 && B_CP >= 1 && (NST - 2) * CPW < 64, "copy counts");
  static_assert(WN == 2 || WN == 4, "wave grid");
  __shared__ u32x4_t sA0[AE], sB0[BE], sA1[AE], sB1[BE];
  __shared__ u32x4_t sA2[NST > 2 ? AE : 1], sB2[NST > 2 ? BE : 1];

  TileJob j;
  if (!resolve_job<MODE, BN>(a, j)) return;
  const bool shared_cls = j.cls != 0;
  const uint16_t *A = static_cast<const uint16_t *>(shared_cls ? a.cls[1].A : a.cls[0].A);
  const int64_t lda = shared_cls ? a.cls[1].lda : a.cls[0].lda;
  const int32_t *arow = shared_cls ? a.cls[1].arow : a.cls[0].arow;
  const uint16_t *B = static_cast<const uint16_t *>(shared_cls ? a.cls[1].B : a.cls[0].B);
  const int64_t strideB = shared_cls ? 0 : a.cls[0].strideB;
  void *Cv = shared_cls ? a.cls[1].C : a.cls[0].C;
  const int64_t ldc = shared_cls ? a.cls[1].ldc : a.cls[0].ldc;
  const int N = shared_cls ? a.cls[1].N : a.cls[0].N;
  const int Kd = shared_cls ? a.cls[1].Kd : a.cls[0].Kd;
  B += static_cast<int64_t>(shared_cls ? 0 : j.g) * strideB;

  const int tid = threadIdx.x;
  const int wave = wave_uniform(tid >> 6);
  const int lane = tid & 63;
  const int r = lane & 31, g = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;

  // Copy q of this wave covers tile rows (wave * CP + q) * RPC + [0, RPC);
  // lane i takes row (wave * CP + q) * RPC + i / CPR and the logical chunk
  // that the swizzle stores at position i % CPR.
  int arow_src[A_CP];
#pragma unroll
  for (int q = 0; q < A_CP; ++q) {
    const int row = (wave * A_CP + q) * L::RPC + lane / L::CPR;
    const int rr = min(row, j.rows - 1);  // tail rows reread a real row
    const int ri = j.row0 + rr;
    arow_src[q] = arow ? arow[ri] : ri;
  }
  auto issue = [&](int kc, u32x4_t *la, u32x4_t *lb) {
    const int ko = kc * BK;
#pragma unroll
    for (int q = 0; q < A_CP; ++q) {
      const int row = (wave * A_CP + q) * L::RPC + lane / L::CPR;
      const int c = (lane % L::CPR) ^ L::swz(row);
      lds_dma16(A + static_cast<int64_t>(arow_src[q]) * lda + ko + c * 8,
                la + (wave * A_CP + q) * 64);
    }
#pragma unroll
    for (int q = 0; q < B_CP; ++q) {
      const int row = (wave * B_CP + q) * L::RPC + lane / L::CPR;
      const int c = (lane % L::CPR) ^ L::swz(row);
      int brow;
      if (MODE == 0) {
        const int Ih = N / 2;
        const int col = min(j.nt * (BN / 2) + (row & (BN / 2 - 1)), Ih - 1);
        brow = row < BN / 2 ? col : Ih + col;
      } else {
        brow = min(j.nt * BN + row, N - 1);
      }
      lds_dma16(B + static_cast<int64_t>(brow) * Kd + ko + c * 8,
                lb + (wave * B_CP + q) * 64);
    }
  };

  // weight rows of the wave's sub-tiles: with [up; gate] the first NI/2 are
  // up rows and the last NI/2 the gate rows of the same columns
  int nrow[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    if (MODE == 0)
      nrow[ni] = (ni / (NI / 2)) * (BN / 2) + wn * (BN / 2 / WN) + (ni % (NI / 2)) * 32;
    else
      nrow[ni] = wn * (BN / WN) + ni * 32;
  }

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  auto compute = [&](const u32x4_t *la, const u32x4_t *lb) {
    bf16x8_t af[2][MI], bf[2][NI];
    auto load = [&](int buf, int s) {
      const int ch = 2 * s + g;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[buf][mi] = __builtin_bit_cast(bf16x8_t, la[L::pos(wm * (BM / 2) + mi * 32 + r, ch)]);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        bf[buf][ni] = __builtin_bit_cast(bf16x8_t, lb[L::pos(nrow[ni] + r, ch)]);
    };
    load(0, 0);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int cur = s & 1;
      if (s + 1 < BK / 16) load(cur ^ 1, s + 1);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[cur][ni], af[cur][mi],
                                                                acc[mi][ni], 0, 0, 0);
    }
#if HI3_GEMM_SCHED
    // Issue order: the first sub-step's fragment reads, then for each later
    // sub-step its reads one by one between the MFMAs of the sub-step before,
    // so LDS latency hides behind matrix work.
    constexpr int NR = MI + NI;       // fragment reads per sub-step
    constexpr int NM = MI * NI;       // MFMAs per sub-step
    static_assert(NR <= NM, "reads fit between MFMAs");
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int s = 0; s + 1 < BK / 16; ++s) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
#endif
  };

  auto stage_a = [&](auto S) -> u32x4_t * {
    if constexpr (decltype(S)::value == 0) return sA0;
    else if constexpr (decltype(S)::value == 1) return sA1;
    else return sA2;
  };
  auto stage_b = [&](auto S) -> u32x4_t * {
    if constexpr (decltype(S)::value == 0) return sB0;
    else if constexpr (decltype(S)::value == 1) return sB1;
    else return sB2;
  };

  const int nk = Kd / BK;
  // One k step from stage S: start the copy NST - 1 steps ahead into the
  // stage read in the previous step, multiply, then wait for the next
  // step's copy (counted: later copies may stay in flight) and synchronise.
  auto step = [&](auto S, int k) {
    constexpr int s = decltype(S)::value;
    constexpr int p = StageRing<s, NST>::prev;
    if (k + NST - 1 < nk)
      issue(k + NST - 1, stage_a(std::integral_constant<int, p>{}),
            stage_b(std::integral_constant<int, p>{}));
    __builtin_amdgcn_sched_barrier(0);
    compute(stage_a(S), stage_b(S));
    if (NST == 3 && k + 2 < nk)
      wait_vmem<(NST - 2) * CPW>();
    else
      wait_vmem<0>();
    barrier_no_fence();
  };

  issue(0, sA0, sB0);
  if (NST == 3 && nk > 1) issue(1, sA1, sB1);
  wait_vmem<NST == 3 ? CPW : 0>();  // stage 0 landed (stage 1 may be in flight)
  barrier_no_fence();
  int kc = 0;
  for (; kc + NST <= nk; kc += NST) {
    step(std::integral_constant<int, 0>{}, kc);
    step(std::integral_constant<int, 1>{}, kc + 1);
    if constexpr (NST == 3) step(std::integral_constant<int, 2>{}, kc + 2);
  }
  if (kc < nk) step(std::integral_constant<int, 0>{}, kc);
  if (kc + 1 < nk) step(std::integral_constant<int, 1>{}, kc + 1);

  if (MODE == 0) {
    const int Ih = N / 2;
    uint16_t *C = static_cast<uint16_t *>(Cv);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * (BM / 2) + mi * 32 + r;
      if (row >= j.rows) continue;
      uint16_t *crow = C + (static_cast<int64_t>(j.row0) + row) * ldc;
#pragma unroll
      for (int p = 0; p < NI / 2; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = j.nt * (BN / 2) + wn * (BN / 2 / WN) + p * 32 + 8 * q + 4 * g;
          if (col >= Ih) continue;
          float hv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float u = acc[mi][p][4 * q + e];
            const float gt = acc[mi][p + NI / 2][4 * q + e];
            // SiLU(g) * u = g * u / (1 + exp(-g))
            hv[e] = gt * u * __builtin_amdgcn_rcpf(1.0f + __expf(-gt));
          }
          u32x2_t o;
          o[0] = pack_bf16x2(hv[0], hv[1]);
          o[1] = pack_bf16x2(hv[2], hv[3]);
          *reinterpret_cast<u32x2_t *>(crow + col) = o;
        }
    }
  } else {
    float *C = static_cast<float *>(Cv);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * (BM / 2) + mi * 32 + r;
      if (row >= j.rows) continue;
      float *crow = C + (static_cast<int64_t>(j.row0) + row) * ldc;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = j.nt * BN + wn * (BN / WN) + ni * 32 + 8 * q + 4 * g;
          if (col >= N) continue;
          f32x4_t o = {acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                       acc[mi][ni][4 * q + 3]};
          *reinterpret_cast<f32x4_t *>(crow + col) = o;
        }
    }
  }
}

// --------------------------------------------------------------- fp32

// fp32 layers: LDS-tiled FMA, 64 rows x 64 weight rows per block ([up; gate]:
// 32 up + the matching 32 gate rows), k step 16; thread (ty, tx) owns rows
// 4ty..4ty+3 and four weight columns.
template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BM = kGemmF32BM, BN = kGemmF32BN, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  TileJob j;
  if (!resolve_job<MODE, BN>(a, j)) return;
  const bool shared_cls = j.cls != 0;
  const GemmClass &c = shared_cls ? a.cls[1] : a.cls[0];
  const float *A = static_cast<const float *>(c.A);
  const float *B = static_cast<const float *>(c.B) +
                   static_cast<int64_t>(shared_cls ? 0 : j.g) * c.strideB;
  const int N = c.N, Kd = c.Kd;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;

  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int arr = min(lrow, j.rows - 1);
  const int64_t ari = static_cast<int64_t>(j.row0) + arr;
  const float *aptr = A + (c.arow ? static_cast<int64_t>(c.arow[ari]) : ari) * c.lda + lk;
  int brow;
  if (MODE == 0) {
    const int Ih = N / 2;
    const int col = min(j.nt * (BN / 2) + (lrow & (BN / 2 - 1)), Ih - 1);
    brow = lrow < BN / 2 ? col : Ih + col;
  } else {
    brow = min(j.nt * BN + lrow, N - 1);
  }
  const float *bptr = B + static_cast<int64_t>(brow) * Kd + lk;

  int bcol[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    bcol[q] = MODE == 0 ? (q >> 1) * (BN / 2) + tx * 2 + (q & 1) : tx * 4 + q;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = 0.0f;

  for (int k0 = 0; k0 < Kd; k0 += BK) {
    const f32x4_t av = *reinterpret_cast<const f32x4_t *>(aptr + k0);
    const f32x4_t bv = *reinterpret_cast<const f32x4_t *>(bptr + k0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      As[lk + q][lrow] = av[q];
      Bs[lk + q][lrow] = bv[q];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av4[4], bv4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av4[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int q = 0; q < 4; ++q) bv4[q] = Bs[kk][bcol[q]];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(av4[i], bv4[q], acc[i][q]);
    }
    __syncthreads();
  }

  float *C = static_cast<float *>(c.C);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (row >= j.rows) continue;
    float *crow = C + (static_cast<int64_t>(j.row0) + row) * c.ldc;
    if (MODE == 0) {
      const int Ih = N / 2;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = j.nt * (BN / 2) + tx * 2 + q;
        const float u = acc[i][q], gt = acc[i][2 + q];
        if (col < Ih) crow[col] = gt / (1.0f + expf(-gt)) * u;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = j.nt * BN + tx * 4 + q;
        if (col < N) crow[col] = acc[i][q];
      }
    }
  }
}

// --------------------------------------------------------------- launches

static int col_tiles_host(int N, int BN, bool upgate) {
  return upgate ? (N / 2 + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
}

static hipError_t launch_gemm(GemmArgs a, int max_tiles, int dtype, bool upgate,
                              hipStream_t s) {
  const int BN = dtype == kBF16 ? kGemmBN : kGemmF32BN;
  a.NTn = std::max(col_tiles_host(a.cls[0].N, BN, upgate), col_tiles_host(a.cls[1].N, BN, upgate));
  const int64_t work = static_cast<int64_t>(max_tiles) * a.NTn;
  const unsigned grid = static_cast<unsigned>((work + 7) / 8 * 8);
  if (grid == 0) return hipSuccess;
  if (dtype == kBF16) {
    if (upgate)
      hipLaunchKernelGGL((gemm_bf16_kernel<0, kGemmBM, kGemmBK, kGemmStages, kGemmWN>),
                         dim3(grid), dim3(128 * kGemmWN), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<1, kGemmBM, kGemmBK, kGemmStages, kGemmWN>),
                         dim3(grid), dim3(128 * kGemmWN), 0, s, a);
  } else {
    if (upgate)
      hipLaunchKernelGGL(gemm_f32_kernel<0>, dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(gemm_f32_kernel<1>, dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_upgate(const GemmArgs &a, int max_tiles, int dtype, hipStream_t s) {
  return launch_gemm(a, max_tiles, dtype, true, s);
}

hipError_t launch_gemm_down(const GemmArgs &a, int max_tiles, int dtype, hipStream_t s) {
  return launch_gemm(a, max_tiles, dtype, false, s);
}

}  // namespace hi3
