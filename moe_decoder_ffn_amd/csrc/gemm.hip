// Grouped GEMMs of the experts.
//
//   [up; gate] projection with the SwiGLU epilogue: for every group (routed
//   expert e, or the shared expert) and each of its rows x,
//       h = SiLU(g) * u,  [u; g] = W13 x,  W13 [2I, H] with the up rows first
//   (layers API page, HunyuanSharedMLP: gate_and_up_proj holds [up; gate]);
//   h is stored in the layer dtype.
//   down projection: y = W2 h with W2 [H, I] (down_proj), y stored in fp32.
//
// Backward (the gradient of sum(dout . out) with the routes held fixed; the
// pages' fine-tuning, HunyuanImage-3.0 model-coverage page, "Train"):
//   mode 2: dh = w W2^T dout per routed row (w applied in fp32), and in the epilogue
//       du = dh SiLU(g), dg = dh u SiLU'(g) from the stored u, g, plus the
//       partial sums of dh . h that give the router's gradient;
//   mode 3: dx = W13^T [du; dg] per row, fp32;
//   mode 4: weight gradients dW2 = sum dy h^T, dW13 = sum [du; dg] x^T over
//       each expert's rows, in the layer dtype.
//
// Forward operands are k-contiguous (activations [rows, k], weights
// [out, in]): every MFMA operand fragment is one 16-byte LDS read. The
// backward's weights in modes 2 and 3, and both operands of mode 4, are
// k-major (row k holds the n or m values): they are copied to LDS as stored
// and their fragments are read with the transposing LDS read of gfx950, so no
// transposed copy is ever written to HBM.
//
// Work list: the row tiles of all groups (written on the device by the
// dispatch kernel, expert-major, the shared expert last) times the column
// tiles; the gradient through the down projection (mode 2) runs each listed
// row tile as `split` blocks of sub_rows rows. The grid is sized for the largest
// possible tile count; surplus blocks exit. Block b runs on XCD b % 8 (the
// hardware's round-robin); how jobs map to blocks is resolve_job's. When no
// row is padding, the forward runs the shared expert alone instead, as dense
// launches over its rows 0 .. T-1 with no tile list (gemm_bf16_dense_kernel,
// resolve_dense), on a stream beside the routing.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.h"

namespace hi3 {

struct TileJob {
  int g;       // group: expert id, or E for the shared expert
  int row0;    // first row of the tile in the group's row space (mode 4: first output row)
  int rows;    // rows in the tile (<= BM)
  int nt;      // column tile
  int cls;     // 0 routed, 1 shared
  int kstart;  // mode 4: first row of the group in A and B
  int kcount;  // mode 4: the group's rows (the reduction length)
};

// ntile_cols(c): column tiles of class c.
template <int MODE, int BN>
__device__ __forceinline__ int class_col_tiles(const GemmClass &c) {
  return MODE == 0 ? (c.N / 2 + BN / 2 - 1) / (BN / 2) : (c.N + BN - 1) / BN;
}

// The job list: groups in order. Modes 0, 1 and 2: within a group, chunks of
// kGemmColChunk column tiles, each chunk taking every row (sub-)tile of the
// group, row tile major, so the blocks that share a weight tile or a row
// tile's rows are neighbours; block b runs on XCD b % 8, and XCD x takes
// the contiguous part [x per, (x + 1) per) of the list (per = ceil(jobs /
// 8)): a group's weights and rows are fetched into one XCD's L2 (two at a
// part boundary), where the neighbours run at the same time. Mode 3
// (measured faster so): row tile major, column fastest, block b = job b.
template <int MODE, int BN>
__device__ __forceinline__ bool resolve_job(const GemmArgs &a, TileJob &j) {
  const int ntiles = a.gto[a.E + 1];
  const int SP = a.split;
  const int W = ntiles * SP * a.NTn;
  constexpr bool XM = MODE <= 2;
  const int per = (W + 7) / 8;
  if (XM && static_cast<int>(blockIdx.x) / 8 >= per) return false;
  const int L = XM ? (blockIdx.x % 8) * per + blockIdx.x / 8 : blockIdx.x;
  if (L >= W) return false;
  // group: the largest g with gto[g] * SP * NTn <= L (empty groups have
  // empty ranges)
  int lo = 0, hi = a.E;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.gto[mid] * SP * a.NTn <= L) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int first = a.gto[g] * SP;              // first row sub-tile of the group
  const int off = L - first * a.NTn;
  const int R = a.gto[g + 1] * SP - first;      // row sub-tiles of the group
  constexpr int CC = XM ? kGemmColChunk : (1 << 30);  // one chunk: column fastest
  const int full = a.NTn / CC;                  // whole chunks; the last may be narrower
  int nt, rt;
  if (off < full * CC * R) {
    const int c = off / (CC * R), rem = off - c * CC * R;
    rt = rem / CC;
    nt = c * CC + rem % CC;
  } else {
    const int cw = a.NTn - full * CC, rem = off - full * CC * R;
    rt = rem / cw;
    nt = full * CC + rem % cw;
  }
  const int ms = first + rt;
  const int4 tile = a.tiles[ms / SP];
  const int part = ms % SP;
  j.g = tile.x;
  j.row0 = tile.y + part * a.sub_rows;
  j.rows = min(a.sub_rows, tile.z - part * a.sub_rows);
  if (j.rows <= 0) return false;  // a short tile's empty part
  j.nt = nt;
  j.cls = tile.x == a.E ? 1 : 0;
  const GemmClass &c = j.cls ? a.cls[1] : a.cls[0];
  return nt < class_col_tiles<MODE, BN>(c);
}

// A dense launch (modes 0 and 1): class 1 alone over rows 0 .. dense_rows-1,
// in row tiles of BM, with resolve_job's job order (chunks of kGemmColChunk
// column tiles over every row tile, each XCD a contiguous part).
template <int MODE, int BM, int BN>
__device__ __forceinline__ bool resolve_dense(const GemmArgs &a, TileJob &j) {
  const int R = (a.dense_rows + BM - 1) / BM;
  const int W = R * a.NTn;
  const int per = (W + 7) / 8;
  if (static_cast<int>(blockIdx.x) / 8 >= per) return false;
  const int L = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (L >= W) return false;
  constexpr int CC = kGemmColChunk;
  const int full = a.NTn / CC;
  int nt, rt;
  if (L < full * CC * R) {
    const int c = L / (CC * R), rem = L - c * CC * R;
    rt = rem / CC;
    nt = c * CC + rem % CC;
  } else {
    const int cw = a.NTn - full * CC, rem = L - full * CC * R;
    rt = rem / cw;
    nt = full * CC + rem % cw;
  }
  j.g = 0;
  j.cls = 1;
  j.row0 = rt * BM;
  j.rows = min(BM, a.dense_rows - j.row0);
  j.nt = nt;
  return nt < class_col_tiles<MODE, BN>(a.cls[1]);
}

// Mode 4: the shared group's output tiles come first (they reduce over every
// real row, the longest jobs); then the routed experts, placed so that all
// tiles of expert g run on XCD g % 8 (block b runs on XCD b % 8), where that
// XCD's L2 serves the expert's rows to all of its tiles.
template <int BM, int BN>
__device__ __forceinline__ bool resolve_wgrad(const GemmArgs &a, TileJob &j) {
  int b = blockIdx.x;
  int cls, g, tt;
  if (b < a.wg_shared_blocks) {
    cls = 1;
    g = a.E;
    tt = b;
  } else {
    b -= a.wg_shared_blocks;
    const GemmClass &c0 = a.cls[0];
    const int tpe = ((c0.M + BM - 1) / BM) * ((c0.N + BN - 1) / BN);
    const int li = b / 8;
    cls = 0;
    g = b % 8 + 8 * (li / tpe);
    tt = li % tpe;
    if (g >= a.E) return false;
  }
  const GemmClass &c = a.cls[cls];
  const int NT = (c.N + BN - 1) / BN, MT = (c.M + BM - 1) / BM;
  if (tt >= MT * NT) return false;
  // tiles in groups of GR row tiles, down the group's rows first and then
  // across its columns, so the tiles resident together read a few row
  // slices of A and a few column slices of B (which then stay in the L2)
  constexpr int GR = kWgradGroupRows;
  const int grp = tt / (GR * NT), rem = tt - grp * GR * NT;
  const int gr = min(GR, MT - grp * GR);  // rows in this group (the last may have fewer)
  j.g = g;
  j.cls = cls;
  j.row0 = (grp * GR + rem % gr) * BM;
  j.rows = min(BM, c.M - j.row0);
  j.nt = rem / gr;
  j.kstart = cls ? 0 : a.goff[g];
  j.kcount = cls ? *a.nreal : a.gcnt[g];
  return true;
}

// --------------------------------------------------------------- bf16 MFMA

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS copy of 16 bytes per lane; lane i writes
// lds_base + 16 i (lds_base must be the same for the whole wave). The copy
// has no register result; the kernel waits for it with counted vmcnt waits
// (wait_vmem) before the workgroup barrier that publishes its stage.
// It is issued as the three instructions the compiler's own global_load_lds
// builtin expands to (M0 = LDS base, one wait state,
// global_load_lds_dwordx4), written as inline assembly that declares M0
// clobbered. With the builtin, the compiler cannot order the copy against
// the kernel's LDS reads and drains every outstanding LDS read (lgkmcnt(0))
// before each MFMA that consumes a fragment, instead of waiting for the
// fragment's own read (measured: 2-3% slower forward GEMMs); the backward's
// transposing reads also get a vmcnt(0) drain each. The build disassembles
// every kernel that uses this copy and fails if anything else in it reads
// or writes M0 (moe_decoder_ffn_amd/build.py).
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

// LDS layout of a k-major operand stage: BK rows of k, W columns (2 W bytes
// per row). 16-byte chunk c of row k is stored at chunk
// ((c / 4) ^ (k % 4)) * 4 + c % 4: the same 64-byte column unit of four
// consecutive k rows lands in the four distinct 64-byte windows of the
// 256-byte bank cycle, which is what a transposing fragment read touches.
template <int W>
struct LdsKM {
  static constexpr int CPR = W / 8;           // 16-byte chunks per row
  static constexpr int RPC = 1024 / (W * 2);  // rows per 1 KiB copy instruction
  static_assert(W == 128 || W == 256, "k-major tile width");
  __device__ static __forceinline__ int pos(int k, int c) {
    return k * CPR + (((c >> 2) ^ (k & 3)) << 2) + (c & 3);
  }
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// One MFMA operand fragment (lane l: k = 16 s + 8 (l / 32) + 0..7 of column
// cb + l % 32) from a k-major stage, with two ds_read_b64_tr_b16. That read
// works on groups of 16 lanes: lane i of a group receives element i % 4 of
// the 8 bytes that lane 4 j + i / 4 addressed, as its element j. So lane q
// of a group addresses row k0 + q / 4 at columns c0 + 4 (q % 4) .. + 3, and
// receives rows k0 .. k0 + 3 of column c0 + q.
template <int W>
__device__ __forceinline__ bf16x8_t read_frag_km(const u32x4_t *stage, int s, int cb, int lane) {
  using LK = LdsKM<W>;
  const int q = lane & 15;
  const int k0 = 16 * s + 8 * (lane >> 5) + (q >> 2);
  const int col = cb + 16 * ((lane >> 4) & 1) + 4 * (q & 3);
  const int c = col >> 3;
  const char *base = reinterpret_cast<const char *>(stage) + (col & 4) * 2;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t *)(const_cast<char *>(base + LK::pos(k0, c) * 16)));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t *)(const_cast<char *>(base + LK::pos(k0 + 4, c) * 16)));
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

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

// Workgroup barrier of the epilogues, which stage the tile in the idle LDS
// ring: waits for this wave's LDS operations only (its staging writes, or
// its reads of the staged chunk), so the wave's global stores and loads stay
// in flight across it. __syncthreads() would wait for them to complete (its
// fence drains vmcnt), which exposed the store latency at every chunk.
__device__ __forceinline__ void epi_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// f(integral_constant<int, i>) for i = 0 .. N - 1, unrolled at compile time.
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

template <int S, int NST>
struct StageRing {
  static constexpr int prev = (S + NST - 1) % NST;
};

// Block: 2 x WN waves (the row half wm, the column group wn); tile BM rows x
// 256 weight rows (down: 256 output columns; [up; gate]: 128 up rows + the
// matching 128 gate rows); k step BK; NST-stage ring of LDS buffers filled by
// direct global -> LDS copies: while stage k is multiplied, the copies of
// the next NST - 1 stages are in flight. The stages are slices of one LDS
// array, which the epilogues reuse once the ring is idle. With WN = 4 (512
// threads) two waves share each SIMD, so one wave's LDS waits overlap the
// other's MFMAs.
// Wave (wm, wn) owns rows [BM/2 wm, BM/2 (wm + 1)) and NI 32-row weight
// sub-tiles; with [up; gate] the first NI/2 are up rows and the last NI/2
// the gate rows of the same columns, so each lane holds u and g of the same
// (row, column) for the SwiGLU epilogue.
// The MFMA is issued as C^T = W x^T (v_mfma_f32_32x32x16_bf16 with the
// weight fragment first): result element v of lane l is token l % 32 and
// weight column 8 (v / 4) + 4 (l / 32) + v % 4 of the 32 x 32 sub-tile, so
// every lane holds runs of 4 adjacent output columns and stores them with
// one 8-byte (bf16) or 16-byte (fp32) write. Mode 4 has the same shape with
// output rows m in place of tokens and output columns n in place of weight
// rows.
// The tile body: BM is the row capacity of this body (the LDS stages may be
// larger); the stage arrays are the kernel's.
// DB (8-wave blocks with a 2-stage ring whose B operand is a weight: the
// forward GEMMs and the backward's dx GEMM): a third B stage; the B copies
// (the weights, whose latency the L2 does not hide) run two steps ahead,
// the A copies one.
template <int MODE, int BM, int BK, int NST, int WN, bool DB = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs &a, const TileJob &j, u32x4_t *sA0,
                                          u32x4_t *sB0, u32x4_t *sA1, u32x4_t *sB1,
                                          u32x4_t *sA2, u32x4_t *sB2, u32x4_t *sA3,
                                          u32x4_t *sB3, u32x4_t *sA4, u32x4_t *sB4) {
  constexpr int BN = kGemmBN;
  constexpr bool AT = MODE == 4;  // A stage k-major
  constexpr bool BT = MODE >= 2;  // B stage k-major
  using L = LdsLayout<BK>;
  constexpr int NW = 2 * WN;                // waves: 2 along rows x WN along columns
  constexpr int A_CP = BM * BK * 2 / 1024 / NW;  // copies per wave per stage
  constexpr int B_CP = BN * BK * 2 / 1024 / NW;
  constexpr int CPW = A_CP + B_CP;
  constexpr int MI = BM / 64;               // 32-row sub-tiles per wave
  constexpr int NI = BN / WN / 32;          // 32-column sub-tiles per wave
  static_assert(BN == 256 && BM % 64 == 0 && BM <= 256 && (BK == 32 || BK == 64), "tile");
  static_assert(!AT || BM == 128 || BM == 256, "k-major A tile");
  static_assert(!(AT || BT) || BK == 32 || BK == 64, "k-major k step");
  static_assert(NST >= 2 && NST <= 5, "stages");
  static_assert(!DB || (NST == 2 && !AT), "deep B ring: 2 + 3 stages, k-contiguous A");
  static_assert(BM * BK * 2 % (1024 * NW) == 0 && BN * BK * 2 % (1024 * NW) == 0,
                "each wave copies a whole number of 1 KiB blocks");
  static_assert(A_CP >= 1 && B_CP >= 1 && (NST - 2) * CPW < 64, "copy counts");
  static_assert(WN == 2 || WN == 4, "wave grid");

  const bool shared_cls = j.cls != 0;
  const GemmClass &cl = shared_cls ? a.cls[1] : a.cls[0];
  const uint16_t *A = static_cast<const uint16_t *>(cl.A);
  const int64_t lda = cl.lda;
  const int32_t *arow = cl.arow;
  const uint16_t *B = static_cast<const uint16_t *>(cl.B);
  const int64_t strideB = shared_cls ? 0 : cl.strideB;
  void *Cv = cl.C;
  const int64_t ldc = cl.ldc;
  const int N = cl.N;
  const int Kd = cl.Kd;
  const int64_t ldb = cl.ldb;
  if constexpr (!AT) B += static_cast<int64_t>(shared_cls ? 0 : j.g) * strideB;

  const int tid = threadIdx.x;
  const int wave = wave_uniform(tid >> 6);
  const int lane = tid & 63;
  const int r = lane & 31, g = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;

  // k-contiguous A: copy q of this wave covers tile rows
  // (wave * CP + q) * RPC + [0, RPC); lane i takes row
  // (wave * CP + q) * RPC + i / CPR and the logical chunk that the swizzle
  // stores at position i % CPR.
  int arow_src[AT ? 1 : A_CP];
  if constexpr (!AT) {
#pragma unroll
    for (int q = 0; q < A_CP; ++q) {
      const int row = (wave * A_CP + q) * L::RPC + lane / L::CPR;
      const int rr = min(row, j.rows - 1);  // tail rows reread a real row
      const int ri = j.row0 + rr;
      arow_src[q] = arow ? arow[ri] : ri;
    }
  }
  // k-major stage of width W: copy ci covers k rows ci * RPC + [0, RPC);
  // lane i takes row ci * RPC + i / CPR and the logical chunk stored at
  // position i % CPR. Source row pointer for global k row kg: rowp(kg).
  auto km_copy = [&](auto Wc, int ci, int col0, int cmax, u32x4_t *stage,
                     auto rowp) __attribute__((always_inline)) {
    constexpr int W = decltype(Wc)::value;
    using LK = LdsKM<W>;
    const int krow = ci * LK::RPC + lane / LK::CPR;
    const int p = lane % LK::CPR;
    const int c = (((p >> 2) ^ (krow & 3)) << 2) | (p & 3);
    const int col = min(col0 + c * 8, cmax - 8);
    lds_dma16(rowp(krow, col), stage + ci * 64);
  };
  const uint16_t *zrow = static_cast<const uint16_t *>(a.zrow) + 8 * (lane & 31);
  // Copies [q0, q1) of this wave (A copies first, then B) for k step kc.
  // (DB: the B copies are of step kcb; okA / okB select the operands)
  auto issue_range = [&](int kc, u32x4_t *la, u32x4_t *lb, auto Q0, auto Q1, int kcb = -1,
                         bool okA = true, bool okB = true) __attribute__((always_inline)) {
    constexpr int q0 = decltype(Q0)::value, q1 = decltype(Q1)::value;
    const int ko = kc * BK;
    const int kob = (DB ? kcb : kc) * BK;
#pragma unroll
    for (int q = 0; q < A_CP; ++q) {
      if (q < q0 || q >= q1) continue;
      if (!okA) continue;
      if constexpr (AT) {
        km_copy(std::integral_constant<int, BM>{}, wave * A_CP + q, j.row0, cl.M, la,
                [&](int krow, int col) {
                  const int kg = ko + krow;
                  return kg < j.kcount ? A + static_cast<int64_t>(j.kstart + kg) * lda + col
                                       : zrow;
                });
      } else {
        const int row = (wave * A_CP + q) * L::RPC + lane / L::CPR;
        const int c = (lane % L::CPR) ^ L::swz(row);
        lds_dma16(A + static_cast<int64_t>(arow_src[q]) * lda + ko + c * 8,
                  la + (wave * A_CP + q) * 64);
      }
    }
#pragma unroll
    for (int q = 0; q < B_CP; ++q) {
      if (A_CP + q < q0 || A_CP + q >= q1) continue;
      if (!okB) continue;
      if constexpr (AT) {
        km_copy(std::integral_constant<int, BN>{}, wave * B_CP + q, j.nt * BN, N, lb,
                [&](int krow, int col) {
                  const int kg = ko + krow;
                  return kg < j.kcount ? B + static_cast<int64_t>(j.kstart + kg) * ldb + col
                                       : zrow;
                });
      } else if constexpr (BT) {
        km_copy(std::integral_constant<int, BN>{}, wave * B_CP + q, j.nt * BN, N, lb,
                [&](int krow, int col) { return B + static_cast<int64_t>(kob + krow) * ldb + col; });
      } else {
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
        lds_dma16(B + static_cast<int64_t>(brow) * Kd + kob + c * 8,
                  lb + (wave * B_CP + q) * 64);
      }
    }
  };
  auto issue = [&](int kc, u32x4_t *la, u32x4_t *lb) __attribute__((always_inline)) {
    issue_range(kc, la, lb, std::integral_constant<int, 0>{},
                std::integral_constant<int, CPW>{});
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


  // One k step from LDS stage (la, lb): NSUB = BK / 16 sub-steps; sub-step
  // s multiplies fragments read during sub-step s - 1, in MI groups of NI
  // MFMAs (one group per 32-row A fragment), and reads the fragments of
  // sub-step s + 1 between those MFMAs. The copies of step kn (into stage
  // pa, pb) are issued one per group (more if there are more copies than
  // groups), from the second group on: a copy waits in the vector-memory
  // queue while the MFMAs just issued keep the matrix unit busy, whereas a
  // burst of copies would stall the wave (and its matrix work) until the
  // whole burst was accepted.
  constexpr int NSUB = BK / 16;
  constexpr int NR = MI + NI;   // fragment reads per sub-step
  constexpr int NG = NSUB * MI; // MFMA groups per step
  static_assert(NG >= 2, "copies go after the first MFMA group");
  // copies per group: one while they last (PER = 1) unless there are more
  // copies than groups after the first
  constexpr int PER = (CPW + NG - 2) / (NG - 1);
  // (DB: the B copies are of step knb, into stage pbb)
  auto compute = [&](const u32x4_t *la, const u32x4_t *lb, bool pre, int kn, u32x4_t *pa,
                     u32x4_t *pb, int knb = 0, u32x4_t *pbb = nullptr)
      __attribute__((always_inline)) {
    bf16x8_t af[2][MI], bf[2][NI];
    // fragment read i (A fragments first, then B) of sub-step s into buffer buf
    auto read = [&](int buf, int s, int i) __attribute__((always_inline)) {
      const int ch = 2 * s + g;
      if (i < MI) {
        if constexpr (AT)
          af[buf][i] = read_frag_km<BM>(la, s, wm * (BM / 2) + i * 32, lane);
        else
          af[buf][i] = __builtin_bit_cast(bf16x8_t, la[L::pos(wm * (BM / 2) + i * 32 + r, ch)]);
      } else {
        if constexpr (BT)
          bf[buf][i - MI] = read_frag_km<BN>(lb, s, nrow[i - MI], lane);
        else
          bf[buf][i - MI] = __builtin_bit_cast(bf16x8_t, lb[L::pos(nrow[i - MI] + r, ch)]);
      }
    };
#pragma unroll
    for (int i = 0; i < NR; ++i) read(0, 0, i);
    static_for<NSUB>([&](auto Sv) __attribute__((always_inline)) {
      constexpr int s = decltype(Sv)::value;
      constexpr int cur = s & 1;
      static_for<MI>([&](auto Mv) __attribute__((always_inline)) {
        constexpr int mi = decltype(Mv)::value;
        constexpr int grp = s * MI + mi;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[cur][ni], af[cur][mi],
                                                                acc[mi][ni], 0, 0, 0);
        if constexpr (s + 1 < NSUB) {
          constexpr int i0 = mi * NR / MI, i1 = (mi + 1) * NR / MI;
#pragma unroll
          for (int i = i0; i < i1; ++i) read(cur ^ 1, s + 1, i);
          // MFMA, read, MFMA, read, ...
          constexpr int NT_ = NI > i1 - i0 ? NI : i1 - i0;
          static_for<NT_>([&](auto Tv) __attribute__((always_inline)) {
            constexpr int t = decltype(Tv)::value;
            if constexpr (t < NI) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            // LDS read instructions of fragment read i0 + t (two if k-major)
            constexpr int nrd = ((i0 + t) < MI ? AT : BT) ? 2 : 1;
            if constexpr (t < i1 - i0) __builtin_amdgcn_sched_group_barrier(0x100, nrd, 0);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
        constexpr int q0 = (grp - 1) * PER < CPW ? (grp - 1) * PER : CPW;
        constexpr int q1 = grp * PER < CPW ? grp * PER : CPW;
        if constexpr (grp >= 1 && q0 < q1) {
          if constexpr (DB)
            issue_range(kn, pa, pbb, std::integral_constant<int, q0>{},
                        std::integral_constant<int, q1>{}, knb);
          else if (pre)
            issue_range(kn, pa, pb, std::integral_constant<int, q0>{},
                        std::integral_constant<int, q1>{});
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    });
  };

  auto stage_a = [&](auto S) __attribute__((always_inline)) -> u32x4_t * {
    constexpr int v = decltype(S)::value;
    if constexpr (v == 0) return sA0;
    else if constexpr (v == 1) return sA1;
    else if constexpr (v == 2) return sA2;
    else if constexpr (v == 3) return sA3;
    else return sA4;
  };
  auto stage_b = [&](auto S) __attribute__((always_inline)) -> u32x4_t * {
    constexpr int v = decltype(S)::value;
    if constexpr (v == 0) return sB0;
    else if constexpr (v == 1) return sB1;
    else if constexpr (v == 2) return sB2;
    else if constexpr (v == 3) return sB3;
    else return sB4;
  };
  // Wait until at most n (0 <= n <= NST - 2) later stages of this wave's
  // copies are still in flight; copies complete in issue order.
  auto wait_stages = [&](int n) __attribute__((always_inline)) {
    if constexpr (NST > 4) if (n >= 3) { wait_vmem<3 * CPW>(); return; }
    if constexpr (NST > 3) if (n >= 2) { wait_vmem<2 * CPW>(); return; }
    if constexpr (NST > 2) if (n >= 1) { wait_vmem<CPW>(); return; }
    wait_vmem<0>();
  };

  const int nk = AT ? (j.kcount + BK - 1) / BK : Kd / BK;
  // One k step from stage S: start the copy NST - 1 steps ahead into the
  // stage read in the previous step, multiply, then wait for the next
  // step's copy (the copies of the steps after it may stay in flight) and
  // synchronise.
  auto step = [&](auto S, int k) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    constexpr int p = StageRing<s, NST>::prev;
    compute(stage_a(S), stage_b(S), k + NST - 1 < nk, k + NST - 1,
            stage_a(std::integral_constant<int, p>{}), stage_b(std::integral_constant<int, p>{}));
    wait_stages(max(min(k + NST - 1, nk - 1) - (k + 1), 0));
    barrier_no_fence();
  };

  // DB step k (A stage k % 2, B stage k % 3): copy A of step k + 1 into
  // the A stage read in step k - 1, then B of step k + 2 into the B stage
  // read in step k - 1; at the end wait for step k + 1's copies (the B
  // copies of step k + 2, issued last, may stay in flight). Near the end
  // the copies repeat the last step into those free stages, which are not
  // read again, so that they need no branch.
  auto step_db = [&](auto S6, int k) __attribute__((always_inline)) {
    constexpr int s6 = decltype(S6)::value;
    constexpr int sa = s6 % 2, sb = s6 % 3, na = (s6 + 1) % 2, nb = (s6 + 2) % 3;
    compute(stage_a(std::integral_constant<int, sa>{}), stage_b(std::integral_constant<int, sb>{}),
            true, min(k + 1, nk - 1), stage_a(std::integral_constant<int, na>{}),
            stage_b(std::integral_constant<int, sb>{}), min(k + 2, nk - 1),
            stage_b(std::integral_constant<int, nb>{}));
    wait_vmem<B_CP>();
    barrier_no_fence();
  };

  int kc = 0;
  if constexpr (DB) {
    // prologue: A and B of step 0, then B of step 1; wait for step 0
    issue_range(0, sA0, sB0, std::integral_constant<int, 0>{}, std::integral_constant<int, CPW>{},
                0);
    issue_range(0, sA0, sB1, std::integral_constant<int, 0>{}, std::integral_constant<int, CPW>{},
                min(1, nk - 1), false, true);
    wait_vmem<B_CP>();
    barrier_no_fence();
    for (; kc + 6 <= nk; kc += 6)
      static_for<6>([&](auto S) __attribute__((always_inline)) { step_db(S, kc + decltype(S)::value); });
    static_for<5>([&](auto S) __attribute__((always_inline)) {
      if (kc + decltype(S)::value < nk) step_db(S, kc + decltype(S)::value);
    });
    // the last B copies are still in flight: drain them before the
    // epilogue reuses the ring
    wait_vmem<0>();
    barrier_no_fence();
  } else {
    // prologue: stages 0 .. NST - 2 (those that exist), then stage 0 landed
    static_for<NST - 1>([&](auto S) __attribute__((always_inline)) {
      constexpr int v = decltype(S)::value;
      if (v < nk) issue(v, stage_a(S), stage_b(S));
    });
    wait_stages(min(NST - 2, nk - 1));
    barrier_no_fence();
    for (; kc + NST <= nk; kc += NST)
      static_for<NST>([&](auto S) __attribute__((always_inline)) { step(S, kc + decltype(S)::value); });
    static_for<NST - 1>([&](auto S) __attribute__((always_inline)) {
      if (kc + decltype(S)::value < nk) step(S, kc + decltype(S)::value);
    });
  }

  if constexpr (MODE == 0 && kGemmStagedStore) {
    // h = SiLU(g) u (the layer dtype), and with ug also u and g (fp32),
    // written through the idle LDS ring (see mode 2): first the BM x BN/2 h
    // tile, then u and g in chunks of UGR rows; each wave writes whole row
    // segments.
    const int Ih = N / 2;
    constexpr int HC = BN / 2;         // columns of the h tile
    constexpr int HLD = HC + 8;        // staged h row stride (bf16, 16 B pad)
    constexpr int ULD = HC + 4;        // staged u / g row stride (fp32, 16 B pad)
    constexpr int RING = (NST * (BM + BN) + (DB ? BN : 0)) * BK * 2;
    constexpr int UGR = 2 * 64 * ULD * 4 <= RING ? 64 : 32;
    static_assert(BM * HLD * 2 <= RING && 2 * UGR * ULD * 4 <= RING && NI == 2 * (NI / 2),
                  "staged h / ug tiles fit in the LDS ring");
    uint16_t *C = static_cast<uint16_t *>(Cv);
    float *ug = cl.ug;
    uint16_t *sh = reinterpret_cast<uint16_t *>(sA0);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int p = 0; p < NI / 2; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
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
          const int row = wm * (BM / 2) + mi * 32 + r;
          const int c = wn * (HC / WN) + p * 32 + 8 * q + 4 * g;
          *reinterpret_cast<u32x2_t *>(sh + row * HLD + c) = o;
        }
    epi_barrier();
    // two rows per wave instruction: lanes 0-31 one row, 32-63 the next;
    // lane l takes columns 4 (l % 32) .. + 3
    const int hcol = j.nt * HC + 4 * (lane & 31);
    const bool hok = hcol < Ih;
#pragma unroll 4
    for (int rl = 2 * wave + (lane >> 5); rl < j.rows; rl += 2 * NW) {
      if (hok)
        *reinterpret_cast<u32x2_t *>(C + (static_cast<int64_t>(j.row0) + rl) * ldc + hcol) =
            *reinterpret_cast<const u32x2_t *>(sh + rl * HLD + 4 * (lane & 31));
    }
    const float *dhp = cl.dh_in;
    if (ug || dhp) {
      float *su = reinterpret_cast<float *>(sA0);
      float *sgt = su + UGR * ULD;
      // with dh_in: this lane's rows of a chunk (2 per wave step) and their dh,
      // loaded before the chunk is staged so that the loads overlap it
      constexpr int DPR = (UGR + 2 * NW - 1) / (2 * NW);
      f32x4_t dhv[DPR];
#pragma unroll 1
      for (int ch = 0; ch < BM / UGR && ch * UGR < j.rows; ++ch) {
        if (dhp) {
          const int nr = min(UGR, j.rows - ch * UGR);
#pragma unroll
          for (int i = 0; i < DPR; ++i) {
            const int rl = 2 * wave + (lane >> 5) + 2 * NW * i;
            dhv[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (hok && rl < nr)
              dhv[i] = *reinterpret_cast<const f32x4_t *>(
                  dhp + (static_cast<int64_t>(j.row0) + ch * UGR + rl) * Ih + hcol);
          }
        }
        epi_barrier();
        static_for<MI>([&](auto Mv) __attribute__((always_inline)) {
          constexpr int mi = decltype(Mv)::value;
          const int rb = wm * (BM / 2) + mi * 32;
          if (rb / UGR != ch) return;
#pragma unroll
          for (int p = 0; p < NI / 2; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int o = (rb - ch * UGR + r) * ULD + wn * (HC / WN) + p * 32 + 8 * q + 4 * g;
              *reinterpret_cast<f32x4_t *>(su + o) =
                  f32x4_t{acc[mi][p][4 * q], acc[mi][p][4 * q + 1], acc[mi][p][4 * q + 2],
                          acc[mi][p][4 * q + 3]};
              *reinterpret_cast<f32x4_t *>(sgt + o) =
                  f32x4_t{acc[mi][p + NI / 2][4 * q], acc[mi][p + NI / 2][4 * q + 1],
                          acc[mi][p + NI / 2][4 * q + 2], acc[mi][p + NI / 2][4 * q + 3]};
            }
        });
        epi_barrier();
        const int nr = min(UGR, j.rows - ch * UGR);
        if (dhp) {
          // the SwiGLU backward (as mode 2's epilogue computes it from stored
          // u, g, h; the same operations in the same order): h as stored
          // above, du = dh SiLU(g), dg = dh u SiLU'(g), and the sum of dh h
          // over the tile's 128 columns of each row (lanes 0-31 one row,
          // 32-63 the next)
          uint16_t *D = static_cast<uint16_t *>(cl.dd_out);
#pragma unroll
          for (int i = 0; i < DPR; ++i) {
            const int rl = 2 * wave + (lane >> 5) + 2 * NW * i;
            if (rl >= nr) break;  // uniform in each half-wave (one row)
            const int64_t grow = static_cast<int64_t>(j.row0) + ch * UGR + rl;
            const f32x4_t u4 = *reinterpret_cast<const f32x4_t *>(su + rl * ULD + 4 * (lane & 31));
            const f32x4_t g4 = *reinterpret_cast<const f32x4_t *>(sgt + rl * ULD + 4 * (lane & 31));
            const f32x4_t dh4 = dhv[i];
            float du[4], dg[4], asum = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float u = u4[e], gt = g4[e], dh = dh4[e];
              const float hv = gt * u * __builtin_amdgcn_rcpf(1.0f + __expf(-gt));
              const float hq = __uint_as_float(static_cast<uint32_t>(f32_to_bf16(hv)) << 16);
              const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gt));
              du[e] = dh * (gt * sg);
              dg[e] = dh * u * (sg * (1.0f + gt * (1.0f - sg)));
              asum += dh * hq;
            }
            if (hok) {
              u32x2_t o;
              o[0] = pack_bf16x2(du[0], du[1]);
              o[1] = pack_bf16x2(du[2], du[3]);
              *reinterpret_cast<u32x2_t *>(D + grow * N + hcol) = o;
              o[0] = pack_bf16x2(dg[0], dg[1]);
              o[1] = pack_bf16x2(dg[2], dg[3]);
              *reinterpret_cast<u32x2_t *>(D + grow * N + Ih + hcol) = o;
            } else {
              asum = 0.0f;
            }
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) asum += __shfl_xor(asum, o, kWave);
            if (cl.apart && (lane & 31) == 0) cl.apart[grow * cl.apart_ld + j.nt] = asum;
          }
          continue;
        }
#pragma unroll 2
        for (int rl = 2 * wave + (lane >> 5); rl < nr; rl += 2 * NW) {
          if (!hok) continue;
          float *ur = ug + (static_cast<int64_t>(j.row0) + ch * UGR + rl) * N;
          *reinterpret_cast<f32x4_t *>(ur + hcol) =
              *reinterpret_cast<const f32x4_t *>(su + rl * ULD + 4 * (lane & 31));
          *reinterpret_cast<f32x4_t *>(ur + Ih + hcol) =
              *reinterpret_cast<const f32x4_t *>(sgt + rl * ULD + 4 * (lane & 31));
        }
      }
    }
  } else if constexpr (MODE == 0) {
    const int Ih = N / 2;
    uint16_t *C = static_cast<uint16_t *>(Cv);
    float *ug = cl.ug;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * (BM / 2) + mi * 32 + r;
      if (row >= j.rows) continue;
      const int64_t grow = static_cast<int64_t>(j.row0) + row;
      uint16_t *crow = C + grow * ldc;
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
          if (ug) {
            float *ur = ug + grow * N;
            *reinterpret_cast<f32x4_t *>(ur + col) =
                f32x4_t{acc[mi][p][4 * q], acc[mi][p][4 * q + 1], acc[mi][p][4 * q + 2],
                        acc[mi][p][4 * q + 3]};
            *reinterpret_cast<f32x4_t *>(ur + Ih + col) =
                f32x4_t{acc[mi][p + NI / 2][4 * q], acc[mi][p + NI / 2][4 * q + 1],
                        acc[mi][p + NI / 2][4 * q + 2], acc[mi][p + NI / 2][4 * q + 3]};
          }
        }
    }
  } else if constexpr (MODE == 2) {
    // dh = rowscale * acc of (row, column) (the routing weight of the row:
    // acc = W2^T dout); u and g as the forward computed them, h as it stored
    // them. du = dh SiLU(g), dg = dh u SiLU'(g) with
    // SiLU'(g) = s (1 + g (1 - s)), s = 1 / (1 + exp(-g)); [du; dg] is
    // stored in the layer dtype (row stride 2N, du first); the sum of dh h
    // over each 128 columns of each row goes to apart[row, 128-column block].
    // Without u and g (ug null: the recompute that follows runs the SwiGLU
    // backward in its own epilogue) this epilogue stores dh itself (fp32, C).
    // The accumulators hold one row per lane, which would make every global
    // access of this epilogue touch 64 rows; so the tile of acc is staged in
    // the (now idle) LDS ring and each wave then walks whole rows: lane l
    // takes columns 4 l .. 4 l + 3, and the u, g, h reads and the du, dg
    // writes are contiguous row segments.
    constexpr int SLD = BN + 4;  // staged row stride in floats (16 B pad: bank spread)
    constexpr int RING = (NST * (BM + BN) + (DB ? BN : 0)) * BK * 2;
    // rows staged at a time: the whole tile when it fits the ring
    constexpr int CH = BM * SLD * 4 <= RING ? BM : (BM / 2) * SLD * 4 <= RING ? BM / 2 : BM / 4;
    static_assert(CH * SLD * 4 <= RING && CH % 32 == 0 && BM % CH == 0,
                  "the dh chunk fits in the LDS ring");
    float *stg = reinterpret_cast<float *>(sA0);
    uint16_t *D = static_cast<uint16_t *>(Cv);
    const float *ugp = cl.ug;
    const uint16_t *hp = static_cast<const uint16_t *>(cl.hsave);
    const int col = j.nt * BN + 4 * lane;
    const bool cok = col < N;
    constexpr int UR = kDgradEpilogueRows;  // rows per wave in flight
    // every wave's last LDS reads have completed (the MFMAs consumed them)
    // and the last step ended with a workgroup barrier: the ring is free
#pragma unroll 1
    for (int ch = 0; ch < BM / CH && ch * CH < j.rows; ++ch) {
      if (ch > 0) epi_barrier();
      static_for<MI>([&](auto Mv) __attribute__((always_inline)) {
        constexpr int mi = decltype(Mv)::value;
        const int rb = wm * (BM / 2) + mi * 32;
        if (rb / CH != ch) return;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = wn * (BN / WN) + ni * 32 + 8 * q + 4 * g;
            *reinterpret_cast<f32x4_t *>(stg + (rb - ch * CH + r) * SLD + c) =
                f32x4_t{acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                        acc[mi][ni][4 * q + 3]};
          }
      });
      epi_barrier();
      const int nr = min(CH, j.rows - ch * CH);
      if (!ugp) {
        // dh alone (the recompute's epilogue runs the SwiGLU backward), fp32
        float *Cf = static_cast<float *>(Cv);
#pragma unroll 2
        for (int rl = wave; rl < nr; rl += NW) {
          const int64_t grow = static_cast<int64_t>(j.row0) + ch * CH + rl;
          const float rs = cl.rowscale ? cl.rowscale[grow] : 1.0f;
          const f32x4_t a4 = *reinterpret_cast<const f32x4_t *>(stg + rl * SLD + 4 * lane);
          if (cok)
            *reinterpret_cast<f32x4_t *>(Cf + grow * ldc + col) =
                f32x4_t{rs * a4[0], rs * a4[1], rs * a4[2], rs * a4[3]};
        }
        continue;
      }
#pragma unroll 1
      for (int r0 = wave; r0 < nr; r0 += NW * UR) {
        f32x4_t u4[UR], g4[UR];
        u32x2_t h2[UR];
        float rs[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
          const int row = r0 + NW * u;
          const int64_t grow = static_cast<int64_t>(j.row0) + ch * CH + row;
          u4[u] = g4[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          h2[u] = u32x2_t{0u, 0u};
          rs[u] = 1.0f;
          if (row < nr) {
            if (cl.rowscale) rs[u] = cl.rowscale[grow];
            if (cok) {
              u4[u] = *reinterpret_cast<const f32x4_t *>(ugp + grow * 2 * N + col);
              g4[u] = *reinterpret_cast<const f32x4_t *>(ugp + grow * 2 * N + N + col);
              h2[u] = *reinterpret_cast<const u32x2_t *>(hp + grow * N + col);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
          const int row = r0 + NW * u;
          if (row >= nr) break;  // wave-uniform
          const int64_t grow = static_cast<int64_t>(j.row0) + ch * CH + row;
          const f32x4_t acc4 = *reinterpret_cast<const f32x4_t *>(stg + row * SLD + 4 * lane);
          float du[4], dg[4], asum = 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float dh = rs[u] * acc4[e];
            const float gt = g4[u][e];
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gt));
            du[e] = dh * (gt * sg);
            dg[e] = dh * u4[u][e] * (sg * (1.0f + gt * (1.0f - sg)));
            const uint32_t hw = h2[u][e >> 1];
            asum += dh * __uint_as_float((e & 1) ? (hw & 0xffff0000u) : (hw << 16));
          }
          if (cok) {
            u32x2_t o;
            o[0] = pack_bf16x2(du[0], du[1]);
            o[1] = pack_bf16x2(du[2], du[3]);
            *reinterpret_cast<u32x2_t *>(D + grow * ldc + col) = o;
            o[0] = pack_bf16x2(dg[0], dg[1]);
            o[1] = pack_bf16x2(dg[2], dg[3]);
            *reinterpret_cast<u32x2_t *>(D + grow * ldc + N + col) = o;
          } else {
            asum = 0.0f;
          }
          // one partial per 128 columns: lanes 0-31 and 32-63 cover the two
          // halves of the tile's 256 columns
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) asum += __shfl_xor(asum, o, kWave);
          const int pi = 2 * j.nt + (lane >> 5);
          if (cl.apart && (lane & 31) == 0 && pi < cl.apart_ld)
            cl.apart[grow * cl.apart_ld + pi] = asum;
        }
      }
    }
  } else if constexpr (kGemmStagedStore) {
    // modes 1, 3 (fp32 rows) and 4 (weight gradient, layer dtype): the tile
    // goes through the idle LDS ring (as in mode 2) in chunks of CH rows that
    // fit there; each wave then writes whole row segments (lane l: columns
    // 4 l .. 4 l + 3), instead of one row per lane.
    using OT = std::conditional_t<MODE == 4, uint16_t, float>;
    constexpr int OB = sizeof(OT);
    constexpr int LD = BN + 16 / OB;  // staged row stride in elements (16 B pad)
    // (the dx GEMM keeps 64-row chunks: with 128-row chunks its body spills
    // 320 B/lane instead of 76)
    constexpr int RING = (NST * (BM + BN) + (DB && MODE != 3 ? BN : 0)) * BK * 2;
    constexpr int CH = BM * LD * OB <= RING ? BM : (BM / 2) * LD * OB <= RING ? BM / 2 : BM / 4;
    static_assert(CH * LD * OB <= RING && CH % 32 == 0 && BM % CH == 0, "staged chunk fits");
    OT *stg = reinterpret_cast<OT *>(sA0);
    OT *C = static_cast<OT *>(Cv);
    if constexpr (MODE == 4) C += static_cast<int64_t>(j.g < a.E ? j.g : 0) * cl.strideC;
    const int col = j.nt * BN + 4 * lane;
    const bool cok = col < N;
#pragma unroll 1
    for (int ch = 0; ch < BM / CH && ch * CH < j.rows; ++ch) {
      static_for<MI>([&](auto Mv) __attribute__((always_inline)) {
        constexpr int mi = decltype(Mv)::value;
        const int rb = wm * (BM / 2) + mi * 32;
        if (rb / CH != ch) return;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            OT *p = stg + (rb - ch * CH + r) * LD + wn * (BN / WN) + ni * 32 + 8 * q + 4 * g;
            if constexpr (MODE == 4) {
              u32x2_t o;
              o[0] = pack_bf16x2(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1]);
              o[1] = pack_bf16x2(acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]);
              *reinterpret_cast<u32x2_t *>(p) = o;
            } else {
              *reinterpret_cast<f32x4_t *>(p) =
                  f32x4_t{acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                          acc[mi][ni][4 * q + 3]};
            }
          }
      });
      epi_barrier();
      const int nr = min(CH, j.rows - ch * CH);
#pragma unroll 4
      for (int rl = wave; rl < nr; rl += NW) {
        OT *dst = C + (static_cast<int64_t>(j.row0) + ch * CH + rl) * ldc + col;
        const OT *src = stg + rl * LD + 4 * lane;
        if (cok) {
          if constexpr (MODE == 4)
            *reinterpret_cast<u32x2_t *>(dst) = *reinterpret_cast<const u32x2_t *>(src);
          else
            *reinterpret_cast<f32x4_t *>(dst) = *reinterpret_cast<const f32x4_t *>(src);
        }
      }
      epi_barrier();
    }
  } else if constexpr (MODE == 4) {
    uint16_t *C = static_cast<uint16_t *>(Cv) + static_cast<int64_t>(j.g < a.E ? j.g : 0) * cl.strideC;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * (BM / 2) + mi * 32 + r;
      if (row >= j.rows) continue;
      uint16_t *crow = C + (static_cast<int64_t>(j.row0) + row) * ldc;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = j.nt * BN + wn * (BN / WN) + ni * 32 + 8 * q + 4 * g;
          if (col >= N) continue;
          u32x2_t o;
          o[0] = pack_bf16x2(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1]);
          o[1] = pack_bf16x2(acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]);
          *reinterpret_cast<u32x2_t *>(crow + col) = o;
        }
    }
  } else {
    // modes 1 and 3: fp32 rows
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

// Block: one (row tile, column tile) job. Row tiles hold up to BM rows; a
// group's last tile is often much shorter: one with at most BM / 4, BM / 2
// or 3 BM / 4 rows runs the quarter-, half- or three-quarter-height body
// (that share of the MFMAs and A copies, the same B copies; each where the
// height is a multiple of 64). The bodies are straight-line code over the
// same LDS ring. Mode 4 jobs are whole output tiles (one body).
// OCC: blocks per CU the register allocation must allow (the 128-row
// weight-gradient tile runs two per CU).
template <int MODE, int BM, int BK, int NST, int WN, int OCC = 1>
__global__ __launch_bounds__(128 * WN, OCC * 2 * WN / 4) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int BN = kGemmBN;
  constexpr int AE = BM * BK / 8, BE = BN * BK / 8;  // 16-byte chunks per stage
  static_assert(NST * (BM + BN) * BK * 2 <= 160 * 1024, "LDS ring fits in 160 KiB");
  // the 8-wave blocks whose B is a weight (modes 0, 1, 3) take a third B
  // stage where it fits
  constexpr bool DB = kGemmDeepB && WN == 4 && NST == 2 && BK == 64 &&
                      (MODE == 0 || MODE == 1 || MODE == 3 || (MODE == 2 && kDgradDownDeepB)) &&
                      (NST * (BM + BN) + BN) * BK * 2 <= 160 * 1024;
  // one array: stage s holds A at (AE + BE) s and B right after it (with DB
  // the third B stage follows); the whole ring is reused by the epilogues
  // that stage their tile in LDS
  __shared__ u32x4_t smem[NST * (AE + BE) + (DB ? BE : 0)];
  u32x4_t *sA0 = smem, *sB0 = smem + AE;
  u32x4_t *sA1 = smem + (AE + BE), *sB1 = sA1 + AE;
  u32x4_t *sA2 = NST > 2 ? smem + 2 * (AE + BE) : smem;
  u32x4_t *sB2 = NST > 2 ? sA2 + AE : DB ? smem + 2 * (AE + BE) : smem;
  u32x4_t *sA3 = NST > 3 ? smem + 3 * (AE + BE) : smem, *sB3 = NST > 3 ? sA3 + AE : smem;
  u32x4_t *sA4 = NST > 4 ? smem + 4 * (AE + BE) : smem, *sB4 = NST > 4 ? sA4 + AE : smem;

  TileJob j;
  if constexpr (MODE == 4) {
    if (!resolve_wgrad<BM, BN>(a, j)) return;
    gemm_tile<MODE, BM, BK, NST, WN>(a, j, sA0, sB0, sA1, sB1, sA2, sB2, sA3, sB3, sA4, sB4);
  } else {
    if (!resolve_job<MODE, BN>(a, j)) return;
    constexpr int BMS = BM / 2, BM3 = BM / 4 * 3, BMQ = BM / 4;
    // a body exists where its A stage splits into whole 1 KiB copies per wave
    constexpr bool whole = [] (int bm) constexpr { return bm * BK * 2 % (1024 * 2 * WN) == 0; }(BM3);
    constexpr bool whole_s = [] (int bm) constexpr { return bm * BK * 2 % (1024 * 2 * WN) == 0; }(BMS);
    constexpr bool whole_q = [] (int bm) constexpr { return bm * BK * 2 % (1024 * 2 * WN) == 0; }(BMQ);
    if constexpr (kGemmQuarterBody && BMQ >= 64 && BMQ % 64 == 0 && whole_q) {
      if (j.rows <= BMQ) {
        gemm_tile<MODE, BMQ, BK, NST, WN, DB>(a, j, sA0, sB0, sA1, sB1, sA2, sB2, sA3, sB3, sA4, sB4);
        return;
      }
    }
    if constexpr (BMS >= 64 && BMS % 64 == 0 && whole_s) {
      if (j.rows <= BMS) {
        gemm_tile<MODE, BMS, BK, NST, WN, DB>(a, j, sA0, sB0, sA1, sB1, sA2, sB2, sA3, sB3, sA4, sB4);
        return;
      }
    }
    if constexpr (BM3 > BMS && BM3 % 64 == 0 && whole) {
      if (j.rows <= BM3) {
        gemm_tile<MODE, BM3, BK, NST, WN, DB>(a, j, sA0, sB0, sA1, sB1, sA2, sB2, sA3, sB3, sA4, sB4);
        return;
      }
    }
    gemm_tile<MODE, BM, BK, NST, WN, DB>(a, j, sA0, sB0, sA1, sB1, sA2, sB2, sA3, sB3, sA4, sB4);
  }
}

// The shared expert on its own (resolve_dense; the bodies and LDS ring of
// gemm_bf16_kernel, modes 0 and 1). A kernel of its own name, so that
// profiles keep it apart from the grouped launches.
template <int MODE, int BM, int BK, int NST, int WN>
__global__ __launch_bounds__(128 * WN, 2 * WN / 4) void gemm_bf16_dense_kernel(GemmArgs a) {
  static_assert(MODE == 0 || MODE == 1, "dense launches: [up; gate] or down");
  constexpr int BN = kGemmBN;
  constexpr int AE = BM * BK / 8, BE = BN * BK / 8;
  static_assert(NST * (BM + BN) * BK * 2 <= 160 * 1024, "LDS ring fits in 160 KiB");
  constexpr bool DB = kGemmDeepB && WN == 4 && NST == 2 && BK == 64 &&
                      (NST * (BM + BN) + BN) * BK * 2 <= 160 * 1024;
  __shared__ u32x4_t smem[NST * (AE + BE) + (DB ? BE : 0)];
  u32x4_t *sA0 = smem, *sB0 = smem + AE;
  u32x4_t *sA1 = smem + (AE + BE), *sB1 = sA1 + AE;
  u32x4_t *sA2 = NST > 2 ? smem + 2 * (AE + BE) : smem;
  u32x4_t *sB2 = NST > 2 ? sA2 + AE : DB ? smem + 2 * (AE + BE) : smem;
  u32x4_t *sA3 = NST > 3 ? smem + 3 * (AE + BE) : smem, *sB3 = NST > 3 ? sA3 + AE : smem;
  u32x4_t *sA4 = NST > 4 ? smem + 4 * (AE + BE) : smem, *sB4 = NST > 4 ? sA4 + AE : smem;
  TileJob j;
  if (!resolve_dense<MODE, BM, BN>(a, j)) return;
  // only the last row tile is short
  constexpr int BMS = BM / 2, BMQ = BM / 4;
  constexpr bool whole_s = BMS * BK * 2 % (1024 * 2 * WN) == 0;
  constexpr bool whole_q = BMQ * BK * 2 % (1024 * 2 * WN) == 0;
  if constexpr (kGemmQuarterBody && BMQ >= 64 && BMQ % 64 == 0 && whole_q) {
    if (j.rows <= BMQ) {
      gemm_tile<MODE, BMQ, BK, NST, WN, DB>(a, j, sA0, sB0, sA1, sB1, sA2, sB2, sA3, sB3, sA4, sB4);
      return;
    }
  }
  if constexpr (BMS >= 64 && BMS % 64 == 0 && whole_s) {
    if (j.rows <= BMS) {
      gemm_tile<MODE, BMS, BK, NST, WN, DB>(a, j, sA0, sB0, sA1, sB1, sA2, sB2, sA3, sB3, sA4, sB4);
      return;
    }
  }
  gemm_tile<MODE, BM, BK, NST, WN, DB>(a, j, sA0, sB0, sA1, sB1, sA2, sB2, sA3, sB3, sA4, sB4);
}

// --------------------------------------------------------------- fp32

// fp32 layers: LDS-tiled FMA, 64 rows x 64 columns per block ([up; gate]:
// 32 up + the matching 32 gate rows), k step 16; thread (ty, tx) owns rows
// 4ty..4ty+3 and four columns. Operands are staged k-major in LDS whatever
// their layout in memory.
template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int BM = kGemmF32BM, BN = kGemmF32BN, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ float red[BM][17];
  TileJob j;
  if constexpr (MODE == 4) {
    if (!resolve_wgrad<BM, BN>(a, j)) return;
  } else {
    if (!resolve_job<MODE, BN>(a, j)) return;
  }
  const bool shared_cls = j.cls != 0;
  const GemmClass &c = shared_cls ? a.cls[1] : a.cls[0];
  const float *A = static_cast<const float *>(c.A);
  const float *B = static_cast<const float *>(c.B);
  if (MODE != 4) B += static_cast<int64_t>(shared_cls ? 0 : j.g) * c.strideB;
  const int N = c.N;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;

  // k-contiguous operands: thread loads 4 consecutive k of row lrow;
  // k-major operands: 4 consecutive columns (lcol) of k row lkk
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int lkk = tid >> 4, lcol = (tid & 15) * 4;
  const float *aptr = nullptr, *bptr = nullptr;
  if (MODE != 4) {
    const int arr = min(lrow, j.rows - 1);
    const int64_t ari = static_cast<int64_t>(j.row0) + arr;
    aptr = A + (c.arow ? static_cast<int64_t>(c.arow[ari]) : ari) * c.lda + lk;
  }
  if (MODE <= 1) {
    int brow;
    if (MODE == 0) {
      const int Ih = N / 2;
      const int col = min(j.nt * (BN / 2) + (lrow & (BN / 2 - 1)), Ih - 1);
      brow = lrow < BN / 2 ? col : Ih + col;
    } else {
      brow = min(j.nt * BN + lrow, N - 1);
    }
    bptr = B + static_cast<int64_t>(brow) * c.Kd + lk;
  }

  int bcol[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    bcol[q] = MODE == 0 ? (q >> 1) * (BN / 2) + tx * 2 + (q & 1) : tx * 4 + q;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = 0.0f;

  const int klen = MODE == 4 ? j.kcount : c.Kd;
  for (int k0 = 0; k0 < klen; k0 += BK) {
    if (MODE == 4) {
      const int kg = k0 + lkk;
      f32x4_t av = {0.0f, 0.0f, 0.0f, 0.0f}, bv = {0.0f, 0.0f, 0.0f, 0.0f};
      if (kg < j.kcount) {
        const int64_t kr = static_cast<int64_t>(j.kstart) + kg;
        av = *reinterpret_cast<const f32x4_t *>(A + kr * c.lda + j.row0 + lcol);
        bv = *reinterpret_cast<const f32x4_t *>(B + kr * c.ldb + j.nt * BN + lcol);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        As[lkk][lcol + q] = av[q];
        Bs[lkk][lcol + q] = bv[q];
      }
    } else {
      const f32x4_t av = *reinterpret_cast<const f32x4_t *>(aptr + k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) As[lk + q][lrow] = av[q];
      if (MODE <= 1) {
        const f32x4_t bv = *reinterpret_cast<const f32x4_t *>(bptr + k0);
#pragma unroll
        for (int q = 0; q < 4; ++q) Bs[lk + q][lrow] = bv[q];
      } else {
        const f32x4_t bv = *reinterpret_cast<const f32x4_t *>(
            B + static_cast<int64_t>(k0 + lkk) * c.ldb + j.nt * BN + lcol);
#pragma unroll
        for (int q = 0; q < 4; ++q) Bs[lkk][lcol + q] = bv[q];
      }
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

  if (MODE == 2) {
    // as the bf16 mode-2 epilogue, in fp32; the partial sums of dh h are
    // reduced over the block's 64 columns in a fixed order
    float *D = static_cast<float *>(c.C);
    const float *hp = static_cast<const float *>(c.hsave);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = ty * 4 + i;
      float ps = 0.0f;
      if (row < j.rows) {
        const int64_t grow = static_cast<int64_t>(j.row0) + row;
        const float rs = c.rowscale ? c.rowscale[grow] : 1.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = j.nt * BN + tx * 4 + q;
          const float dh = rs * acc[i][q];
          const float u = c.ug[grow * 2 * N + col], gt = c.ug[grow * 2 * N + N + col];
          const float sg = 1.0f / (1.0f + expf(-gt));
          D[grow * c.ldc + col] = dh * (gt * sg);
          D[grow * c.ldc + N + col] = dh * u * (sg * (1.0f + gt * (1.0f - sg)));
          ps += dh * hp[grow * N + col];
        }
      }
      red[row][tx] = ps;
    }
    __syncthreads();
    if (c.apart && tx == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = ty * 4 + i;
        if (row >= j.rows) continue;
        float t = 0.0f;
        for (int x = 0; x < 16; ++x) t += red[row][x];
        c.apart[(static_cast<int64_t>(j.row0) + row) * c.apart_ld + j.nt] = t;
      }
    }
    return;
  }
  float *C = static_cast<float *>(c.C);
  if (MODE == 4) C += static_cast<int64_t>(j.g < a.E ? j.g : 0) * c.strideC;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ty * 4 + i;
    if (row >= j.rows) continue;
    const int64_t grow = static_cast<int64_t>(j.row0) + row;
    float *crow = C + grow * c.ldc;
    if (MODE == 0) {
      const int Ih = N / 2;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = j.nt * (BN / 2) + tx * 2 + q;
        const float u = acc[i][q], gt = acc[i][2 + q];
        if (col < Ih) {
          crow[col] = gt / (1.0f + expf(-gt)) * u;
          if (c.ug) {
            c.ug[grow * N + col] = u;
            c.ug[grow * N + Ih + col] = gt;
          }
        }
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

// mode 0 ([up; gate]) and mode 3 run the default tile; modes 1 and 2 (the
// down projection's shapes) split each listed row tile.
static hipError_t launch_gemm(GemmArgs a, int max_tiles, int tile_rows, int dtype, int mode,
                              hipStream_t s) {
  const int BN = dtype == kBF16 ? kGemmBN : kGemmF32BN;
  const bool stream = dtype == kBF16 && tile_rows == kGemmStreamBM;
  const bool upgate = mode == 0;
  a.NTn = std::max(col_tiles_host(a.cls[0].N, BN, upgate), col_tiles_host(a.cls[1].N, BN, upgate));
  a.split = dtype != kBF16 || stream ? 1 : mode == 1 ? kGemmDownSplit : mode == 2 ? kDgradDownSplit : 1;
  a.sub_rows = a.split > 1 ? kGemmBM / a.split : 1 << 30;
  const int64_t work = static_cast<int64_t>(max_tiles) * a.split * a.NTn;
  const unsigned grid = static_cast<unsigned>((work + 7) / 8 * 8);
  if (grid == 0) return hipSuccess;
  const dim3 block(128 * kGemmWN);
#define HI3_LAUNCH(M, BMv, BKv, NSTv)                                                      \
  hipLaunchKernelGGL((gemm_bf16_kernel<M, BMv, BKv, NSTv, kGemmWN>), dim3(grid), block, 0, s, a)
  if (dtype == kBF16) {
    constexpr int DBM = kGemmBM / kGemmDownSplit;
    switch (mode) {
      case 0:
        if (stream) HI3_LAUNCH(0, kGemmStreamBM, kGemmStreamBK, kGemmStreamStages);
        else HI3_LAUNCH(0, kGemmBM, kGemmBK, kGemmStages);
        break;
      case 1:
        if (stream) HI3_LAUNCH(1, kGemmStreamBM, kGemmStreamBK, kGemmStreamStages);
        else HI3_LAUNCH(1, DBM, kGemmBK, kGemmDownStages);
        break;
      case 2:
        if (stream) HI3_LAUNCH(2, kGemmStreamBM, 64, kGemmStreamStages);
        else
          hipLaunchKernelGGL((gemm_bf16_kernel<2, kGemmBM / kDgradDownSplit, kDgradDownBK,
                                               kDgradDownStages, kGemmWN, kDgradDownOcc>),
                             dim3(grid), block, 0, s, a);
        break;
      default:
        if (stream) HI3_LAUNCH(3, kGemmStreamBM, 64, kGemmStreamStages);
        else HI3_LAUNCH(3, kGemmBM, kDgradUpBK, kDgradUpStages);
        break;
    }
  } else {
    switch (mode) {
      case 0: hipLaunchKernelGGL(gemm_f32_kernel<0>, dim3(grid), dim3(256), 0, s, a); break;
      case 1: hipLaunchKernelGGL(gemm_f32_kernel<1>, dim3(grid), dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL(gemm_f32_kernel<2>, dim3(grid), dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL(gemm_f32_kernel<3>, dim3(grid), dim3(256), 0, s, a); break;
    }
  }
#undef HI3_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemm_dense(const GemmArgs &a0, int rows, int mode, hipStream_t s) {
  if (mode != 0 && mode != 1) return hipErrorInvalidValue;
  GemmArgs a = a0;
  a.cls[0] = a.cls[1];
  a.E = 0;
  a.split = 1;
  a.sub_rows = 1 << 30;
  a.dense_rows = rows;
  a.NTn = col_tiles_host(a.cls[1].N, kGemmBN, mode == 0);
  constexpr int DBM = kGemmBM / kGemmDownSplit;
  const int BMv = mode == 0 ? kGemmBM : DBM;
  const int64_t work = static_cast<int64_t>((rows + BMv - 1) / BMv) * a.NTn;
  const unsigned grid = static_cast<unsigned>((work + 7) / 8 * 8);
  if (grid == 0) return hipSuccess;
  const dim3 block(128 * kGemmWN);
  if (mode == 0)
    hipLaunchKernelGGL((gemm_bf16_dense_kernel<0, kGemmBM, kGemmBK, kGemmStages, kGemmWN>),
                       dim3(grid), block, 0, s, a);
  else
    hipLaunchKernelGGL((gemm_bf16_dense_kernel<1, DBM, kGemmBK, kGemmDownStages, kGemmWN>),
                       dim3(grid), block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_upgate(const GemmArgs &a, int max_tiles, int tile_rows, int dtype,
                              hipStream_t s) {
  return launch_gemm(a, max_tiles, tile_rows, dtype, 0, s);
}

hipError_t launch_gemm_down(const GemmArgs &a, int max_tiles, int tile_rows, int dtype,
                            hipStream_t s) {
  return launch_gemm(a, max_tiles, tile_rows, dtype, 1, s);
}

hipError_t launch_gemm_dgrad_down(const GemmArgs &a, int max_tiles, int tile_rows, int dtype,
                                  hipStream_t s) {
  return launch_gemm(a, max_tiles, tile_rows, dtype, 2, s);
}

hipError_t launch_gemm_dgrad_up_gate(const GemmArgs &a, int max_tiles, int tile_rows,
                                     int dtype, hipStream_t s) {
  return launch_gemm(a, max_tiles, tile_rows, dtype, 3, s);
}

// Mode 4: a class whose C is null is skipped.
hipError_t launch_gemm_wgrad(const GemmArgs &a0, int E, int dtype, hipStream_t s) {
  GemmArgs a = a0;
  const int TM = dtype == kBF16 ? kWgradBM : kGemmF32BM;  // output tile rows
  const int TN = dtype == kBF16 ? kGemmBN : kGemmF32BN;   // output tile columns
  auto tiles_of = [&](const GemmClass &c) {
    return static_cast<int64_t>((c.M + TM - 1) / TM) * ((c.N + TN - 1) / TN);
  };
  a.wg_shared_blocks = a.cls[1].C ? static_cast<int>((tiles_of(a.cls[1]) + 7) / 8 * 8) : 0;
  const int64_t routed = a.cls[0].C ? 8 * tiles_of(a.cls[0]) * ((E + 7) / 8) : 0;
  const int64_t grid = a.wg_shared_blocks + routed;
  if (grid == 0) return hipSuccess;
  if (dtype == kBF16)
    hipLaunchKernelGGL((gemm_bf16_kernel<4, kWgradBM, kWgradBK, kWgradStages, kWgradWN,
                                         kWgradBM == 128 ? 2 : 1>),
                       dim3(static_cast<unsigned>(grid)), dim3(128 * kWgradWN), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<4>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hi3
