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

// LDS holds 64-wide k slices as 8 chunks of 16 bytes per row; chunk c of
// row r sits at position c ^ (r & 7) so the 8 lanes that read one chunk
// column of 8 consecutive rows hit 8 different bank groups.
__device__ __forceinline__ int lds_pos(int row, int chunk) {
  return row * 8 + (chunk ^ (row & 7));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS copy of 16 bytes per lane; lane i writes
// lds_base + 16 i (lds_base must be the same for the whole wave).
__device__ __forceinline__ void lds_dma16(const void *g, u32x4_t *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t *)(lds_base), 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Block: 256 threads = 4 waves in a 2 x 2 grid; tile 256 rows x 256 weight
// rows (down: 256 output columns; [up; gate]: 128 up rows + the matching 128
// gate rows); k step 64. Operand tiles move from global memory straight into
// LDS (global_load_lds_dwordx4), double-buffered in two separate LDS arrays
// (128 KiB): the copy of k step i+1 is in flight while step i is multiplied.
// Each 1 KiB copy instruction covers 8 rows; lane i fetches the logical chunk
// that the swizzle places at position i.
// Wave (wm, wn) owns rows [128 wm, 128 wm + 128) and four 32-row weight
// sub-tiles; with [up; gate] these are up sub-tiles 2wn, 2wn+1 and the gate
// sub-tiles at the same columns, so each lane holds u and g of the same
// (row, column) for the SwiGLU epilogue.
// v_mfma_f32_32x32x16_bf16 result element v of lane l is row
// 8*(v/4) + 4*(l/32) + v%4, column l%32 of the 32x32 sub-tile.
template <int MODE>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
  static_assert(BM == 256 && BN == 256 && BK == 64, "tile shape");
  __shared__ u32x4_t ldsA0[BM * 8], ldsB0[BN * 8], ldsA1[BM * 8], ldsB1[BN * 8];

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
  const int wm = wave >> 1, wn = wave & 1;

  // copy sources: instruction q (0..7) of this wave covers tile rows
  // 64 wave + 8 q + [0, 8); lane i takes row 64 wave + 8 q + i/8 and the
  // logical chunk (i % 8) ^ (row & 7) = (i % 8) ^ (i / 8).
  const int lchunk = (lane & 7) ^ (lane >> 3);
  int arow_src[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = wave * 64 + q * 8 + (lane >> 3);
    const int rr = min(row, j.rows - 1);  // tail rows reread a real row
    const int ri = j.row0 + rr;
    arow_src[q] = arow ? arow[ri] : ri;
  }
  const uint16_t *Ac = A + lchunk * 8;
  const uint16_t *Bc = B + lchunk * 8;
  auto issue = [&](int kc, u32x4_t *la, u32x4_t *lb) {
    const int ko = kc * BK;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      lds_dma16(Ac + static_cast<int64_t>(arow_src[q]) * lda + ko,
                la + (wave * 64 + q * 8) * 8);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = wave * 64 + q * 8 + (lane >> 3);
      int brow;
      if (MODE == 0) {
        const int Ih = N / 2;
        const int col = min(j.nt * (BN / 2) + (row & (BN / 2 - 1)), Ih - 1);
        brow = row < BN / 2 ? col : Ih + col;
      } else {
        brow = min(j.nt * BN + row, N - 1);
      }
      lds_dma16(Bc + static_cast<int64_t>(brow) * Kd + ko, lb + (wave * 64 + q * 8) * 8);
    }
  };

  int nrow[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    if (MODE == 0)
      nrow[ni] = (ni >> 1) * (BN / 2) + wn * 64 + (ni & 1) * 32;
    else
      nrow[ni] = wn * 128 + ni * 32;
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  auto compute = [&](const u32x4_t *la, const u32x4_t *lb) {
    bf16x8_t af[2][4], bf[2][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      af[0][mi] = __builtin_bit_cast(bf16x8_t, la[lds_pos(wm * 128 + mi * 32 + r, g)]);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      bf[0][ni] = __builtin_bit_cast(bf16x8_t, lb[lds_pos(nrow[ni] + r, g)]);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int cur = s & 1;
      if (s + 1 < BK / 16) {
        const int ch = 2 * (s + 1) + g;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          af[cur ^ 1][mi] =
              __builtin_bit_cast(bf16x8_t, la[lds_pos(wm * 128 + mi * 32 + r, ch)]);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          bf[cur ^ 1][ni] = __builtin_bit_cast(bf16x8_t, lb[lds_pos(nrow[ni] + r, ch)]);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][mi], bf[cur][ni],
                                                                acc[mi][ni], 0, 0, 0);
    }
  };

  // k steps in pairs (buffer 0 then buffer 1), one exit; an odd last step
  // runs after the loop from buffer 0.
  const int nk = Kd / BK;
  issue(0, ldsA0, ldsB0);
  wait_vmem();
  __syncthreads();
  int kc = 0;
  for (; kc + 2 <= nk; kc += 2) {
    // the copies are issued before the multiplies (the scheduler may not
    // sink them below the MFMAs, or they would not overlap)
    issue(kc + 1, ldsA1, ldsB1);
    __builtin_amdgcn_sched_barrier(0);
    compute(ldsA0, ldsB0);
    wait_vmem();
    __syncthreads();
    if (kc + 2 < nk) issue(kc + 2, ldsA0, ldsB0);
    __builtin_amdgcn_sched_barrier(0);
    compute(ldsA1, ldsB1);
    wait_vmem();
    __syncthreads();
  }
  if (kc < nk) compute(ldsA0, ldsB0);

  if (MODE == 0) {
    const int Ih = N / 2;
    uint16_t *C = static_cast<uint16_t *>(Cv);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int col = j.nt * (BN / 2) + wn * 64 + p * 32 + r;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * 128 + mi * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
          if (row < j.rows && col < Ih) {
            const float u = acc[mi][p][v];
            const float gt = acc[mi][p + 2][v];
            const float hval = gt / (1.0f + expf(-gt)) * u;
            C[(static_cast<int64_t>(j.row0) + row) * ldc + col] = f32_to_bf16(hval);
          }
        }
      }
  } else {
    float *C = static_cast<float *>(Cv);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int col = j.nt * BN + wn * 128 + ni * 32 + r;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * 128 + mi * 32 + (v >> 2) * 8 + g * 4 + (v & 3);
          if (row < j.rows && col < N)
            C[(static_cast<int64_t>(j.row0) + row) * ldc + col] = acc[mi][ni][v];
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
      hipLaunchKernelGGL(gemm_bf16_kernel<0>, dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(gemm_bf16_kernel<1>, dim3(grid), dim3(256), 0, s, a);
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
