// Dispatch: groups the routed (token, k) pairs by expert (the pages'
// "grouped experts": model-coverage page, "Model Class") with a stable
// counting sort, without atomics and without any device-to-host copy.
//
//   1. per-block expert histograms (router kernel, or histogram_kernel);
//   2. scan_kernel: column-wise exclusive scan of the histograms over blocks,
//      plus the exclusive scan over experts, gives the first slot of every
//      (block, expert); the same kernel writes the expert offsets, the list
//      of real rows and the row-tile list of the grouped GEMMs;
//   3. scatter_kernel: inside a block, the rank of token t among the block's
//      tokens routed to expert e (tokens ascending) completes the slot;
//   4. gather_kernel: copies each real token row to its K slots.
//
// Slot order is expert-major, then ascending token, then k: the order of a
// stable sort of the flattened pairs by expert id.
#include "common.h"

namespace hi3 {

// Exclusive scan across a 1024-thread block; returns this thread's prefix and
// the block total through *total.
__device__ int block_exclusive_scan_1024(int v, int *total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += n;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += wsum[w];
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// One block of 1024 threads. The per-block expert histograms [NB][E] are
// staged in LDS, kScanRows token blocks at a time, with coalesced loads;
// thread (seg, e) = (tid / 64, tid % 64) then walks expert e's column over
// rows [16 seg, 16 seg + 16) of the staged rows. Pass 1 sums each column
// (the experts' totals, hence their offsets); pass 2 writes the first slot
// of every (block, expert). With NB <= kScanRows the rows stay in LDS for
// both passes.
constexpr int kScanRows = 256;

__global__ __launch_bounds__(1024) void scan_kernel(ScanArgs a) {
  __shared__ int hist[kScanRows][kMaxE];
  __shared__ int seg_sum[16][kMaxE];
  __shared__ int tot[kMaxE];
  __shared__ int eoff[kMaxE + 1];
  __shared__ int toff[kMaxE + 2];
  __shared__ int chunk_base[kMaxE];
  __shared__ int nvalid_s;
  const int tid = threadIdx.x;
  const int e = tid & 63, seg = tid >> 6;
  const int E = a.E;
  const int nch = (a.NB + kScanRows - 1) / kScanRows;
  static_assert(kScanRows == 16 * 16, "16 segments of 16 rows");
  // real rows per block (loaded first, scanned after the histograms)
  const int vper = (a.NB + 1023) / 1024;
  const int v_lo = tid * vper, v_hi = min(a.NB, v_lo + vper);
  int vs = 0;
  for (int b = v_lo; b < v_hi; ++b) vs += a.blkval[b];

  // (eight loads in flight per thread before any store: a chunk is at most
  // 256 x 64 = 16 x 1024 values)
  auto stage = [&](int ch) {
    const int b0 = ch * kScanRows;
    const int n = min(kScanRows, a.NB - b0) * E;
    const int32_t *src = a.blkcnt + static_cast<int64_t>(b0) * E;
    for (int i0 = 0; i0 < n; i0 += 8 * 1024) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 1024 + tid;
        v[u] = i < n ? src[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 1024 + tid;
        if (i < n) hist[i / E][i % E] = v[u];
      }
    }
  };
  // sum of this thread's 16 rows of column e in the staged chunk
  auto seg_total = [&](int ch) {
    const int nb = min(kScanRows, a.NB - ch * kScanRows);
    int s = 0;
    if (e < E)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int b = seg * 16 + j;
        if (b < nb) s += hist[b][e];
      }
    return s;
  };

  // pass 1: column totals
  int colsum = 0;  // (segment 0) expert e's total over the chunks so far
  for (int ch = 0; ch < nch; ++ch) {
    stage(ch);
    __syncthreads();
    seg_sum[seg][e] = seg_total(ch);
    __syncthreads();
    if (seg == 0)
      for (int q = 0; q < 16; ++q) colsum += seg_sum[q][e];
    __syncthreads();
  }
  if (seg == 0) tot[e] = e < E ? colsum : 0;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int x = 0; x < E; ++x) {
      eoff[x] = run;
      run += tot[x];
    }
    eoff[E] = run;
  }
  __syncthreads();
  if (seg == 0) chunk_base[e] = e < E ? eoff[e] : 0;
  // pass 2: first slot of every (block, expert)
  for (int ch = 0; ch < nch; ++ch) {
    if (nch > 1) stage(ch);  // a single chunk is still staged
    __syncthreads();
    const int b0 = ch * kScanRows;
    const int nb = min(kScanRows, a.NB - b0);
    seg_sum[seg][e] = seg_total(ch);
    __syncthreads();
    if (e < E) {
      int base = chunk_base[e];
      for (int q = 0; q < seg; ++q) base += seg_sum[q][e];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int b = seg * 16 + j;
        if (b < nb) {
          a.blkoff[static_cast<int64_t>(b0 + b) * E + e] = base;
          base += hist[b][e];
        }
      }
    }
    __syncthreads();
    if (seg == 0 && e < E)
      for (int q = 0; q < 16; ++q) chunk_base[e] += seg_sum[q][e];
    __syncthreads();
  }

  // real rows: scan of per-block counts over all blocks
  int vtotal = 0;
  int vbase = block_exclusive_scan_1024(vs, &vtotal);
  for (int b = v_lo; b < v_hi; ++b) {
    a.blkvoff[b] = vbase;
    vbase += a.blkval[b];
  }
  if (tid == 0) nvalid_s = vtotal;
  __syncthreads();

  // outputs + grouped-GEMM row tiles (experts 0..E-1, then the shared group)
  if (tid <= a.E) a.eoff[tid] = eoff[tid];
  if (tid < a.E) {
    a.counts[tid] = tot[tid];
    if (a.counts_out) a.counts_out[tid] = tot[tid];
  }
  if (tid == 0) {
    a.misc[0] = nvalid_s;
    int run = 0;
    for (int x = 0; x < a.E; ++x) {
      toff[x] = run;
      run += (tot[x] + a.BM - 1) / a.BM;
    }
    toff[a.E] = run;
    if (!a.no_shared) run += (nvalid_s + a.BM - 1) / a.BM;
    toff[a.E + 1] = run;
  }
  __syncthreads();
  if (tid < a.E + 2) a.gto[tid] = toff[tid];
  if (tid < a.E) {
    const int n = tot[tid];
    for (int j = 0, m0 = 0; m0 < n; ++j, m0 += a.BM)
      a.tiles[toff[tid] + j] = make_int4(tid, eoff[tid] + m0, min(a.BM, n - m0), 0);
  }
  if (!a.no_shared) {
    const int n = nvalid_s;
    const int nt = (n + a.BM - 1) / a.BM;
    for (int j = tid; j < nt; j += blockDim.x)
      a.tiles[toff[a.E] + j] = make_int4(a.E, j * a.BM, min(a.BM, n - j * a.BM), 0);
  }
}

hipError_t launch_scan(const ScanArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

// One block per 32 tokens (the histogram blocking).
__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a) {
  __shared__ int ids[kRouterTB][kMaxE];
  __shared__ uint64_t selmask[kRouterTB];
  __shared__ int rank[kRouterTB][kMaxE];
  __shared__ int first[kMaxE];
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouterTB;
  // this block's first slot per expert, fetched alongside the routes
  if (tid < a.E) first[tid] = a.blkoff[static_cast<int64_t>(blockIdx.x) * a.E + tid];
  for (int i = tid; i < kRouterTB * a.K; i += blockDim.x) {
    const int rr = i / a.K, k = i % a.K;
    const int64_t t = t0 + rr;
    int e = -1;
    if (t < a.T && !(a.pad && a.pad[t])) {
      e = a.idx[t * a.K + k];
      if (e < 0 || e >= a.E) e = -1;
    }
    ids[rr][k] = e;
  }
  __syncthreads();
  if (tid < kRouterTB) {
    uint64_t m = 0;
    for (int k = 0; k < a.K; ++k) {
      const int e = ids[tid][k];
      if (e >= 0) m |= 1ull << e;
    }
    selmask[tid] = m;
  }
  __syncthreads();
  if (tid < a.E) {
    int c = 0;
    for (int rr = 0; rr < kRouterTB; ++rr)
      if ((selmask[rr] >> tid) & 1u) rank[rr][tid] = c++;
  }
  __syncthreads();
  for (int i = tid; i < kRouterTB * a.K; i += blockDim.x) {
    const int rr = i / a.K, k = i % a.K;
    const int64_t t = t0 + rr;
    if (t >= a.T) continue;
    int e = ids[rr][k];
    for (int q = 0; q < k && e >= 0; ++q)
      if (ids[rr][q] == e) e = -1;  // a repeated id in one row is ignored
    int slot = -1;
    if (e >= 0) {
      slot = first[e] + rank[rr][e];
      a.perm[slot] = static_cast<int32_t>(t);
    }
    a.slotof[t * a.K + k] = slot;
  }
  if (a.vtok && tid < 64) {
    const int64_t t = t0 + tid;
    const bool ok = tid < kRouterTB && t < a.T && !(a.pad && a.pad[t]);
    const uint64_t bal = __ballot(ok);
    const int vi = a.blkvoff[blockIdx.x] + __popcll(bal & ((1ull << tid) - 1ull));
    if (ok) a.vtok[vi] = static_cast<int32_t>(t);
    if (tid < kRouterTB && t < a.T) a.vidx[t] = ok ? vi : -1;
  }
}

hipError_t launch_scatter(const ScatterArgs &a, hipStream_t s) {
  const int nb = static_cast<int>((a.T + kRouterTB - 1) / kRouterTB);
  hipLaunchKernelGGL(scatter_kernel, dim3(nb), dim3(256), 0, s, a);
  return hipGetLastError();
}

// One wave per token: reads the row once (16-byte loads) and writes it to
// each of its K slots.
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t *__restrict__ x,
                                                     int64_t row_bytes,
                                                     const int32_t *__restrict__ slotof,
                                                     const uint8_t *__restrict__ pad,
                                                     int64_t T, int K,
                                                     uint8_t *__restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave_uniform(threadIdx.x >> 6);
  if (t >= T || (pad && pad[t])) return;
  const int64_t nchunk = row_bytes / 16;
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + t * row_bytes);
  for (int64_t c = lane; c < nchunk; c += 64) {
    const u32x4_t v = src[c];
    for (int k = 0; k < K; ++k) {
      const int s = slotof[t * K + k];
      if (s >= 0) reinterpret_cast<u32x4_t *>(xs + static_cast<int64_t>(s) * row_bytes)[c] = v;
    }
  }
}

hipError_t launch_gather(const void *x, int64_t row_bytes, const int32_t *slotof,
                         const uint8_t *pad, int64_t T, int K, void *xs, hipStream_t s) {
  const unsigned nb = static_cast<unsigned>((T + 3) / 4);
  hipLaunchKernelGGL(gather_kernel, dim3(nb), dim3(256), 0, s,
                     static_cast<const uint8_t *>(x), row_bytes, slotof, pad, T, K,
                     static_cast<uint8_t *>(xs));
  return hipGetLastError();
}

}  // namespace hi3
