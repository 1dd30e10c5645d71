// Dispatch: groups the routed (token, k) pairs by expert (the pages'
// "grouped experts": model-coverage page, "Model Class") with a stable
// counting sort, without atomics and without any device-to-host copy.
//
//   1. per-block expert histograms (router kernel, or histogram_kernel);
//   2. dispatch_kernel: every block sums the histograms' columns (the
//      experts' offsets) and the rows before its own (its first slot per
//      expert), then ranks its tokens per expert to place each pair; block
//      0 also writes the expert offsets, counts and the grouped GEMMs'
//      row-tile list;
//   3. gather_kernel (only for hi3_moe_dispatch's optional output): copies
//      each real token row to its K slots.
//
// Slot order is expert-major, then ascending token, then k: the order of a
// stable sort of the flattened pairs by expert id.
#include "common.h"

namespace hi3 {

// Inclusive sum of v over lanes 0 .. lane of the wave (fixed shuffle order).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

// Counting sort of the routed (token, k) pairs, one block per 32 tokens (the
// histogram blocking), no atomics. Every block reads all per-block expert
// histograms [NB][E] and real-row counts [NB] (coalesced, 16 waves with up
// to 16 loads in flight per thread): the column totals give the experts' offsets, the
// rows before its own give its first slot per expert and its first real-row
// index. Block 0 also writes the global results: expert offsets, counts,
// the real-row count and the grouped GEMMs' row-tile list (experts
// 0 .. E-1, then the shared expert as group E unless no_shared). Then the
// block places its own pairs: the rank of token t among the block's tokens
// routed to expert e (tokens ascending) completes the slot. With
// do_scatter = 0 (counts only) the grid is block 0 alone.
constexpr int kDispThreads = 1024;
constexpr int kDispGroups = kDispThreads / 64;  // waves, each summing every 16th histogram row

__global__ __launch_bounds__(kDispThreads) void dispatch_kernel(ScanArgs a, ScatterArgs c,
                                                                int do_scatter) {
  __shared__ int part_all[kDispGroups][kMaxE];
  __shared__ int part_pre[kDispGroups][kMaxE];
  __shared__ int vred[2][kDispGroups];
  __shared__ int eoff[kMaxE + 1];
  __shared__ int first[kMaxE];
  __shared__ int toff[kMaxE + 2];
  __shared__ int nvalid_s, vbase_s;
  __shared__ int ids[kRouterTB][kMaxE];
  __shared__ uint64_t selmask[kRouterTB];
  __shared__ int rank[kRouterTB][kMaxE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, grp = tid >> 6;
  const int E = a.E, NB = a.NB;
  const int me = blockIdx.x;

  // this block's pairs (issued first: independent of the histograms)
  if (do_scatter) {
    const int64_t t0 = static_cast<int64_t>(me) * kRouterTB;
    for (int i = tid; i < kRouterTB * c.K; i += blockDim.x) {
      const int rr = i / c.K, k = i % c.K;
      const int64_t t = t0 + rr;
      int e = -1;
      if (t < c.T && !(c.pad && c.pad[t])) {
        e = c.idx[t * c.K + k];
        if (e < 0 || e >= E) e = -1;
      }
      ids[rr][k] = e;
    }
  }

  // column sums of the histograms: thread (grp, lane) takes rows grp,
  // grp + 16, ... (all loads of up to 16 rows in flight at once); all rows,
  // and the rows before this block
  int s_all = 0, s_pre = 0;
  for (int b0 = grp; b0 < NB; b0 += kDispGroups * 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int b = b0 + kDispGroups * u;
      v[u] = lane < E && b < NB ? a.blkcnt[static_cast<int64_t>(b) * E + lane] : 0;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      s_all += v[u];
      if (b0 + kDispGroups * u < me) s_pre += v[u];
    }
  }
  part_all[grp][lane] = s_all;
  part_pre[grp][lane] = s_pre;
  // real rows per block: all blocks, and the blocks before this one
  int va = 0, vp = 0;
  for (int b0 = tid; b0 < NB; b0 += kDispThreads * 4) {
    int v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = b0 + kDispThreads * u;
      v[u] = b < NB ? a.blkval[b] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      va += v[u];
      if (b0 + kDispThreads * u < me) vp += v[u];
    }
  }
  va = wave_inclusive_sum(va);
  vp = wave_inclusive_sum(vp);
  if (lane == 63) {
    vred[0][grp] = va;
    vred[1][grp] = vp;
  }
  __syncthreads();
  if (grp == 0) {
    // expert totals and offsets (an exclusive scan over the experts)
    int tot = 0, pre = 0;
#pragma unroll
    for (int q = 0; q < kDispGroups; ++q) {
      tot += part_all[q][lane];
      pre += part_pre[q][lane];
    }
    if (lane >= E) tot = 0;
    const int inc = wave_inclusive_sum(tot);
    eoff[lane] = inc - tot;
    if (lane == 63) eoff[64] = inc;
    first[lane] = inc - tot + pre;
    if (lane == 0) {
      int nv = 0, vb = 0;
      for (int q = 0; q < kDispGroups; ++q) {
        nv += vred[0][q];
        vb += vred[1][q];
      }
      nvalid_s = nv;
      vbase_s = vb;
    }
    if (me == 0) {
      // row tiles per expert, then their offsets
      const int nt = lane < E ? (tot + a.BM - 1) / a.BM : 0;
      const int tinc = wave_inclusive_sum(nt);
      toff[lane] = tinc - nt;
      if (lane == 63) toff[64] = tinc;
      if (lane < E) {
        a.counts[lane] = tot;
        if (a.counts_out) a.counts_out[lane] = tot;
      }
    }
  }
  __syncthreads();
  if (me == 0) {
    if (tid == 0) {
      eoff[E] = eoff[64];
      a.misc[0] = nvalid_s;
      int run = toff[64];
      toff[E] = run;
      if (!a.no_shared) run += (nvalid_s + a.BM - 1) / a.BM;
      toff[E + 1] = run;
    }
    __syncthreads();
    if (tid <= E) a.eoff[tid] = eoff[tid];
    if (tid < E + 2) a.gto[tid] = toff[tid];
    if (tid < E) {
      const int n = eoff[tid + 1] - eoff[tid];
      for (int j = 0, m0 = 0; m0 < n; ++j, m0 += a.BM)
        a.tiles[toff[tid] + j] = make_int4(tid, eoff[tid] + m0, min(a.BM, n - m0), 0);
    }
    if (!a.no_shared) {
      const int n = nvalid_s;
      const int nt = (n + a.BM - 1) / a.BM;
      for (int j = tid; j < nt; j += blockDim.x)
        a.tiles[toff[E] + j] = make_int4(E, j * a.BM, min(a.BM, n - j * a.BM), 0);
    }
  }
  if (!do_scatter) return;

  // this block's slots
  const int64_t t0 = static_cast<int64_t>(me) * kRouterTB;
  if (tid < kRouterTB) {
    uint64_t msk = 0;
    for (int k = 0; k < c.K; ++k) {
      const int e = ids[tid][k];
      if (e >= 0) msk |= 1ull << e;
    }
    selmask[tid] = msk;
  }
  __syncthreads();
  if (tid < E) {
    int cnt = 0;
    for (int rr = 0; rr < kRouterTB; ++rr)
      if ((selmask[rr] >> tid) & 1u) rank[rr][tid] = cnt++;
  }
  __syncthreads();
  for (int i = tid; i < kRouterTB * c.K; i += blockDim.x) {
    const int rr = i / c.K, k = i % c.K;
    const int64_t t = t0 + rr;
    if (t >= c.T) continue;
    int e = ids[rr][k];
    for (int q = 0; q < k && e >= 0; ++q)
      if (ids[rr][q] == e) e = -1;  // a repeated id in one row is ignored
    int slot = -1;
    if (e >= 0) {
      slot = first[e] + rank[rr][e];
      c.perm[slot] = static_cast<int32_t>(t);
    }
    c.slotof[t * c.K + k] = slot;
  }
  if (c.vtok && tid < 64) {
    const int64_t t = t0 + tid;
    const bool ok = tid < kRouterTB && t < c.T && !(c.pad && c.pad[t]);
    const uint64_t bal = __ballot(ok);
    const int vi = vbase_s + __popcll(bal & ((1ull << tid) - 1ull));
    if (ok) c.vtok[vi] = static_cast<int32_t>(t);
    if (tid < kRouterTB && t < c.T) c.vidx[t] = ok ? vi : -1;
  }
}

hipError_t launch_dispatch(const ScanArgs &a, const ScatterArgs *c, hipStream_t s) {
  if (c) {
    hipLaunchKernelGGL(dispatch_kernel, dim3(static_cast<unsigned>(a.NB)), dim3(kDispThreads), 0,
                       s, a,
                       *c, 1);
  } else {
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kDispThreads), 0, s, a, ScatterArgs{}, 0);
  }
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
