// Backward pass of the layer, outside the grouped GEMMs: the gradient of
// L = sum over real rows of dout . out with the routes held fixed (the
// pages' fine-tuning: HunyuanImage-3.0 model-coverage page, "Train"; the
// forward is the model API page's HunyuanImage3Block MoE + shared MLP with
// build_moe_config's renormalised top-k weights).
//
// With w_k the renormalised weight of the token's k-th expert and
// y_k = W2 h_k its output, the weights are a softmax over the selected
// logits alone, so the logit gradient is zero for the other experts and
//   dl_k = a_k - w_k sum_j a_j,   a_k = w_k (dout . y_k) = dh_k . h_k
// where dh_k = W2^T (w_k dout) is what the mode-2 GEMM computes (it leaves
// the sum a_k in per-column-block partials). Then
//   dx = sum_k W13_k^T [du_k; dg_k] + W13s^T [du_s; dg_s] + sum_k dl_k Wr[e_k]
//   dWr[e] = sum over e's rows of dl x.
// Every sum runs in a fixed order (no atomics): results are deterministic.
#include <algorithm>

#include "common.h"

namespace hi3 {

// One wave per real token: reads x and dout once, writes x and w_k dout
// (rounded to the layer dtype) to each of the token's K slots, w_k by slot,
// and, when the caller asked for them, x and dout by real-row index.
template <int DT>
__global__ __launch_bounds__(256) void bwd_gather_kernel(BwdGatherArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + wave_uniform(threadIdx.x >> 6);
  if (t >= a.T || (a.pad && a.pad[t])) return;
  constexpr int es = DT == kBF16 ? 2 : 4;
  const int64_t row_bytes = static_cast<int64_t>(a.H) * es;
  const int nchunk = static_cast<int>(row_bytes / 16);
  const u32x4_t *xr = reinterpret_cast<const u32x4_t *>(static_cast<const char *>(a.x) + t * row_bytes);
  const u32x4_t *dr =
      reinterpret_cast<const u32x4_t *>(static_cast<const char *>(a.dout) + t * row_bytes);
  const int vi = a.xv ? a.vidx[t] : -1;
  auto row = [&](void *base, int64_t r) {
    return reinterpret_cast<u32x4_t *>(static_cast<char *>(base) + r * row_bytes);
  };
  for (int c = lane; c < nchunk; c += 64) {
    const u32x4_t xv = xr[c];
    const u32x4_t dv = dr[c];
    for (int k = 0; k < a.K; ++k) {
      const int s = a.slotof[t * a.K + k];
      if (s < 0) continue;
      const float w = a.wts[t * a.K + k];
      u32x4_t o;
      if (DT == kBF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = pack_bf16x2(w * __uint_as_float(dv[e] << 16),
                             w * __uint_as_float(dv[e] & 0xffff0000u));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(w * __uint_as_float(dv[e]));
      }
      row(a.xs, s)[c] = xv;
      row(a.dys, s)[c] = o;
      if (c == 0) a.wslot[s] = w;
    }
    if (vi >= 0) {
      row(a.xv, vi)[c] = xv;
      row(a.doutv, vi)[c] = dv;
    }
  }
}

hipError_t launch_bwd_gather(const BwdGatherArgs &a, int dtype, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((a.T + 3) / 4));
  if (dtype == kBF16)
    hipLaunchKernelGGL(bwd_gather_kernel<kBF16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_gather_kernel<kF32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// One block per token: a_k from the partials (in column-block order),
// dl_k = a_k - w_k sum_j a_j (stored by slot for the router's weight
// gradient), then dx = sum_k dxs[slot_k] + dxsh + sum_k dl_k Wr[e_k], summed
// in fp32 in that order and rounded once to the layer dtype (or kept in fp32
// when the block's RMSNorm backward follows).
template <int DT>
__global__ __launch_bounds__(256) void bwd_combine_kernel(BwdCombineArgs a) {
  __shared__ float ak[kMaxE], dl[kMaxE];
  __shared__ int sl[kMaxE], ex[kMaxE];
  const int64_t t = blockIdx.x;
  if (a.pad && a.pad[t]) return;
  const int vi = a.vidx[t];
  if (vi < 0) return;
  const int K = a.K;
  if (static_cast<int>(threadIdx.x) < K) {
    const int k = threadIdx.x;
    const int s = a.slotof[t * K + k];
    sl[k] = s;
    ex[k] = a.idx[t * K + k];
    float v = 0.0f;
    if (s >= 0)
      for (int p = 0; p < a.P; ++p) v += a.apart[static_cast<int64_t>(s) * a.P + p];
    ak[k] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float A = 0.0f;
    for (int k = 0; k < K; ++k) A += ak[k];
    for (int k = 0; k < K; ++k) {
      const float d = ak[k] - a.wts[t * K + k] * A;
      dl[k] = sl[k] >= 0 ? d : 0.0f;
      if (sl[k] >= 0) a.dls[sl[k]] = d;
    }
  }
  __syncthreads();
  if (!a.dx && !a.dx_f32) return;
  const int nq = a.H / 4;
  for (int q = threadIdx.x; q < nq; q += blockDim.x) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < K; ++k) {
      const int s = sl[k];
      if (s < 0) continue;
      const f32x4_t v = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4_t *>(a.dxs + static_cast<int64_t>(s) * a.H) + q);
      acc += v;
    }
    acc += __builtin_nontemporal_load(
        reinterpret_cast<const f32x4_t *>(a.dxsh + static_cast<int64_t>(vi) * a.H) + q);
    for (int k = 0; k < K; ++k) {
      if (sl[k] < 0) continue;
      const f32x4_t wr =
          reinterpret_cast<const f32x4_t *>(a.w_router + static_cast<int64_t>(ex[k]) * a.H)[q];
      const float d = dl[k];
      acc[0] = fmaf(d, wr[0], acc[0]);
      acc[1] = fmaf(d, wr[1], acc[1]);
      acc[2] = fmaf(d, wr[2], acc[2]);
      acc[3] = fmaf(d, wr[3], acc[3]);
    }
    if (a.dx_f32) {
      reinterpret_cast<f32x4_t *>(a.dx_f32 + t * a.H)[q] = acc;
    } else if (DT == kBF16) {
      u32x2_t o;
      o[0] = pack_bf16x2(acc[0], acc[1]);
      o[1] = pack_bf16x2(acc[2], acc[3]);
      reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.dx) + t * a.H)[q] = o;
    } else {
      reinterpret_cast<f32x4_t *>(static_cast<float *>(a.dx) + t * a.H)[q] = acc;
    }
  }
}

hipError_t launch_bwd_combine(const BwdCombineArgs &a, int dtype, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(a.T));
  if (dtype == kBF16)
    hipLaunchKernelGGL(bwd_combine_kernel<kBF16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_combine_kernel<kF32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// dWr[e, h] = sum over expert e's slots s (ascending) of dl[s] x_s[h], in
// fp32, in two fixed-order steps so that an expert with many rows does not
// serialise: (1) one block per (row tile of the grouped GEMMs' list, 512
// columns) sums its tile's slots into part[tile]; (2) one block per
// (expert, 512 columns) sums its tiles' parts in list order. Each thread
// owns two adjacent columns; the slot loop is unrolled so several rows are
// in flight.
template <int DT>
__global__ __launch_bounds__(256) void dw_router_part_kernel(
    const float *__restrict__ dls, const void *__restrict__ xs, const int4 *__restrict__ tiles,
    const int32_t *__restrict__ gto, int E, int H, float *__restrict__ part) {
  const int tj = blockIdx.x;
  if (tj >= gto[E]) return;  // only the routed experts' tiles
  const int h = (blockIdx.y * 256 + threadIdx.x) * 2;
  if (h >= H) return;
  const int4 tile = tiles[tj];
  const int s0 = tile.y, s1 = tile.y + tile.z;
  float a0 = 0.0f, a1 = 0.0f;
  auto load = [&](int r, float &v0, float &v1) {
    if (DT == kBF16) {
      const uint32_t w = *reinterpret_cast<const uint32_t *>(
          static_cast<const uint16_t *>(xs) + static_cast<int64_t>(r) * H + h);
      v0 = __uint_as_float(w << 16);
      v1 = __uint_as_float(w & 0xffff0000u);
    } else {
      const float *p = static_cast<const float *>(xs) + static_cast<int64_t>(r) * H + h;
      v0 = p[0];
      v1 = p[1];
    }
  };
  int s = s0;
  for (; s + 8 <= s1; s += 8) {
    float v0[8], v1[8], d[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      load(s + u, v0[u], v1[u]);
      d[u] = dls[s + u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a0 = fmaf(d[u], v0[u], a0);
      a1 = fmaf(d[u], v1[u], a1);
    }
  }
  for (; s < s1; ++s) {
    float v0, v1;
    load(s, v0, v1);
    a0 = fmaf(dls[s], v0, a0);
    a1 = fmaf(dls[s], v1, a1);
  }
  *reinterpret_cast<float2 *>(part + static_cast<int64_t>(tj) * H + h) = make_float2(a0, a1);
}

__global__ __launch_bounds__(256) void dw_router_sum_kernel(const float *__restrict__ part,
                                                            const int32_t *__restrict__ gto,
                                                            int H, float *__restrict__ dwr) {
  const int e = blockIdx.x;
  const int h = (blockIdx.y * 256 + threadIdx.x) * 2;
  if (h >= H) return;
  float a0 = 0.0f, a1 = 0.0f;
  for (int tj = gto[e]; tj < gto[e + 1]; ++tj) {
    const float2 v = *reinterpret_cast<const float2 *>(part + static_cast<int64_t>(tj) * H + h);
    a0 += v.x;
    a1 += v.y;
  }
  *reinterpret_cast<float2 *>(dwr + static_cast<int64_t>(e) * H + h) = make_float2(a0, a1);
}

hipError_t launch_dw_router(const float *dls, const void *xs, const int4 *tiles,
                            const int32_t *gto, int max_tiles, int E, int H, int dtype,
                            float *part, float *dwr, hipStream_t s) {
  const unsigned cb = static_cast<unsigned>((H / 2 + 255) / 256);
  const dim3 g1(static_cast<unsigned>(max_tiles), cb), g2(static_cast<unsigned>(E), cb);
  if (dtype == kBF16)
    hipLaunchKernelGGL(dw_router_part_kernel<kBF16>, g1, dim3(256), 0, s, dls, xs, tiles, gto, E,
                       H, part);
  else
    hipLaunchKernelGGL(dw_router_part_kernel<kF32>, g1, dim3(256), 0, s, dls, xs, tiles, gto, E,
                       H, part);
  hipLaunchKernelGGL(dw_router_sum_kernel, g2, dim3(256), 0, s, part, gto, H, dwr);
  return hipGetLastError();
}

// Fills bytes (a multiple of 16) with zeros; a kernel, so that it can be
// captured in a graph.
__global__ __launch_bounds__(256) void zero_kernel(u32x4_t *p, int64_t n) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = z;
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 16);
  if (n == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 4096));
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, static_cast<u32x4_t *>(p), n);
  return hipGetLastError();
}

}  // namespace hi3
