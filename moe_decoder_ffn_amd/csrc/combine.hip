// Combine: out[t] = sum_k w[t,k] y[slot(t,k)] + y_shared[t] for every real
// token (model API page, HunyuanImage3Block: routed experts plus the fused
// shared expert; build_moe_config: renormalised top-k weights), summed in fp32
// in k order, then the shared term, rounded once to the layer dtype. With a
// residual (the block's residual around the layer, HunyuanImage3Block being a
// pre-norm layer) the residual row is added last, before that one rounding;
// out may be the residual itself (each element is read, then written, by the
// same thread).
// Deterministic: each output element is produced by one thread in a fixed
// order; no atomics. Padding rows are neither read nor written.
#include "common.h"

namespace hi3 {

// KT > 0: K is known at compile time (the slots and weights of the token
// stay in registers); KT = 0: any K. The fp32 expert rows are read once, so
// their loads are marked non-temporal.
template <int DT, int KT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int64_t t = blockIdx.x;
  if (a.pad && a.pad[t]) return;
  const int vi = a.vidx[t];
  if (vi < 0) return;
  const int K = KT > 0 ? KT : a.K;
  const int nq = a.H / 4;
  const f32x4_t *ys = reinterpret_cast<const f32x4_t *>(a.ys + static_cast<int64_t>(vi) * a.H);
  int slot[KT > 0 ? KT : 1];
  float wk[KT > 0 ? KT : 1];
  if (KT > 0) {
#pragma unroll
    for (int k = 0; k < (KT > 0 ? KT : 1); ++k) {
      slot[k] = a.slotof[t * K + k];
      wk[k] = a.wts[t * K + k];
    }
  }
  for (int q = threadIdx.x; q < nq; q += blockDim.x) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (KT > 0) {
      f32x4_t v[KT > 0 ? KT : 1];
#pragma unroll
      for (int k = 0; k < (KT > 0 ? KT : 1); ++k)
        v[k] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_t *>(a.y + static_cast<int64_t>(slot[k]) * a.H) + q);
#pragma unroll
      for (int k = 0; k < (KT > 0 ? KT : 1); ++k) {
        acc[0] = fmaf(wk[k], v[k][0], acc[0]);
        acc[1] = fmaf(wk[k], v[k][1], acc[1]);
        acc[2] = fmaf(wk[k], v[k][2], acc[2]);
        acc[3] = fmaf(wk[k], v[k][3], acc[3]);
      }
    } else {
      for (int k = 0; k < K; ++k) {
        const int s = a.slotof[t * K + k];
        const float w = a.wts[t * K + k];
        const f32x4_t v = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_t *>(a.y + static_cast<int64_t>(s) * a.H) + q);
        acc[0] = fmaf(w, v[0], acc[0]);
        acc[1] = fmaf(w, v[1], acc[1]);
        acc[2] = fmaf(w, v[2], acc[2]);
        acc[3] = fmaf(w, v[3], acc[3]);
      }
    }
    const f32x4_t sv = __builtin_nontemporal_load(ys + q);
    acc[0] += sv[0];
    acc[1] += sv[1];
    acc[2] += sv[2];
    acc[3] += sv[3];
    if (a.resid) {
      if (DT == kBF16) {
        const u32x2_t rv =
            reinterpret_cast<const u32x2_t *>(static_cast<const uint16_t *>(a.resid) + t * a.H)[q];
        acc[0] += __uint_as_float(rv[0] << 16);
        acc[1] += __uint_as_float(rv[0] & 0xffff0000u);
        acc[2] += __uint_as_float(rv[1] << 16);
        acc[3] += __uint_as_float(rv[1] & 0xffff0000u);
      } else {
        const f32x4_t rv =
            reinterpret_cast<const f32x4_t *>(static_cast<const float *>(a.resid) + t * a.H)[q];
        acc[0] += rv[0];
        acc[1] += rv[1];
        acc[2] += rv[2];
        acc[3] += rv[3];
      }
    }
    if (DT == kBF16) {
      u32x2_t o;
      o[0] = pack_bf16x2(acc[0], acc[1]);
      o[1] = pack_bf16x2(acc[2], acc[3]);
      reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(a.out) + t * a.H)[q] = o;
    } else {
      reinterpret_cast<f32x4_t *>(static_cast<float *>(a.out) + t * a.H)[q] = acc;
    }
  }
}

hipError_t launch_combine(const CombineArgs &a, int dtype, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(a.T));
  if (dtype == kBF16 && a.K == 8)
    hipLaunchKernelGGL((combine_kernel<kBF16, 8>), grid, dim3(256), 0, s, a);
  else if (dtype == kBF16)
    hipLaunchKernelGGL((combine_kernel<kBF16, 0>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((combine_kernel<kF32, 0>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hi3
