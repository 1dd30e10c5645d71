// The decoder block's normalisation in front of the layer (layers API page,
// HunyuanRMSNorm: normalize in fp32 over the hidden axis, return weight * x
// in the input dtype, eps 1e-5 by default; model API page,
// HunyuanImage3Block: a pre-norm layer, post_attention_layernorm ahead of the
// routed and shared experts). For every real row t:
//   m  = mean of x[t,h]^2, accumulated in fp64 (the squares are exact) and
//        rounded to fp32 after the division by H
//   d  = m + eps in fp32
//   r  = 1 / sqrt(d), evaluated in fp64 and rounded once to fp32
//   n  = x * r as an fp32 product, converted to the layer dtype
//   xn = weight * n, rounded once to the layer dtype (for bf16 the product
//        of two bf16 values is exact in fp32)
// The bf16 roundings decide the router's inputs, so every step is spelled
// out to the rounding. Padding rows are neither read nor written.
// One wave per row, four rows per block: each lane keeps its 16-byte chunks
// of the row (CPL of them, 8 or 16) in registers, so the row is read once;
// the sum of squares is a wave reduction. Longer rows (CPL = 0) take a
// two-pass loop that reads the row again (from L2).
#include "common.h"

namespace hi3 {

template <int DT, int CPL>
__global__ __launch_bounds__(256) void rmsnorm_kernel(NormArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  if (a.pad && a.pad[t]) return;
  constexpr int PER = DT == kBF16 ? 8 : 4;  // elements per 16-byte chunk
  const int nc = a.H / PER;
  const int64_t row_bytes = static_cast<int64_t>(a.H) * (DT == kBF16 ? 2 : 4);
  const u32x4_t *xr =
      reinterpret_cast<const u32x4_t *>(static_cast<const char *>(a.x) + t * row_bytes);
  const u32x4_t *wr = static_cast<const u32x4_t *>(a.weight);
  u32x4_t *outr = reinterpret_cast<u32x4_t *>(static_cast<char *>(a.xn) + t * row_bytes);

  // m = mean of x^2 (fp64 sum, fixed butterfly order), d = m + eps in fp32,
  // r = 1 / sqrt(d) rounded once to fp32; every lane computes the same r.
  auto finish = [&](double ss) { return rms_finish(ss, a.H, a.eps); };

  if constexpr (CPL > 0) {
    u32x4_t v[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (lane + 64 * i < nc) v[i] = xr[lane + 64 * i];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (lane + 64 * i < nc) ss += chunk_sq<DT>(v[i]);
    const float r = finish(ss);
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (lane + 64 * i < nc) outr[lane + 64 * i] = norm_chunk<DT>(v[i], wr[lane + 64 * i], r);
  } else {
    double ss = 0.0;
    for (int c = lane; c < nc; c += 64) ss += chunk_sq<DT>(xr[c]);
    const float r = finish(ss);
    for (int c = lane; c < nc; c += 64) outr[c] = norm_chunk<DT>(xr[c], wr[c], r);
  }
}

hipError_t launch_rmsnorm(const NormArgs &a, int dtype, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((a.T + 3) / 4)), block(256);
  const int nc = a.H / (dtype == kBF16 ? 8 : 4);
  if (dtype == kBF16) {
    if (nc <= 64 * 8) hipLaunchKernelGGL((rmsnorm_kernel<kBF16, 8>), grid, block, 0, s, a);
    else if (nc <= 64 * 16) hipLaunchKernelGGL((rmsnorm_kernel<kBF16, 16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((rmsnorm_kernel<kBF16, 0>), grid, block, 0, s, a);
  } else {
    if (nc <= 64 * 8) hipLaunchKernelGGL((rmsnorm_kernel<kF32, 8>), grid, block, 0, s, a);
    else if (nc <= 64 * 16) hipLaunchKernelGGL((rmsnorm_kernel<kF32, 16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((rmsnorm_kernel<kF32, 0>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- backward
//
// The block's backward through RMSNorm and the residual (the derivative of
// xn = weight * x * r(x), r = (mean x^2 + eps)^(-1/2), at the forward's fp32
// r, the roundings of n and xn passed straight through):
//   dx = r w g - r^3 x s / H,  s = sum over h of x w g;  dh = dout + dx
//   dweight = sum over real rows of g n,  n = dtype(x r) as the forward has it
// One wave per row: the first pass over the row sums x^2 (fp64, fixed order,
// so r is the forward's bit for bit) and x w g (fp32); the second writes dh,
// rounded once. r is kept per row for the weight gradient, which is summed
// in two fixed-order steps: per chunk of kNormBwdRows rows, then over the
// chunks.
template <int DT>
__global__ __launch_bounds__(256) void rmsnorm_bwd_row_kernel(NormBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  if (a.pad && a.pad[t]) return;
  constexpr int PER = DT == kBF16 ? 8 : 4;
  const int nc = a.H / PER;
  const int64_t row_bytes = static_cast<int64_t>(a.H) * (DT == kBF16 ? 2 : 4);
  const u32x4_t *xr =
      reinterpret_cast<const u32x4_t *>(static_cast<const char *>(a.x) + t * row_bytes);
  const u32x4_t *wr = static_cast<const u32x4_t *>(a.weight);
  const float *gr = a.g + t * a.H;
  double ss = 0.0;
  float sv = 0.0f;
  for (int c = lane; c < nc; c += 64) {
    float f[PER], w[PER];
    unpack16<DT>(xr[c], f);
    unpack16<DT>(wr[c], w);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      ss += static_cast<double>(f[e]) * static_cast<double>(f[e]);
      sv += f[e] * (w[e] * gr[c * PER + e]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ss += __shfl_xor(ss, o, kWave);
    sv += __shfl_xor(sv, o, kWave);
  }
  // as the forward: m rounded to fp32, d = m + eps in fp32, r rounded once
  const float m = static_cast<float>(ss / static_cast<double>(a.H));
  const float d = m + a.eps;
  const float r = static_cast<float>(1.0 / sqrt(static_cast<double>(d)));
  if (lane == 0) a.r[t] = r;
  if (!a.dh) return;
  const float c3 = r * r * r * sv / static_cast<float>(a.H);
  const u32x4_t *dr =
      reinterpret_cast<const u32x4_t *>(static_cast<const char *>(a.dout) + t * row_bytes);
  u32x4_t *hr = reinterpret_cast<u32x4_t *>(static_cast<char *>(a.dh) + t * row_bytes);
  for (int c = lane; c < nc; c += 64) {
    float f[PER], w[PER], dv[PER], o[PER];
    unpack16<DT>(xr[c], f);
    unpack16<DT>(wr[c], w);
    unpack16<DT>(dr[c], dv);
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = dv[e] + (r * (w[e] * gr[c * PER + e]) - c3 * f[e]);
    u32x4_t q;
    if (DT == kBF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = __float_as_uint(o[e]);
    }
    hr[c] = q;
  }
}

// part[chunk, h] = sum over the chunk's real rows (ascending) of g n; each
// thread owns two adjacent columns.
template <int DT>
__global__ __launch_bounds__(256) void rmsnorm_bwd_part_kernel(NormBwdArgs a) {
  const int h = (blockIdx.x * 256 + threadIdx.x) * 2;
  if (h >= a.H) return;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kNormBwdRows;
  const int64_t t1 = min(a.T, t0 + kNormBwdRows);
  float a0 = 0.0f, a1 = 0.0f;
  for (int64_t t = t0; t < t1; ++t) {
    if (a.pad && a.pad[t]) continue;
    const float r = a.r[t];
    float x0, x1;
    if (DT == kBF16) {
      const uint32_t v = *reinterpret_cast<const uint32_t *>(
          static_cast<const uint16_t *>(a.x) + t * a.H + h);
      x0 = __uint_as_float(v << 16);
      x1 = __uint_as_float(v & 0xffff0000u);
    } else {
      const float *p = static_cast<const float *>(a.x) + t * a.H + h;
      x0 = p[0];
      x1 = p[1];
    }
    float n0 = x0 * r, n1 = x1 * r;
    if (DT == kBF16) {
      n0 = bf16_to_f32(f32_to_bf16(n0));
      n1 = bf16_to_f32(f32_to_bf16(n1));
    }
    const float2 g2 = *reinterpret_cast<const float2 *>(a.g + t * a.H + h);
    a0 = fmaf(g2.x, n0, a0);
    a1 = fmaf(g2.y, n1, a1);
  }
  *reinterpret_cast<float2 *>(a.part + static_cast<int64_t>(blockIdx.y) * a.H + h) =
      make_float2(a0, a1);
}

template <int DT>
__global__ __launch_bounds__(256) void rmsnorm_bwd_sum_kernel(NormBwdArgs a, int nchunks) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= a.H) return;
  float acc = 0.0f;
  for (int c = 0; c < nchunks; ++c) acc += a.part[static_cast<int64_t>(c) * a.H + h];
  if (DT == kBF16)
    static_cast<uint16_t *>(a.dweight)[h] = f32_to_bf16(acc);
  else
    static_cast<float *>(a.dweight)[h] = acc;
}

hipError_t launch_rmsnorm_backward(const NormBwdArgs &a, int dtype, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int nchunks = static_cast<int>((a.T + kNormBwdRows - 1) / kNormBwdRows);
  const dim3 g1(static_cast<unsigned>((a.T + 3) / 4));
  const dim3 g2(static_cast<unsigned>((a.H / 2 + 255) / 256), static_cast<unsigned>(nchunks));
  const dim3 g3(static_cast<unsigned>((a.H + 255) / 256));
  if (dtype == kBF16) {
    hipLaunchKernelGGL(rmsnorm_bwd_row_kernel<kBF16>, g1, dim3(256), 0, s, a);
    if (a.dweight) {
      hipLaunchKernelGGL(rmsnorm_bwd_part_kernel<kBF16>, g2, dim3(256), 0, s, a);
      hipLaunchKernelGGL(rmsnorm_bwd_sum_kernel<kBF16>, g3, dim3(256), 0, s, a, nchunks);
    }
  } else {
    hipLaunchKernelGGL(rmsnorm_bwd_row_kernel<kF32>, g1, dim3(256), 0, s, a);
    if (a.dweight) {
      hipLaunchKernelGGL(rmsnorm_bwd_part_kernel<kF32>, g2, dim3(256), 0, s, a);
      hipLaunchKernelGGL(rmsnorm_bwd_sum_kernel<kF32>, g3, dim3(256), 0, s, a, nchunks);
    }
  }
  return hipGetLastError();
}

}  // namespace hi3
