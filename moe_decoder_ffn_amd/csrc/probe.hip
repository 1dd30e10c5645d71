// Measurement probe: the bf16 matrix-core rate this GPU sustains with no
// memory traffic at all, the ceiling the grouped GEMMs are compared with
// next to the published dense peak. Each wave runs independent chains of
// v_mfma_f32_32x32x16_bf16 on operands it loaded once from a caller's
// buffer (the clock the chip holds depends on how much the operands switch,
// so zeros would overstate it: the caller passes values with the layer's
// statistics), rotating through several operand registers so consecutive
// instructions see different data.
#include "hi3_moe.h"

#include "common.h"

namespace hi3 {

constexpr int kProbeChains = 4;   // independent accumulators per wave
constexpr int kProbeOperands = 4; // operand registers each chain cycles through

__global__ __launch_bounds__(256) void mfma_probe_kernel(const u32x4_t *__restrict__ bits,
                                                         float *__restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a[kProbeOperands], b[kProbeOperands];
#pragma unroll
  for (int i = 0; i < kProbeOperands; ++i) {
    a[i] = __builtin_bit_cast(bf16x8_t, bits[(2 * i) * 64 + lane]);
    b[i] = __builtin_bit_cast(bf16x8_t, bits[(2 * i + 1) * 64 + lane]);
  }
  f32x16_t acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kProbeOperands; ++i)
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(i + c) % kProbeOperands],
                                                          b[i], acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  // one value per wave, so the chains cannot be removed
  if (lane == 0) out[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = s;
}

}  // namespace hi3

extern "C" {

int64_t hi3_moe_probe_mfma_bf16(const void *operands, float *out, int32_t blocks,
                                int32_t iters, void *hip_stream) {
  if (!operands || !out) return HI3_E_NULL;
  if (blocks <= 0 || iters <= 0) return HI3_E_SHAPE;
  if ((reinterpret_cast<uintptr_t>(operands) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 15u) != 0)
    return HI3_E_UNSUPPORTED;
  hipLaunchKernelGGL(hi3::mfma_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(hip_stream),
                     static_cast<const hi3::u32x4_t *>(operands), out, iters);
  if (hipGetLastError() != hipSuccess) return HI3_E_HIP;
  // FLOP of the launch: 4 waves per block, each iteration kProbeOperands *
  // kProbeChains MFMAs of 2 * 32 * 32 * 16
  return static_cast<int64_t>(blocks) * 4 * iters * hi3::kProbeOperands * hi3::kProbeChains *
         (2 * 32 * 32 * 16);
}

}  // extern "C"
