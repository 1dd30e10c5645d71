// hi3_moe_forward_noalloc: the layer's forward for callers that cannot
// allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid allocation). Its kernels are hi3_moe_forward's; the
// workspace they need is a file-scope device array of a fixed size instead
// of a buffer of the caller's.
//
// Each GPU the library runs on holds one copy of the array until the process
// ends. Its device address is obtained once per device, on the first call
// made with that device current (hipGetSymbolAddress), and kept per device;
// host code uses only that address, never the array's name (which in host
// code is a host-side stand-in, not a device address).
//
// Every call on one GPU shares that GPU's array: calls that overlap on one
// GPU (two streams, or two host threads) race on it and must be ordered by
// the caller. The array keeps the last call's contents; nothing in it needs
// to start at zero, since the forward's kernels write every byte of the
// workspace they read.
#include <atomic>

#include "hi3_moe.h"

#include "common.h"

namespace {

constexpr size_t kScratchBytes = HI3_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
// Device address of each device's copy of scratch (null until the first
// call on that device). Two threads may both look it up at once; they store
// the same address.
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The device address of the current device's scratch, or null on failure.
void *scratch_of_current_device(int dev) {
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

int hi3_moe_forward_noalloc(const void *x, const float *w_router, const void *w_up_gate,
                            const void *w_down, const void *w_shared_up_gate,
                            const void *w_shared_down, const uint8_t *pad_mask, int64_t T,
                            int32_t H, int32_t E, int32_t K, int32_t I, int32_t I_shared,
                            int32_t dtype, void *out, int32_t *topk_idx, float *topk_w,
                            int32_t *expert_counts, void *hip_stream) {
  // the forward's own checks, against a workspace of the scratch's size
  // (any aligned non-null address stands in for it: nothing is enqueued)
  void *const stand_in = reinterpret_cast<void *>(uintptr_t{256});
  int st = hi3::forward_single_stream(x, w_router, w_up_gate, w_down, w_shared_up_gate,
                                      w_shared_down, pad_mask, T, H, E, K, I, I_shared, dtype,
                                      out, topk_idx, topk_w, expert_counts, stand_in,
                                      kScratchBytes, hip_stream, true);
  if (st == HI3_E_WORKSPACE) return HI3_E_SCRATCH;
  if (st != HI3_OK || T == 0) return st;
  // the scratch of the current device, which must be the stream's
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return HI3_E_HIP;
  if (dev >= kMaxDevices) return HI3_E_UNSUPPORTED;
  if (hipStreamGetDevice(static_cast<hipStream_t>(hip_stream), &sdev) != hipSuccess)
    return HI3_E_HIP;
  if (sdev != dev) return HI3_E_UNSUPPORTED;
  void *ws = scratch_of_current_device(dev);
  if (!ws) return HI3_E_HIP;
  return hi3::forward_single_stream(x, w_router, w_up_gate, w_down, w_shared_up_gate,
                                    w_shared_down, pad_mask, T, H, E, K, I, I_shared, dtype, out,
                                    topk_idx, topk_w, expert_counts, ws, kScratchBytes,
                                    hip_stream, false);
}

}  // extern "C"
