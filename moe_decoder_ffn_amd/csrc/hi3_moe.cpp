// Host side of the C ABI declared in include/hi3_moe.h: argument validation,
// workspace carve-up and the ordered enqueue of the kernels on the caller's
// stream. No device memory is allocated and no device-to-host copy is made.
#include "hi3_moe.h"

#include <hip/hip_runtime.h>

#include "common.h"

using namespace hi3;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// need_expert: the expert sizes I and Is are used (forward).
int check_sizes(int64_t T, int32_t H, int32_t E, int32_t K, int32_t I, int32_t Is,
                int32_t dtype, bool need_expert) {
  if (T < 0 || H <= 0 || E <= 0 || K <= 0 || K > E) return HI3_E_SHAPE;
  if (need_expert && (I <= 0 || Is <= 0)) return HI3_E_SHAPE;
  if (!need_expert && (I < 0 || Is < 0)) return HI3_E_SHAPE;
  if (dtype != HI3_F32 && dtype != HI3_BF16) return HI3_E_UNSUPPORTED;
  if (E > kMaxE) return HI3_E_UNSUPPORTED;
  if (H % 64 != 0 || I % 64 != 0 || Is % 64 != 0) return HI3_E_UNSUPPORTED;
  if (T * static_cast<int64_t>(K) >= (int64_t{1} << 31)) return HI3_E_UNSUPPORTED;
  return HI3_OK;
}

int all_aligned(std::initializer_list<const void *> ptrs) {
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return HI3_E_UNSUPPORTED;
  return HI3_OK;
}

struct Recorder {
  void *const *ev;
  hipStream_t s;
  bool ok = true;
  void at(int i) {  // NULL entries are skipped
    if (ev && ev[i] && hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) != hipSuccess)
      ok = false;
  }
};

#define HI3_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return HI3_E_HIP; \
  } while (0)

// eps must be a finite number >= 0.
bool eps_ok(float eps) { return eps >= 0.0f && eps <= 3.0e38f; }

// Whether a forward given a side stream runs the shared expert there: bf16,
// every row real, not the activation-saving forward (any tile plan: the
// dense launches take 256-row tiles of their own).
bool shared_on_side(const Plan &p, bool has_pad, bool save) {
  return kOverlapShared && !has_pad && !save && p.dtype == kBF16;
}

// The fork and join of the caller's side stream for one forward: two events
// made for this call and destroyed when it returns (a destroyed event's
// pending record and waits still complete). If the call leaves early after
// the fork, the destructor joins the side stream back into the main stream,
// so nothing enqueued after the call can overtake the side stream's work.
struct SideFork {
  hipStream_t main = nullptr, side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool armed = false;
  bool make() {
    return hipEventCreateWithFlags(&fork, hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&join, hipEventDisableTiming) == hipSuccess;
  }
  bool start() {  // the side stream waits for everything enqueued on main so far
    if (hipEventRecord(fork, main) != hipSuccess) return false;
    if (hipStreamWaitEvent(side, fork, 0) != hipSuccess) return false;
    armed = true;
    return true;
  }
  bool end() {  // main waits for everything enqueued on side so far
    armed = false;
    return hipEventRecord(join, side) == hipSuccess &&
           hipStreamWaitEvent(main, join, 0) == hipSuccess;
  }
  ~SideFork() {
    if (armed) (void)end();
    if (fork) (void)hipEventDestroy(fork);
    if (join) (void)hipEventDestroy(join);
  }
};

// norm_weight != null: the block's RMSNorm runs first (x is the residual
// stream h) and the combine adds h back; otherwise x feeds the layer directly.
int forward_impl(const void *x, const void *norm_weight, float eps, const float *w_router,
                 const void *w_up_gate, const void *w_down, const void *w_shared_up_gate,
                 const void *w_shared_down, const uint8_t *pad_mask, int64_t T, int32_t H,
                 int32_t E, int32_t K, int32_t I, int32_t Is, int32_t dtype, void *out,
                 int32_t *topk_idx, float *topk_w, int32_t *expert_counts, void *workspace,
                 size_t workspace_bytes, void *hip_stream, void *const *events,
                 bool save = false, void *side_stream = nullptr, bool validate_only = false) {
  if (!x || !w_router || !w_up_gate || !w_down || !w_shared_up_gate || !w_shared_down || !out)
    return HI3_E_NULL;
  int st = check_sizes(T, H, E, K, I, Is, dtype, true);
  if (st != HI3_OK) return st;
  if (norm_weight && !eps_ok(eps)) return HI3_E_UNSUPPORTED;
  if (T == 0) return HI3_OK;
  if (!workspace) return HI3_E_NULL;
  st = all_aligned({x, norm_weight, w_router, w_up_gate, w_down, w_shared_up_gate,
                    w_shared_down, pad_mask, out, topk_idx, topk_w, expert_counts, workspace});
  if (st != HI3_OK) return st;
  // save: the backward's layout, so that hi3_moe_backward_after_forward finds
  // the routes, slot maps, u, g and h where it reads them
  const Plan p = make_plan(T, H, E, K, I, Is, dtype, save);
  if (workspace_bytes < p.total) return HI3_E_WORKSPACE;
  if (validate_only) return HI3_OK;

  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  char *ws = static_cast<char *>(workspace);
  auto at = [&](size_t off) { return static_cast<void *>(ws + off); };
  // The shared expert's GEMMs on the caller's side stream, alongside the
  // routing: when the caller gives one, every row is real (the shared rows
  // are then 0 .. T-1 and need nothing from the routing), outside the
  // activation-saving forward (whose layout keeps the shared rows in the
  // grouped list).
  hipStream_t side_s = static_cast<hipStream_t>(side_stream);
  const bool side = side_s && side_s != s && shared_on_side(p, pad_mask != nullptr, save);
  SideFork fork;
  if (side) {
    fork.main = s;
    fork.side = side_s;
    if (!fork.make()) return HI3_E_HIP;
  }
  // The block's RMSNorm: bf16 layers normalise inside the router kernel
  // (below), which writes the normalised rows for the expert GEMMs; fp32
  // layers run the RMSNorm kernel first.
  const void *resid = nullptr;
  const void *x_in = x;
  const bool fused_norm = norm_weight && dtype == HI3_BF16;
  if (norm_weight) {
    if (!fused_norm) {
      NormArgs na{x, norm_weight, pad_mask, T, H, eps, at(p.xn)};
      HI3_TRY(launch_rmsnorm(na, dtype, s));
    }
    resid = x;
    x = at(p.xn);
  }
  // fork: the side stream starts after everything enqueued on s so far and
  // runs the shared expert's rows, the tokens 0 .. T-1 in order (measured:
  // forking here beats forking after the router or the dispatch, though the
  // shared GEMM's blocks then delay the routing's). With the RMSNorm fused
  // into the router, the rows exist only after it: the fork follows it.
  auto fork_shared = [&]() -> int {
    if (!side) return HI3_OK;
    if (!fork.start()) return HI3_E_HIP;
    GemmArgs us{};
    us.cls[1] = GemmClass{x, H, nullptr, w_shared_up_gate, 0, at(p.hs), Is, 2 * Is, H};
    HI3_TRY(launch_gemm_dense(us, static_cast<int>(T), 0, side_s));
    GemmArgs ds{};
    ds.cls[1] = GemmClass{at(p.hs), Is, nullptr, w_shared_down, 0, at(p.ys), H, H, Is};
    HI3_TRY(launch_gemm_dense(ds, static_cast<int>(T), 1, side_s));
    return HI3_OK;
  };
  if (!fused_norm) {
    st = fork_shared();
    if (st != HI3_OK) return st;
  }
  // the main list holds the shared group's row tiles only when the side
  // stream does not run them
  const int main_tiles = p.max_tiles - (side ? static_cast<int>((T + p.BM - 1) / p.BM) : 0);
  int32_t *idx = topk_idx && !save ? topk_idx : static_cast<int32_t *>(at(p.idx));
  float *wts = topk_w && !save ? topk_w : static_cast<float *>(at(p.wts));
  int32_t *blkcnt = static_cast<int32_t *>(at(p.blkcnt));
  int32_t *blkval = static_cast<int32_t *>(at(p.blkval));
  int32_t *slotof = static_cast<int32_t *>(at(p.slotof));
  int32_t *vtok = static_cast<int32_t *>(at(p.vtok));
  int32_t *vidx = static_cast<int32_t *>(at(p.vidx));
  const int4 *tiles = static_cast<const int4 *>(at(p.tiles));
  const int32_t *gto = static_cast<const int32_t *>(at(p.gto));
  Recorder rec{events, s};

  // 0: router + per-block histogram
  rec.at(0);
  RouterArgs ra{fused_norm ? x_in : x, w_router, fused_norm ? norm_weight : nullptr, eps,
                fused_norm ? at(p.xn) : nullptr,
                static_cast<float *>(at(p.rnorm)), pad_mask, T, H, E, K, idx, wts, blkcnt,
                blkval};
  HI3_TRY(launch_router(ra, dtype, static_cast<float *>(at(p.rpart)), s));
  if (fused_norm) {
    st = fork_shared();
    if (st != HI3_OK) return st;
  }
  // 1: dispatch: expert offsets, GEMM row tiles, real-row list, stable slots
  rec.at(1);
  ScanArgs sa{blkcnt, blkval, p.NB, E, p.BM, static_cast<int32_t *>(at(p.eoff)), expert_counts,
              static_cast<int32_t *>(at(p.counts)), static_cast<int32_t *>(at(p.misc)),
              static_cast<int32_t *>(at(p.gto)), static_cast<int4 *>(at(p.tiles))};
  sa.no_shared = side ? 1 : 0;
  int32_t *perm = static_cast<int32_t *>(at(p.perm));
  ScatterArgs sc{idx, pad_mask, T, E, K, perm, slotof, vtok, vidx};
  HI3_TRY(launch_dispatch(sa, &sc, s));
  // 2: grouped [up; gate] projection + SwiGLU (routed experts and the shared
  // expert); the routed rows are gathered from x through the slot -> token map
  // by the GEMM's operand copies, so no grouped copy of x is materialised
  rec.at(2);
  GemmArgs up{};
  up.cls[0] = GemmClass{x, H, perm, w_up_gate, int64_t{2} * I * H, at(p.h), I, 2 * I, H};
  up.cls[1] = GemmClass{x, H, vtok, w_shared_up_gate, 0, at(p.hs), Is, 2 * Is, H};
  if (save) {
    up.cls[0].ug = static_cast<float *>(at(p.ug));
    up.cls[1].ug = static_cast<float *>(at(p.ugs));
  }
  up.tiles = tiles;
  up.gto = gto;
  up.E = E;
  HI3_TRY(launch_gemm_upgate(up, main_tiles, p.BM, dtype, s));
  // 3: grouped down projection
  rec.at(3);
  GemmArgs dn{};
  dn.cls[0] = GemmClass{at(p.h), I, nullptr, w_down, int64_t{H} * I, at(p.y), H, H, I};
  dn.cls[1] = GemmClass{at(p.hs), Is, nullptr, w_shared_down, 0, at(p.ys), H, H, Is};
  dn.tiles = tiles;
  dn.gto = gto;
  dn.E = E;
  HI3_TRY(launch_gemm_down(dn, main_tiles, p.BM, dtype, s));
  // 4: combine (after the shared expert's output, when the side stream made it)
  rec.at(4);
  if (side && !fork.end()) return HI3_E_HIP;
  CombineArgs ca{static_cast<const float *>(at(p.y)), static_cast<const float *>(at(p.ys)),
                 slotof, vidx, wts, pad_mask, T, H, K, out, resid};
  HI3_TRY(launch_combine(ca, dtype, s));
  if (save && topk_idx)
    HI3_TRY(hipMemcpyAsync(topk_idx, idx, size_t(T) * K * 4, hipMemcpyDeviceToDevice, s));
  if (save && topk_w)
    HI3_TRY(hipMemcpyAsync(topk_w, wts, size_t(T) * K * 4, hipMemcpyDeviceToDevice, s));
  rec.at(5);
  return rec.ok ? HI3_OK : HI3_E_HIP;
}

// Gradient of sum over real rows of dout . out with the routes held fixed:
// the routes and the [up; gate] projection are recomputed (u and g kept in
// fp32), then the gradients flow through the down projection (mode 2, with
// the SwiGLU backward in its epilogue), the [up; gate] projection (mode 3),
// the router, and into the weight gradients (mode 4).
int backward_impl(const void *x, const float *w_router, const void *w_up_gate,
                  const void *w_down, const void *w_shared_up_gate, const void *w_shared_down,
                  const uint8_t *pad_mask, const void *dout, int64_t T, int32_t H, int32_t E,
                  int32_t K, int32_t I, int32_t Is, int32_t dtype, void *dx, float *dw_router,
                  void *dw_up_gate, void *dw_down, void *dw_shared_up_gate,
                  void *dw_shared_down, void *workspace, size_t workspace_bytes,
                  void *hip_stream, void *const *events, bool reuse = false,
                  const void *norm_weight = nullptr, float eps = 0.0f,
                  void *dnorm_weight = nullptr) {
  int st = check_sizes(T, H, E, K, I, Is, dtype, true);
  if (st != HI3_OK) return st;
  if (norm_weight && !eps_ok(eps)) return HI3_E_UNSUPPORTED;
  // with no rows the inputs are not read (they may be NULL)
  if (T > 0 &&
      (!x || !w_router || !w_up_gate || !w_down || !w_shared_up_gate || !w_shared_down || !dout))
    return HI3_E_NULL;
  st = all_aligned({x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask,
                    dout, dx, dw_router, dw_up_gate, dw_down, dw_shared_up_gate, dw_shared_down,
                    workspace, norm_weight, dnorm_weight});
  if (st != HI3_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const size_t es = dtype == HI3_BF16 ? 2 : 4;
  if (T == 0) {
    // no rows: every requested weight gradient is zero
    HI3_TRY(launch_zero(dnorm_weight, dnorm_weight ? size_t(H) * es : 0, s));
    HI3_TRY(launch_zero(dw_router, dw_router ? size_t(E) * H * 4 : 0, s));
    HI3_TRY(launch_zero(dw_up_gate, dw_up_gate ? size_t(E) * 2 * I * H * es : 0, s));
    HI3_TRY(launch_zero(dw_down, dw_down ? size_t(E) * H * I * es : 0, s));
    HI3_TRY(launch_zero(dw_shared_up_gate, dw_shared_up_gate ? size_t(2) * Is * H * es : 0, s));
    HI3_TRY(launch_zero(dw_shared_down, dw_shared_down ? size_t(H) * Is * es : 0, s));
    return HI3_OK;
  }
  if (!workspace) return HI3_E_NULL;
  const Plan p = make_plan(T, H, E, K, I, Is, dtype, true);
  if (workspace_bytes < p.total) return HI3_E_WORKSPACE;

  char *ws = static_cast<char *>(workspace);
  auto at = [&](size_t off) { return static_cast<void *>(ws + off); };
  int32_t *idx = static_cast<int32_t *>(at(p.idx));
  float *wts = static_cast<float *>(at(p.wts));
  int32_t *blkcnt = static_cast<int32_t *>(at(p.blkcnt));
  int32_t *blkval = static_cast<int32_t *>(at(p.blkval));
  int32_t *slotof = static_cast<int32_t *>(at(p.slotof));
  int32_t *perm = static_cast<int32_t *>(at(p.perm));
  int32_t *vtok = static_cast<int32_t *>(at(p.vtok));
  int32_t *vidx = static_cast<int32_t *>(at(p.vidx));
  const int4 *tiles = static_cast<const int4 *>(at(p.tiles));
  const int32_t *gto = static_cast<const int32_t *>(at(p.gto));
  const int32_t *eoff = static_cast<const int32_t *>(at(p.eoff));
  const int32_t *counts = static_cast<const int32_t *>(at(p.counts));
  const int32_t *misc = static_cast<const int32_t *>(at(p.misc));
  Recorder rec{events, s};

  // the block's backward: the layer runs on the normalised rows, and its dx
  // (dL/dxn) stays in fp32 for RMSNorm's backward at the end
  const void *h_in = x;
  const bool norm = norm_weight != nullptr;
  const bool fused_norm = norm && dtype == HI3_BF16;  // normalised in the router kernel
  void *dh = dx;
  if (norm) {
    if (!fused_norm) {
      NormArgs na{x, norm_weight, pad_mask, T, H, eps, at(p.xn)};
      HI3_TRY(launch_rmsnorm(na, dtype, s));
    }
    x = at(p.xn);
    dx = nullptr;
  }
  const bool want_dxn = norm && (dh || dnorm_weight);

  // 0-2: routes, offsets, slots (as in the forward); 3: the [up; gate]
  // projection again: h as the forward stores it, u and g in fp32. After
  // hi3_moe_forward_train all of this is already in the workspace.
  rec.at(0);
  if (!reuse) {
    RouterArgs ra{fused_norm ? h_in : x, w_router, fused_norm ? norm_weight : nullptr, eps,
                  fused_norm ? at(p.xn) : nullptr,
                  static_cast<float *>(at(p.rnorm)), pad_mask, T, H, E, K, idx, wts, blkcnt,
                  blkval};
    HI3_TRY(launch_router(ra, dtype, static_cast<float *>(at(p.rpart)), s));
  }
  rec.at(1);
  if (!reuse) {
    ScanArgs sa{blkcnt, blkval, p.NB, E, p.BM, static_cast<int32_t *>(at(p.eoff)), nullptr,
                static_cast<int32_t *>(at(p.counts)), static_cast<int32_t *>(at(p.misc)),
                static_cast<int32_t *>(at(p.gto)), static_cast<int4 *>(at(p.tiles))};
    ScatterArgs sc{idx, pad_mask, T, E, K, perm, slotof, vtok, vidx};
    HI3_TRY(launch_dispatch(sa, &sc, s));
  }
  // The [up; gate] projection again (h as the forward stores it). bf16
  // layers run it after dh, with the SwiGLU backward in its epilogue (u and g
  // never leave the registers; dh is kept in the u, g buffer); fp32 layers
  // store u and g (fp32) for the dh GEMM's epilogue, as the training forward
  // does for hi3_moe_backward_after_forward.
  const bool fused_swiglu_bwd = !reuse && dtype == HI3_BF16 && kGemmStagedStore;
  float *apart = static_cast<float *>(at(p.apart));
  auto recompute = [&](bool with_bwd) -> int {
    GemmArgs up{};
    up.cls[0] = GemmClass{x, H, perm, w_up_gate, int64_t{2} * I * H, at(p.h), I, 2 * I, H};
    up.cls[1] = GemmClass{x, H, vtok, w_shared_up_gate, 0, at(p.hs), Is, 2 * Is, H};
    if (with_bwd) {
      up.cls[0].dh_in = static_cast<const float *>(at(p.ug));
      up.cls[0].dd_out = at(p.dd);
      up.cls[0].apart = apart;
      up.cls[0].apart_ld = p.P;
      up.cls[1].dh_in = static_cast<const float *>(at(p.ugs));
      up.cls[1].dd_out = at(p.dds);
    } else {
      up.cls[0].ug = static_cast<float *>(at(p.ug));
      up.cls[1].ug = static_cast<float *>(at(p.ugs));
    }
    up.tiles = tiles;
    up.gto = gto;
    up.E = E;
    HI3_TRY(launch_gemm_upgate(up, p.max_tiles, p.BM, dtype, s));
    return HI3_OK;
  };
  // 2: x and w dout by slot; x and dout by real row when there is padding
  // (fp32 layers: after the recompute, which this stage then includes)
  rec.at(2);
  if (!reuse && !fused_swiglu_bwd) {
    st = recompute(false);
    if (st != HI3_OK) return st;
  }
  const bool compact = pad_mask != nullptr;
  BwdGatherArgs ga{x, dout, wts, slotof, vidx, pad_mask, T, H, K, at(p.xs), at(p.dys),
                   static_cast<float *>(at(p.wslot)), compact ? at(p.xv) : nullptr,
                   compact ? at(p.doutv) : nullptr};
  HI3_TRY(launch_bwd_gather(ga, dtype, s));
  // 3: dh = w W2^T dout (dout rows gathered through the slot -> token map, w
  // applied in fp32); with u and g stored, the SwiGLU backward in the same
  // epilogue: [du; dg], partial sums of dh h; else dh alone (fp32)
  rec.at(3);
  GemmArgs d2{};
  d2.cls[0] = GemmClass{dout, H, perm, w_down, int64_t{H} * I, at(p.dd), 2 * I, I, H};
  d2.cls[0].rowscale = static_cast<const float *>(at(p.wslot));
  d2.cls[0].ldb = I;
  d2.cls[1] = GemmClass{dout, H, vtok, w_shared_down, 0, at(p.dds), 2 * Is, Is, H};
  d2.cls[1].ldb = Is;
  if (fused_swiglu_bwd) {
    d2.cls[0].C = at(p.ug);  // dh [T*K, I] fp32
    d2.cls[0].ldc = I;
    d2.cls[1].C = at(p.ugs);  // dh [T, Is] fp32
    d2.cls[1].ldc = Is;
  } else {
    d2.cls[0].ug = static_cast<float *>(at(p.ug));
    d2.cls[0].hsave = at(p.h);
    d2.cls[0].apart = apart;
    d2.cls[0].apart_ld = p.P;
    d2.cls[1].ug = static_cast<float *>(at(p.ugs));
    d2.cls[1].hsave = at(p.hs);
  }
  d2.tiles = tiles;
  d2.gto = gto;
  d2.E = E;
  HI3_TRY(launch_gemm_dgrad_down(d2, p.max_tiles, p.BM, dtype, s));
  // 4: (bf16) the recompute with the SwiGLU backward
  rec.at(4);
  if (fused_swiglu_bwd) {
    st = recompute(true);
    if (st != HI3_OK) return st;
  }
  // 6: dx by slot / by real row = W13^T [du; dg]
  rec.at(5);
  if (dx || want_dxn) {
    GemmArgs d3{};
    d3.cls[0] = GemmClass{at(p.dd), 2 * I, nullptr, w_up_gate, int64_t{2} * I * H, at(p.y), H,
                          H, 2 * I};
    d3.cls[0].ldb = H;
    d3.cls[1] = GemmClass{at(p.dds), 2 * Is, nullptr, w_shared_up_gate, 0, at(p.ys), H, H,
                          2 * Is};
    d3.cls[1].ldb = H;
    d3.tiles = tiles;
    d3.gto = gto;
    d3.E = E;
    HI3_TRY(launch_gemm_dgrad_up_gate(d3, p.max_tiles, p.BM, dtype, s));
  }
  // 7: logit gradient and dx
  rec.at(6);
  float *dls = static_cast<float *>(at(p.dls));
  BwdCombineArgs ca{static_cast<const float *>(at(p.y)), static_cast<const float *>(at(p.ys)),
                    static_cast<const float *>(at(p.apart)), p.P, slotof, idx, vidx, wts,
                    w_router, pad_mask, T, H, K, dls, dx,
                    want_dxn ? static_cast<float *>(at(p.dxn)) : nullptr};
  HI3_TRY(launch_bwd_combine(ca, dtype, s));
  // 8: router weight gradient
  rec.at(7);
  if (dw_router)
    HI3_TRY(launch_dw_router(dls, at(p.xs), tiles, gto, p.max_tiles, E, H, dtype,
                             static_cast<float *>(at(p.dwrpart)), dw_router, s));
  // 9, 10: expert weight gradients
  HI3_TRY(launch_zero(at(p.zrow), 512, s));
  rec.at(8);
  GemmArgs w2{};
  w2.goff = eoff;
  w2.gcnt = counts;
  w2.nreal = misc;
  w2.zrow = at(p.zrow);
  w2.E = E;
  if (dw_down) {
    w2.cls[0].A = at(p.dys); w2.cls[0].lda = H;
    w2.cls[0].B = at(p.h); w2.cls[0].ldb = I;
    w2.cls[0].C = dw_down; w2.cls[0].ldc = I; w2.cls[0].strideC = int64_t{H} * I;
    w2.cls[0].M = H; w2.cls[0].N = I;
  }
  if (dw_shared_down) {
    w2.cls[1].A = compact ? at(p.doutv) : dout; w2.cls[1].lda = H;
    w2.cls[1].B = at(p.hs); w2.cls[1].ldb = Is;
    w2.cls[1].C = dw_shared_down; w2.cls[1].ldc = Is;
    w2.cls[1].M = H; w2.cls[1].N = Is;
  }
  HI3_TRY(launch_gemm_wgrad(w2, E, dtype, s));
  rec.at(9);
  GemmArgs w13 = w2;
  w13.cls[0] = GemmClass{};
  w13.cls[1] = GemmClass{};
  if (dw_up_gate) {
    w13.cls[0].A = at(p.dd); w13.cls[0].lda = 2 * I;
    w13.cls[0].B = at(p.xs); w13.cls[0].ldb = H;
    w13.cls[0].C = dw_up_gate; w13.cls[0].ldc = H; w13.cls[0].strideC = int64_t{2} * I * H;
    w13.cls[0].M = 2 * I; w13.cls[0].N = H;
  }
  if (dw_shared_up_gate) {
    w13.cls[1].A = at(p.dds); w13.cls[1].lda = 2 * Is;
    w13.cls[1].B = compact ? at(p.xv) : x; w13.cls[1].ldb = H;
    w13.cls[1].C = dw_shared_up_gate; w13.cls[1].ldc = H;
    w13.cls[1].M = 2 * Is; w13.cls[1].N = H;
  }
  HI3_TRY(launch_gemm_wgrad(w13, E, dtype, s));
  rec.at(10);
  if (want_dxn) {
    NormBwdArgs nb{h_in, norm_weight, pad_mask, T, H, eps,
                   static_cast<const float *>(at(p.dxn)), dout, dh,
                   static_cast<float *>(at(p.rrow)), static_cast<float *>(at(p.nwpart)),
                   dnorm_weight};
    HI3_TRY(launch_rmsnorm_backward(nb, dtype, s));
  }
  return rec.ok ? HI3_OK : HI3_E_HIP;
}

}  // namespace

namespace hi3 {

// hi3_moe_forward with the workspace given by the caller of this function
// (the no-allocation entry point passes its static scratch); validate_only:
// check the arguments as the forward does, enqueue nothing.
int forward_single_stream(const void *x, const float *w_router, const void *w_up_gate,
                          const void *w_down, const void *w_shared_up_gate,
                          const void *w_shared_down, const uint8_t *pad_mask, int64_t T,
                          int32_t H, int32_t E, int32_t K, int32_t I, int32_t I_shared,
                          int32_t dtype, void *out, int32_t *topk_idx, float *topk_w,
                          int32_t *expert_counts, void *workspace, size_t workspace_bytes,
                          void *hip_stream, bool validate_only) {
  return forward_impl(x, nullptr, 0.0f, w_router, w_up_gate, w_down, w_shared_up_gate,
                      w_shared_down, pad_mask, T, H, E, K, I, I_shared, dtype, out, topk_idx,
                      topk_w, expert_counts, workspace, workspace_bytes, hip_stream, nullptr,
                      false, nullptr, validate_only);
}

}  // namespace hi3

extern "C" {

size_t hi3_moe_workspace_size(int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                              int32_t I_shared, int32_t dtype) {
  const bool expert = I > 0 || I_shared > 0;
  if (check_sizes(T, H, E, K, I, I_shared, dtype, expert) != HI3_OK) return 0;
  if (T == 0) return 0;
  return make_plan(T, H, E, K, expert ? I : 0, expert ? I_shared : 0, dtype).total;
}

int hi3_moe_route(const void *x, const float *w_router, const uint8_t *pad_mask, int64_t T,
                  int32_t H, int32_t E, int32_t K, int32_t dtype, int32_t *topk_idx,
                  float *topk_w, int32_t *expert_counts, void *workspace,
                  size_t workspace_bytes, void *hip_stream) {
  if (!x || !w_router || !topk_idx || !topk_w) return HI3_E_NULL;
  int st = check_sizes(T, H, E, K, 0, 0, dtype, false);
  if (st != HI3_OK) return st;
  if (T == 0) return HI3_OK;
  if (!workspace) return HI3_E_NULL;
  st = all_aligned({x, w_router, pad_mask, topk_idx, topk_w, expert_counts, workspace});
  if (st != HI3_OK) return st;
  const Plan p = make_plan(T, H, E, K, 0, 0, dtype);
  if (workspace_bytes < p.total) return HI3_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  char *ws = static_cast<char *>(workspace);
  auto at = [&](size_t off) { return static_cast<void *>(ws + off); };
  RouterArgs ra{x, w_router, nullptr, 0.0f, nullptr, nullptr,
                pad_mask, T, H, E, K, topk_idx, topk_w,
                static_cast<int32_t *>(at(p.blkcnt)),
                static_cast<int32_t *>(at(p.blkval))};
  HI3_TRY(launch_router(ra, dtype, static_cast<float *>(at(p.rpart)), s));
  if (expert_counts) {
    ScanArgs sa{ra.blkcnt, ra.blkval, p.NB, E, p.BM, static_cast<int32_t *>(at(p.eoff)),
                expert_counts, static_cast<int32_t *>(at(p.counts)),
                static_cast<int32_t *>(at(p.misc)), static_cast<int32_t *>(at(p.gto)),
                static_cast<int4 *>(at(p.tiles))};
    HI3_TRY(launch_dispatch(sa, nullptr, s));
  }
  return HI3_OK;
}

int hi3_moe_dispatch(const int32_t *topk_idx, const uint8_t *pad_mask, const void *x,
                     int64_t T, int32_t H, int32_t E, int32_t K, int32_t dtype,
                     int32_t *expert_offsets, int32_t *perm_token, int32_t *slot_of,
                     void *x_sorted, void *workspace, size_t workspace_bytes,
                     void *hip_stream) {
  if (!topk_idx || !expert_offsets || !perm_token || !slot_of) return HI3_E_NULL;
  if (x_sorted && !x) return HI3_E_NULL;
  int st = check_sizes(T, H, E, K, 0, 0, dtype, false);
  if (st != HI3_OK) return st;
  if (T == 0) return HI3_OK;
  if (!workspace) return HI3_E_NULL;
  st = all_aligned({topk_idx, pad_mask, x, expert_offsets, perm_token, slot_of, x_sorted,
                    workspace});
  if (st != HI3_OK) return st;
  const Plan p = make_plan(T, H, E, K, 0, 0, dtype);
  if (workspace_bytes < p.total) return HI3_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  char *ws = static_cast<char *>(workspace);
  auto at = [&](size_t off) { return static_cast<void *>(ws + off); };
  int32_t *blkcnt = static_cast<int32_t *>(at(p.blkcnt));
  int32_t *blkval = static_cast<int32_t *>(at(p.blkval));
  HI3_TRY(launch_histogram(topk_idx, pad_mask, T, E, K, blkcnt, blkval, s));
  ScanArgs sa{blkcnt, blkval, p.NB, E, p.BM, expert_offsets, nullptr,
              static_cast<int32_t *>(at(p.counts)), static_cast<int32_t *>(at(p.misc)),
              static_cast<int32_t *>(at(p.gto)), static_cast<int4 *>(at(p.tiles))};
  ScatterArgs sc{topk_idx, pad_mask, T, E, K, perm_token, slot_of, nullptr, nullptr};
  HI3_TRY(launch_dispatch(sa, &sc, s));
  if (x_sorted) {
    const size_t es = dtype == HI3_BF16 ? 2 : 4;
    HI3_TRY(launch_gather(x, static_cast<int64_t>(H) * es, slot_of, pad_mask, T, K, x_sorted, s));
  }
  return HI3_OK;
}

int hi3_moe_forward(const void *x, const float *w_router, const void *w_up_gate,
                    const void *w_down, const void *w_shared_up_gate,
                    const void *w_shared_down, const uint8_t *pad_mask, int64_t T,
                    int32_t H, int32_t E, int32_t K, int32_t I, int32_t I_shared,
                    int32_t dtype, void *out, int32_t *topk_idx, float *topk_w,
                    int32_t *expert_counts, void *workspace, size_t workspace_bytes,
                    void *hip_stream) {
  return forward_impl(x, nullptr, 0.0f, w_router, w_up_gate, w_down, w_shared_up_gate,
                      w_shared_down, pad_mask, T, H, E, K, I, I_shared, dtype, out, topk_idx,
                      topk_w, expert_counts, workspace, workspace_bytes, hip_stream, nullptr);
}

int hi3_moe_forward_overlap(const void *x, const float *w_router, const void *w_up_gate,
                            const void *w_down, const void *w_shared_up_gate,
                            const void *w_shared_down, const uint8_t *pad_mask, int64_t T,
                            int32_t H, int32_t E, int32_t K, int32_t I, int32_t I_shared,
                            int32_t dtype, void *out, int32_t *topk_idx, float *topk_w,
                            int32_t *expert_counts, void *workspace, size_t workspace_bytes,
                            void *hip_stream, void *side_stream) {
  return forward_impl(x, nullptr, 0.0f, w_router, w_up_gate, w_down, w_shared_up_gate,
                      w_shared_down, pad_mask, T, H, E, K, I, I_shared, dtype, out, topk_idx,
                      topk_w, expert_counts, workspace, workspace_bytes, hip_stream, nullptr,
                      false, side_stream);
}

int hi3_moe_forward_instrumented(const void *x, const float *w_router, const void *w_up_gate,
                                 const void *w_down, const void *w_shared_up_gate,
                                 const void *w_shared_down, const uint8_t *pad_mask,
                                 int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                                 int32_t I_shared, int32_t dtype, void *out,
                                 int32_t *topk_idx, float *topk_w, int32_t *expert_counts,
                                 void *workspace, size_t workspace_bytes, void *hip_stream,
                                 void *side_stream, void *const *stage_events) {
  if (!stage_events) return HI3_E_NULL;
  return forward_impl(x, nullptr, 0.0f, w_router, w_up_gate, w_down, w_shared_up_gate,
                      w_shared_down, pad_mask, T, H, E, K, I, I_shared, dtype, out, topk_idx,
                      topk_w, expert_counts, workspace, workspace_bytes, hip_stream,
                      stage_events, false, side_stream);
}

int hi3_moe_forward_norm_residual(const void *h, const void *norm_weight, float eps,
                                  const float *w_router, const void *w_up_gate,
                                  const void *w_down, const void *w_shared_up_gate,
                                  const void *w_shared_down, const uint8_t *pad_mask,
                                  int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                                  int32_t I_shared, int32_t dtype, void *out,
                                  int32_t *topk_idx, float *topk_w, int32_t *expert_counts,
                                  void *workspace, size_t workspace_bytes,
                                  void *hip_stream) {
  if (!norm_weight) return HI3_E_NULL;
  return forward_impl(h, norm_weight, eps, w_router, w_up_gate, w_down, w_shared_up_gate,
                      w_shared_down, pad_mask, T, H, E, K, I, I_shared, dtype, out, topk_idx,
                      topk_w, expert_counts, workspace, workspace_bytes, hip_stream, nullptr);
}

int hi3_moe_rmsnorm(const void *x, const void *weight, float eps, const uint8_t *pad_mask,
                    int64_t T, int32_t H, int32_t dtype, void *xn, void *hip_stream) {
  if (!x || !weight || !xn) return HI3_E_NULL;
  if (T < 0 || H <= 0) return HI3_E_SHAPE;
  if (dtype != HI3_F32 && dtype != HI3_BF16) return HI3_E_UNSUPPORTED;
  if (H % 64 != 0 || !eps_ok(eps)) return HI3_E_UNSUPPORTED;
  if (all_aligned({x, weight, pad_mask, xn}) != HI3_OK) return HI3_E_UNSUPPORTED;
  if (T == 0) return HI3_OK;
  NormArgs na{x, weight, pad_mask, T, H, eps, xn};
  HI3_TRY(launch_rmsnorm(na, dtype, static_cast<hipStream_t>(hip_stream)));
  return HI3_OK;
}

int hi3_moe_forward_shared_on_side(int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                                   int32_t I_shared, int32_t dtype, int32_t has_pad_mask) {
  if (check_sizes(T, H, E, K, I, I_shared, dtype, true) != HI3_OK || T == 0) return 0;
  return shared_on_side(make_plan(T, H, E, K, I, I_shared, dtype), has_pad_mask != 0, false)
             ? 1 : 0;
}

size_t hi3_moe_backward_workspace_size(int64_t T, int32_t H, int32_t E, int32_t K, int32_t I,
                                       int32_t I_shared, int32_t dtype) {
  if (check_sizes(T, H, E, K, I, I_shared, dtype, true) != HI3_OK) return 0;
  if (T == 0) return 0;
  return make_plan(T, H, E, K, I, I_shared, dtype, true).total;
}

int hi3_moe_backward(const void *x, const float *w_router, const void *w_up_gate,
                     const void *w_down, const void *w_shared_up_gate,
                     const void *w_shared_down, const uint8_t *pad_mask, const void *dout,
                     int64_t T, int32_t H, int32_t E, int32_t K, int32_t I, int32_t I_shared,
                     int32_t dtype, void *dx, float *dw_router, void *dw_up_gate,
                     void *dw_down, void *dw_shared_up_gate, void *dw_shared_down,
                     void *workspace, size_t workspace_bytes, void *hip_stream) {
  return backward_impl(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask,
                       dout, T, H, E, K, I, I_shared, dtype, dx, dw_router, dw_up_gate, dw_down,
                       dw_shared_up_gate, dw_shared_down, workspace, workspace_bytes, hip_stream,
                       nullptr);
}

int hi3_moe_backward_instrumented(const void *x, const float *w_router, const void *w_up_gate,
                                  const void *w_down, const void *w_shared_up_gate,
                                  const void *w_shared_down, const uint8_t *pad_mask,
                                  const void *dout, int64_t T, int32_t H, int32_t E, int32_t K,
                                  int32_t I, int32_t I_shared, int32_t dtype, void *dx,
                                  float *dw_router, void *dw_up_gate, void *dw_down,
                                  void *dw_shared_up_gate, void *dw_shared_down,
                                  void *workspace, size_t workspace_bytes, void *hip_stream,
                                  void *const *stage_events) {
  if (!stage_events) return HI3_E_NULL;
  return backward_impl(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask,
                       dout, T, H, E, K, I, I_shared, dtype, dx, dw_router, dw_up_gate, dw_down,
                       dw_shared_up_gate, dw_shared_down, workspace, workspace_bytes, hip_stream,
                       stage_events);
}

int hi3_moe_forward_train(const void *x, const float *w_router, const void *w_up_gate,
                          const void *w_down, const void *w_shared_up_gate,
                          const void *w_shared_down, const uint8_t *pad_mask, int64_t T,
                          int32_t H, int32_t E, int32_t K, int32_t I, int32_t I_shared,
                          int32_t dtype, void *out, int32_t *topk_idx, float *topk_w,
                          int32_t *expert_counts, void *workspace, size_t workspace_bytes,
                          void *hip_stream) {
  return forward_impl(x, nullptr, 0.0f, w_router, w_up_gate, w_down, w_shared_up_gate,
                      w_shared_down, pad_mask, T, H, E, K, I, I_shared, dtype, out, topk_idx,
                      topk_w, expert_counts, workspace, workspace_bytes, hip_stream, nullptr,
                      true);
}

int hi3_moe_backward_after_forward(const void *x, const float *w_router, const void *w_up_gate,
                                   const void *w_down, const void *w_shared_up_gate,
                                   const void *w_shared_down, const uint8_t *pad_mask,
                                   const void *dout, int64_t T, int32_t H, int32_t E, int32_t K,
                                   int32_t I, int32_t I_shared, int32_t dtype, void *dx,
                                   float *dw_router, void *dw_up_gate, void *dw_down,
                                   void *dw_shared_up_gate, void *dw_shared_down,
                                   void *workspace, size_t workspace_bytes, void *hip_stream) {
  return backward_impl(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask,
                       dout, T, H, E, K, I, I_shared, dtype, dx, dw_router, dw_up_gate, dw_down,
                       dw_shared_up_gate, dw_shared_down, workspace, workspace_bytes, hip_stream,
                       nullptr, true);
}

int hi3_moe_backward_norm_residual(const void *h, const void *norm_weight, float eps,
                                   const float *w_router, const void *w_up_gate,
                                   const void *w_down, const void *w_shared_up_gate,
                                   const void *w_shared_down, const uint8_t *pad_mask,
                                   const void *dout, int64_t T, int32_t H, int32_t E, int32_t K,
                                   int32_t I, int32_t I_shared, int32_t dtype, void *dh,
                                   void *dnorm_weight, float *dw_router, void *dw_up_gate,
                                   void *dw_down, void *dw_shared_up_gate, void *dw_shared_down,
                                   void *workspace, size_t workspace_bytes, void *hip_stream) {
  if (!norm_weight && T > 0) return HI3_E_NULL;
  return backward_impl(h, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask,
                       dout, T, H, E, K, I, I_shared, dtype, dh, dw_router, dw_up_gate, dw_down,
                       dw_shared_up_gate, dw_shared_down, workspace, workspace_bytes, hip_stream,
                       nullptr, false, norm_weight, eps, dnorm_weight);
}

const char *hi3_moe_backward_stage_name(int stage) {
  static const char *names[HI3_NUM_BWD_STAGES] = {
      "router", "dispatch", "gather_bwd", "gemm_dgrad_down", "gemm_up_gate_recompute",
      "gemm_dgrad_up_gate", "combine_bwd", "dw_router", "gemm_wgrad_down",
      "gemm_wgrad_up_gate"};
  if (stage < 0 || stage >= HI3_NUM_BWD_STAGES) return "?";
  return names[stage];
}

const char *hi3_moe_stage_name(int stage) {
  static const char *names[HI3_NUM_STAGES] = {
      "router", "dispatch", "gemm_up_gate_swiglu", "gemm_down", "combine"};
  if (stage < 0 || stage >= HI3_NUM_STAGES) return "?";
  return names[stage];
}

const char *hi3_moe_status_string(int status) {
  switch (status) {
    case HI3_OK: return "ok";
    case HI3_E_NULL: return "a required pointer is NULL";
    case HI3_E_SHAPE: return "invalid sizes (T < 0, a size <= 0, or K > E)";
    case HI3_E_UNSUPPORTED:
      return "unsupported (dtype, E > 64, H/I/I_shared not a multiple of 64, T*K >= 2^31, "
             "or a pointer not 16-byte aligned)";
    case HI3_E_WORKSPACE: return "workspace smaller than hi3_moe_workspace_size";
    case HI3_E_HIP: return "a HIP launch failed";
    case HI3_E_SCRATCH:
      return "the sizes need more scratch than hi3_moe_forward_noalloc holds "
             "(HI3_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
