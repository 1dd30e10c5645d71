"""Python binding of libhi3moe.so, the MI355X (gfx950) routed-expert MoE
feed-forward layer of the HunyuanImage-3.0 decoder.

The functions carry the names of the C entry points in include/hi3_moe.h and
only marshal arguments: sizes are read from tensor shapes, pointers from
tensors, the stream from torch's current stream. Every step of the layer runs
in the library's HIP kernels; torch provides device memory and streams. There
is no fallback: importing this package fails if the library is not built.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhi3moe.so")

HI3_F32 = 0
HI3_BF16 = 1
HI3_OK = 0
HI3_E_NULL = -1
HI3_E_SHAPE = -2
HI3_E_UNSUPPORTED = -3
HI3_E_WORKSPACE = -4
HI3_E_HIP = -5
HI3_E_SCRATCH = -6
HI3_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024
HI3_NUM_STAGES = 5
HI3_NUM_BWD_STAGES = 10

EXPORTED = (
    "hi3_moe_workspace_size",
    "hi3_moe_route",
    "hi3_moe_dispatch",
    "hi3_moe_forward",
    "hi3_moe_forward_overlap",
    "hi3_moe_forward_noalloc",
    "hi3_moe_forward_instrumented",
    "hi3_moe_forward_shared_on_side",
    "hi3_moe_rmsnorm",
    "hi3_moe_forward_norm_residual",
    "hi3_moe_backward_workspace_size",
    "hi3_moe_backward",
    "hi3_moe_backward_instrumented",
    "hi3_moe_backward_stage_name",
    "hi3_moe_forward_train",
    "hi3_moe_backward_after_forward",
    "hi3_moe_backward_norm_residual",
    "hi3_moe_stage_name",
    "hi3_moe_status_string",
    "hi3_moe_probe_mfma_bf16",
)


class Hi3Error(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(f"hi3_moe status {status}: {hi3_moe_status_string(status)}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: run `python moe_decoder_ffn_amd/build.py` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.hi3_moe_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32, i32]
    lib.hi3_moe_workspace_size.restype = sz
    lib.hi3_moe_route.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, sz, P]
    lib.hi3_moe_route.restype = ctypes.c_int
    lib.hi3_moe_dispatch.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    lib.hi3_moe_dispatch.restype = ctypes.c_int
    fwd = [P, P, P, P, P, P, P, i64, i32, i32, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    lib.hi3_moe_forward.argtypes = fwd
    lib.hi3_moe_forward.restype = ctypes.c_int
    lib.hi3_moe_forward_noalloc.argtypes = fwd[:18] + [P]
    lib.hi3_moe_forward_noalloc.restype = ctypes.c_int
    lib.hi3_moe_forward_overlap.argtypes = fwd + [P]
    lib.hi3_moe_forward_overlap.restype = ctypes.c_int
    lib.hi3_moe_forward_instrumented.argtypes = fwd + [P, P]
    lib.hi3_moe_forward_instrumented.restype = ctypes.c_int
    lib.hi3_moe_forward_shared_on_side.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32]
    lib.hi3_moe_forward_shared_on_side.restype = ctypes.c_int
    f32 = ctypes.c_float
    lib.hi3_moe_rmsnorm.argtypes = [P, P, f32, P, i64, i32, i32, P, P]
    lib.hi3_moe_rmsnorm.restype = ctypes.c_int
    lib.hi3_moe_forward_norm_residual.argtypes = [P, P, f32] + fwd[1:]
    lib.hi3_moe_forward_norm_residual.restype = ctypes.c_int
    lib.hi3_moe_backward_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32, i32]
    lib.hi3_moe_backward_workspace_size.restype = sz
    bwd = [P, P, P, P, P, P, P, P, i64, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, sz, P]
    lib.hi3_moe_backward.argtypes = bwd
    lib.hi3_moe_backward.restype = ctypes.c_int
    lib.hi3_moe_backward_instrumented.argtypes = bwd + [P]
    lib.hi3_moe_backward_instrumented.restype = ctypes.c_int
    lib.hi3_moe_backward_norm_residual.argtypes = [P, P, f32] + bwd[1:15] + [P, P] + bwd[16:]
    lib.hi3_moe_backward_norm_residual.restype = ctypes.c_int
    lib.hi3_moe_forward_train.argtypes = fwd
    lib.hi3_moe_forward_train.restype = ctypes.c_int
    lib.hi3_moe_backward_after_forward.argtypes = bwd
    lib.hi3_moe_backward_after_forward.restype = ctypes.c_int
    lib.hi3_moe_backward_stage_name.argtypes = [ctypes.c_int]
    lib.hi3_moe_backward_stage_name.restype = ctypes.c_char_p
    lib.hi3_moe_stage_name.argtypes = [ctypes.c_int]
    lib.hi3_moe_stage_name.restype = ctypes.c_char_p
    lib.hi3_moe_probe_mfma_bf16.argtypes = [P, P, i32, i32, P]
    lib.hi3_moe_probe_mfma_bf16.restype = i64
    lib.hi3_moe_status_string.argtypes = [ctypes.c_int]
    lib.hi3_moe_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


# ---------------------------------------------------------------- marshalling

def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to hi3_moe must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _side(stream):
    """A side stream argument: None stays NULL (no side stream)."""
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return HI3_BF16
    if dt == torch.float32:
        return HI3_F32
    raise TypeError(f"unsupported dtype {dt}")


def _check(status):
    if status != HI3_OK:
        raise Hi3Error(status)


# ---------------------------------------------------------------- entry points

def hi3_moe_workspace_size(T, H, E, K, I, I_shared, dtype) -> int:
    return int(lib.hi3_moe_workspace_size(T, H, E, K, I, I_shared, dtype))


def hi3_moe_route(x, w_router, pad_mask, K, topk_idx, topk_w, expert_counts, workspace,
                  stream=None):
    T, H = x.shape
    E = w_router.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hi3_moe_route(_ptr(x), _ptr(w_router), _ptr(pad_mask), T, H, E, K,
                             dtype_code(x.dtype), _ptr(topk_idx), _ptr(topk_w),
                             _ptr(expert_counts), _ptr(workspace), ws_bytes, _stream(stream)))


def hi3_moe_dispatch(topk_idx, pad_mask, x, E, expert_offsets, perm_token, slot_of,
                     x_sorted, workspace, stream=None):
    T, K = topk_idx.shape
    H = x.shape[1]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hi3_moe_dispatch(_ptr(topk_idx), _ptr(pad_mask), _ptr(x), T, H, E, K,
                                dtype_code(x.dtype), _ptr(expert_offsets), _ptr(perm_token),
                                _ptr(slot_of), _ptr(x_sorted), _ptr(workspace), ws_bytes,
                                _stream(stream)))


def _forward_args(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                  pad_mask, K, out, topk_idx, topk_w, expert_counts, workspace, stream):
    T, H = x.shape
    E = w_router.shape[0]
    I = w_up_gate.shape[1] // 2
    Is = w_shared_up_gate.shape[0] // 2
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (_ptr(x), _ptr(w_router), _ptr(w_up_gate), _ptr(w_down), _ptr(w_shared_up_gate),
            _ptr(w_shared_down), _ptr(pad_mask), T, H, E, K, I, Is, dtype_code(x.dtype),
            _ptr(out), _ptr(topk_idx), _ptr(topk_w), _ptr(expert_counts), _ptr(workspace),
            ws_bytes, _stream(stream))


def hi3_moe_forward(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                    pad_mask, K, out, topk_idx=None, topk_w=None, expert_counts=None,
                    workspace=None, stream=None):
    _check(lib.hi3_moe_forward(*_forward_args(
        x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask, K, out,
        topk_idx, topk_w, expert_counts, workspace, stream)))


def hi3_moe_forward_overlap(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                            pad_mask, K, out, topk_idx=None, topk_w=None, expert_counts=None,
                            workspace=None, side_stream=None, stream=None):
    """side_stream: a second stream (torch.cuda.Stream, raw handle, or None)
    on which the shared expert may run alongside the routing."""
    _check(lib.hi3_moe_forward_overlap(*_forward_args(
        x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask, K, out,
        topk_idx, topk_w, expert_counts, workspace, stream), _side(side_stream)))


def hi3_moe_forward_noalloc(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                            pad_mask, K, out, topk_idx=None, topk_w=None, expert_counts=None,
                            stream=None):
    """hi3_moe_forward on the library's own scratch (no workspace argument)."""
    a = _forward_args(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                      pad_mask, K, out, topk_idx, topk_w, expert_counts, None, stream)
    # drop the workspace pointer and size
    _check(lib.hi3_moe_forward_noalloc(*a[:18], a[20]))


def hi3_moe_forward_instrumented(x, w_router, w_up_gate, w_down, w_shared_up_gate,
                                 w_shared_down, pad_mask, K, out, topk_idx, topk_w,
                                 expert_counts, workspace, stage_events, stream=None,
                                 side_stream=None):
    """stage_events: sequence of HI3_NUM_STAGES + 1 raw hipEvent_t handles (ints);
    side_stream as for hi3_moe_forward_overlap (None: one stream)."""
    arr = (ctypes.c_void_p * len(stage_events))(*stage_events)
    _check(lib.hi3_moe_forward_instrumented(*_forward_args(
        x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask, K, out,
        topk_idx, topk_w, expert_counts, workspace, stream), _side(side_stream), arr))


def hi3_moe_forward_shared_on_side(T, H, E, K, I, I_shared, dtype, has_pad_mask) -> bool:
    return bool(lib.hi3_moe_forward_shared_on_side(T, H, E, K, I, I_shared, dtype,
                                                   1 if has_pad_mask else 0))


def hi3_moe_rmsnorm(x, weight, eps, pad_mask, xn, stream=None):
    T, H = x.shape
    _check(lib.hi3_moe_rmsnorm(_ptr(x), _ptr(weight), float(eps), _ptr(pad_mask), T, H,
                               dtype_code(x.dtype), _ptr(xn), _stream(stream)))


def hi3_moe_forward_norm_residual(h, norm_weight, eps, w_router, w_up_gate, w_down,
                                  w_shared_up_gate, w_shared_down, pad_mask, K, out,
                                  topk_idx=None, topk_w=None, expert_counts=None,
                                  workspace=None, stream=None):
    args = _forward_args(h, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                         pad_mask, K, out, topk_idx, topk_w, expert_counts, workspace, stream)
    _check(lib.hi3_moe_forward_norm_residual(args[0], _ptr(norm_weight), float(eps),
                                             *args[1:]))


def hi3_moe_backward_workspace_size(T, H, E, K, I, I_shared, dtype) -> int:
    return int(lib.hi3_moe_backward_workspace_size(T, H, E, K, I, I_shared, dtype))


def _backward_args(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask,
                   dout, K, dx, dw_router, dw_up_gate, dw_down, dw_shared_up_gate,
                   dw_shared_down, workspace, stream):
    T, H = x.shape
    E = w_router.shape[0]
    I = w_up_gate.shape[1] // 2
    Is = w_shared_up_gate.shape[0] // 2
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (_ptr(x), _ptr(w_router), _ptr(w_up_gate), _ptr(w_down), _ptr(w_shared_up_gate),
            _ptr(w_shared_down), _ptr(pad_mask), _ptr(dout), T, H, E, K, I, Is,
            dtype_code(x.dtype), _ptr(dx), _ptr(dw_router), _ptr(dw_up_gate), _ptr(dw_down),
            _ptr(dw_shared_up_gate), _ptr(dw_shared_down), _ptr(workspace), ws_bytes,
            _stream(stream))


def hi3_moe_backward(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                     pad_mask, dout, K, dx, dw_router, dw_up_gate, dw_down, dw_shared_up_gate,
                     dw_shared_down, workspace, stream=None):
    _check(lib.hi3_moe_backward(*_backward_args(
        x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask, dout, K, dx,
        dw_router, dw_up_gate, dw_down, dw_shared_up_gate, dw_shared_down, workspace, stream)))


def hi3_moe_backward_instrumented(x, w_router, w_up_gate, w_down, w_shared_up_gate,
                                  w_shared_down, pad_mask, dout, K, dx, dw_router, dw_up_gate,
                                  dw_down, dw_shared_up_gate, dw_shared_down, workspace,
                                  stage_events, stream=None):
    """stage_events: sequence of HI3_NUM_BWD_STAGES + 1 raw hipEvent_t handles."""
    arr = (ctypes.c_void_p * len(stage_events))(*stage_events)
    _check(lib.hi3_moe_backward_instrumented(*_backward_args(
        x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask, dout, K, dx,
        dw_router, dw_up_gate, dw_down, dw_shared_up_gate, dw_shared_down, workspace, stream),
        arr))


def hi3_moe_forward_train(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                          pad_mask, K, out, topk_idx=None, topk_w=None, expert_counts=None,
                          workspace=None, stream=None):
    _check(lib.hi3_moe_forward_train(*_forward_args(
        x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask, K, out,
        topk_idx, topk_w, expert_counts, workspace, stream)))


def hi3_moe_backward_after_forward(x, w_router, w_up_gate, w_down, w_shared_up_gate,
                                   w_shared_down, pad_mask, dout, K, dx, dw_router, dw_up_gate,
                                   dw_down, dw_shared_up_gate, dw_shared_down, workspace,
                                   stream=None):
    _check(lib.hi3_moe_backward_after_forward(*_backward_args(
        x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask, dout, K, dx,
        dw_router, dw_up_gate, dw_down, dw_shared_up_gate, dw_shared_down, workspace, stream)))


def hi3_moe_backward_norm_residual(h, norm_weight, eps, w_router, w_up_gate, w_down,
                                   w_shared_up_gate, w_shared_down, pad_mask, dout, K, dh,
                                   dnorm_weight, dw_router, dw_up_gate, dw_down,
                                   dw_shared_up_gate, dw_shared_down, workspace, stream=None):
    a = _backward_args(h, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask,
                       dout, K, dh, dw_router, dw_up_gate, dw_down, dw_shared_up_gate,
                       dw_shared_down, workspace, stream)
    # a: (x, w_router, ..., dtype, dx, dw_router, ...): insert the norm weight
    # and eps after h, and dnorm_weight after dh
    _check(lib.hi3_moe_backward_norm_residual(a[0], _ptr(norm_weight), float(eps), *a[1:16],
                                              _ptr(dnorm_weight), *a[16:]))


def hi3_moe_backward_stage_name(i) -> str:
    return lib.hi3_moe_backward_stage_name(i).decode()


def hi3_moe_stage_name(i) -> str:
    return lib.hi3_moe_stage_name(i).decode()


def hi3_moe_probe_mfma_bf16(operands, out, blocks, iters, stream=None) -> int:
    """Enqueues the matrix-core probe; returns the FLOP of the launch."""
    r = int(lib.hi3_moe_probe_mfma_bf16(_ptr(operands), _ptr(out), blocks, iters,
                                        _stream(stream)))
    if r < 0:
        raise Hi3Error(r)
    return r


def hi3_moe_status_string(status) -> str:
    return lib.hi3_moe_status_string(status).decode()


# ---------------------------------------------------------------- convenience

def workspace_for(x, E, K, I=0, I_shared=0):
    """A device workspace (uint8) of the size hi3_moe_workspace_size asks for."""
    T, H = x.shape
    n = hi3_moe_workspace_size(T, H, E, K, I, I_shared, dtype_code(x.dtype))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)


def moe_forward(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, K,
                pad_mask=None, out=None, workspace=None, return_routes=False,
                side_stream=None):
    """Allocates the outputs and the workspace with torch, then calls
    hi3_moe_forward (hi3_moe_forward_overlap when side_stream is given).
    Padding rows of a freshly allocated out are zero."""
    T, H = x.shape
    E = w_router.shape[0]
    I = w_up_gate.shape[1] // 2
    Is = w_shared_up_gate.shape[0] // 2
    if out is None:
        out = torch.zeros_like(x)
    if workspace is None:
        workspace = workspace_for(x, E, K, I, Is)
    idx = torch.empty((T, K), dtype=torch.int32, device=x.device)
    w = torch.empty((T, K), dtype=torch.float32, device=x.device)
    counts = torch.empty((E,), dtype=torch.int32, device=x.device)
    if side_stream is None:
        hi3_moe_forward(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                        pad_mask, K, out, idx, w, counts, workspace)
    else:
        hi3_moe_forward_overlap(x, w_router, w_up_gate, w_down, w_shared_up_gate,
                                w_shared_down, pad_mask, K, out, idx, w, counts, workspace,
                                side_stream)
    if return_routes:
        return out, idx, w, counts
    return out


def moe_forward_norm_residual(h, norm_weight, w_router, w_up_gate, w_down, w_shared_up_gate,
                              w_shared_down, K, eps=1e-5, pad_mask=None, out=None,
                              workspace=None, return_routes=False):
    """h + layer(RMSNorm(h)) with torch-allocated outputs and workspace; out
    may be h itself. Padding rows of a freshly allocated out are zero."""
    T, H = h.shape
    E = w_router.shape[0]
    I = w_up_gate.shape[1] // 2
    Is = w_shared_up_gate.shape[0] // 2
    if out is None:
        out = torch.zeros_like(h)
    if workspace is None:
        workspace = workspace_for(h, E, K, I, Is)
    idx = torch.empty((T, K), dtype=torch.int32, device=h.device)
    w = torch.empty((T, K), dtype=torch.float32, device=h.device)
    counts = torch.empty((E,), dtype=torch.int32, device=h.device)
    hi3_moe_forward_norm_residual(h, norm_weight, eps, w_router, w_up_gate, w_down,
                                  w_shared_up_gate, w_shared_down, pad_mask, K, out, idx, w,
                                  counts, workspace)
    if return_routes:
        return out, idx, w, counts
    return out


def moe_backward_norm_residual(h, norm_weight, w_router, w_up_gate, w_down, w_shared_up_gate,
                               w_shared_down, dout, K, eps=1e-5, pad_mask=None, workspace=None):
    """All gradients of the block entry point with torch-allocated outputs:
    dict(dh, dnorm_weight, dw_router, dw_up_gate, dw_down, dw_shared_up_gate,
    dw_shared_down); padding rows of dh are zero."""
    T, H = h.shape
    E = w_router.shape[0]
    I = w_up_gate.shape[1] // 2
    Is = w_shared_up_gate.shape[0] // 2
    dev, dt = h.device, h.dtype
    g = {"dh": torch.zeros_like(h), "dnorm_weight": torch.empty_like(norm_weight),
         "dw_router": torch.empty((E, H), dtype=torch.float32, device=dev),
         "dw_up_gate": torch.empty_like(w_up_gate), "dw_down": torch.empty_like(w_down),
         "dw_shared_up_gate": torch.empty_like(w_shared_up_gate),
         "dw_shared_down": torch.empty_like(w_shared_down)}
    if workspace is None:
        n = hi3_moe_backward_workspace_size(T, H, E, K, I, Is, dtype_code(dt))
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    hi3_moe_backward_norm_residual(h, norm_weight, eps, w_router, w_up_gate, w_down,
                                   w_shared_up_gate, w_shared_down, pad_mask, dout, K, g["dh"],
                                   g["dnorm_weight"], g["dw_router"], g["dw_up_gate"],
                                   g["dw_down"], g["dw_shared_up_gate"], g["dw_shared_down"],
                                   workspace)
    return g


def moe_backward(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, dout, K,
                 pad_mask=None, workspace=None,
                 want=("dx", "dw_router", "dw_up_gate", "dw_down", "dw_shared_up_gate",
                       "dw_shared_down")):
    """Allocates the requested gradients and the workspace with torch, then
    calls hi3_moe_backward. Returns a dict of the requested gradients
    (padding rows of dx are zero)."""
    T, H = x.shape
    E = w_router.shape[0]
    I = w_up_gate.shape[1] // 2
    Is = w_shared_up_gate.shape[0] // 2
    dev, dt = x.device, x.dtype
    shapes = {"dx": ((T, H), dt), "dw_router": ((E, H), torch.float32),
              "dw_up_gate": ((E, 2 * I, H), dt), "dw_down": ((E, H, I), dt),
              "dw_shared_up_gate": ((2 * Is, H), dt), "dw_shared_down": ((H, Is), dt)}
    outs = {k: (torch.zeros(sh, dtype=d, device=dev) if k == "dx" else
                torch.empty(sh, dtype=d, device=dev)) if k in want else None
            for k, (sh, d) in shapes.items()}
    if workspace is None:
        n = hi3_moe_backward_workspace_size(T, H, E, K, I, Is, dtype_code(dt))
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    hi3_moe_backward(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask,
                     dout, K, outs["dx"], outs["dw_router"], outs["dw_up_gate"], outs["dw_down"],
                     outs["dw_shared_up_gate"], outs["dw_shared_down"], workspace)
    return {k: v for k, v in outs.items() if v is not None}


class MoEFunction(torch.autograd.Function):
    """The layer as an autograd function: forward runs hi3_moe_forward_train,
    backward runs hi3_moe_backward_after_forward on the workspace the forward
    filled (kept on the context between the two). Gradients: x, the router
    weight (fp32), and the four expert weights; pad_mask and K get none.
    Inputs must not change between forward and backward (as for any saved
    tensor)."""

    @staticmethod
    def forward(ctx, x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, K,
                pad_mask=None):
        T, H = x.shape
        E = w_router.shape[0]
        I = w_up_gate.shape[1] // 2
        Is = w_shared_up_gate.shape[0] // 2
        n = hi3_moe_backward_workspace_size(T, H, E, K, I, Is, dtype_code(x.dtype))
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
        out = torch.zeros_like(x)
        hi3_moe_forward_train(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                              pad_mask, K, out, workspace=ws)
        ctx.save_for_backward(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                              pad_mask)
        ctx.ws, ctx.K = ws, K
        return out

    @staticmethod
    def backward(ctx, dout):
        x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, pad_mask = \
            ctx.saved_tensors
        dout = dout.contiguous()
        need = ctx.needs_input_grad
        g = [torch.zeros_like(x) if need[0] else None]
        for i, wt in ((1, w_router), (2, w_up_gate), (3, w_down), (4, w_shared_up_gate),
                      (5, w_shared_down)):
            g.append(torch.empty_like(wt) if need[i] else None)
        hi3_moe_backward_after_forward(x, w_router, w_up_gate, w_down, w_shared_up_gate,
                                       w_shared_down, pad_mask, dout, ctx.K, *g, ctx.ws)
        ctx.ws = None
        return (*g, None, None)


def moe_layer(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, K,
              pad_mask=None):
    """Differentiable layer output (MoEFunction.apply)."""
    return MoEFunction.apply(x, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down,
                             K, pad_mask)


class MoENormResidualFunction(torch.autograd.Function):
    """The block entry point (h + layer(RMSNorm(h))) as an autograd function:
    forward runs hi3_moe_forward_norm_residual, backward
    hi3_moe_backward_norm_residual (which recomputes the forward's routes and
    activations). Gradients: h, the norm weight, the router weight and the
    four expert weights."""

    @staticmethod
    def forward(ctx, h, norm_weight, w_router, w_up_gate, w_down, w_shared_up_gate,
                w_shared_down, K, eps=1e-5, pad_mask=None):
        out = moe_forward_norm_residual(h, norm_weight, w_router, w_up_gate, w_down,
                                        w_shared_up_gate, w_shared_down, K, eps=eps,
                                        pad_mask=pad_mask)
        ctx.save_for_backward(h, norm_weight, w_router, w_up_gate, w_down, w_shared_up_gate,
                              w_shared_down, pad_mask)
        ctx.K, ctx.eps = K, eps
        return out

    @staticmethod
    def backward(ctx, dout):
        h, nw, wr, w13, w2, ws13, ws2, pad_mask = ctx.saved_tensors
        need = ctx.needs_input_grad
        T, H = h.shape
        E, I, Is = wr.shape[0], w13.shape[1] // 2, ws13.shape[0] // 2
        g = [torch.zeros_like(h) if need[0] else None]
        for i, t in ((1, nw), (2, wr), (3, w13), (4, w2), (5, ws13), (6, ws2)):
            g.append(torch.empty_like(t) if need[i] else None)
        n = hi3_moe_backward_workspace_size(T, H, E, ctx.K, I, Is, dtype_code(h.dtype))
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=h.device)
        hi3_moe_backward_norm_residual(h, nw, ctx.eps, wr, w13, w2, ws13, ws2, pad_mask,
                                       dout.contiguous(), ctx.K, g[0], g[1], *g[2:], ws)
        return (*g, None, None, None)


def moe_block(h, norm_weight, w_router, w_up_gate, w_down, w_shared_up_gate, w_shared_down, K,
              eps=1e-5, pad_mask=None):
    """Differentiable block output h + layer(RMSNorm(h)) (MoENormResidualFunction)."""
    return MoENormResidualFunction.apply(h, norm_weight, w_router, w_up_gate, w_down,
                                         w_shared_up_gate, w_shared_down, K, eps, pad_mask)
