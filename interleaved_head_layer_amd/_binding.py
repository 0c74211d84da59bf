"""ctypes binding of libiha.so (C ABI in include/iha.h).  Argument marshalling only:
every step of the forward pass runs in the library's HIP kernels.  PyTorch supplies
device memory and the current stream.  There is no fallback: without the built
library every call raises."""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libiha.so")

IHA_OK = 0
STATUS_NAMES = ["IHA_OK", "IHA_ERR_INVALID_ARG", "IHA_ERR_SHAPE", "IHA_ERR_EMPTY_ROW",
                "IHA_ERR_NONFINITE", "IHA_ERR_WORKSPACE", "IHA_ERR_UNSUPPORTED", "IHA_ERR_DEVICE",
                "IHA_ERR_RANGE"]
IHA_MASK_NONE, IHA_MASK_CAUSAL, IHA_MASK_WINDOW = 0, 1, 2
IHA_F32, IHA_BF16 = 0, 1
IHA_FLAG_CHECK = 1
IHA_FLAG_FUSED_COLLAPSE = 2   # collapse in the attention epilogue (fp32 atomics); for measurement
IHA_PLAN_MIX_FUSED = 1
TIMED_EVENTS = 7       # IHA_TIMED_EVENTS in include/iha.h
STATIC_WORKSPACE_BYTES = 64 << 20   # IHA_STATIC_WORKSPACE_BYTES in include/iha.h
_MASKS = {"none": IHA_MASK_NONE, "causal": IHA_MASK_CAUSAL, "window": IHA_MASK_WINDOW}


class IHAError(RuntimeError):
    def __init__(self, status: int, where: str = "iha"):
        self.status = status
        super().__init__(f"{where}: {iha_status_str(status)}")


class iha_problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("N", ctypes.c_int64), ("D", ctypes.c_int64),
                ("H", ctypes.c_int64), ("P", ctypes.c_int64), ("window", ctypes.c_int64),
                ("mask", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


_lib = None


def iha_attention_backward(Q, K, V, dO, mask_mode, window: Optional[int] = None,
                           score_scale: Optional[float] = None, workspace=None):
    """Gradients of the attention step on stacked tensors: Q, K, V, dO fp16 [B, L, H, d]
    (V row-major).  Returns (dQ, dK, dV), fp32 [B, L, H, d].  score_scale defaults to
    log2(e)/sqrt(d)."""
    import torch
    B, L, H, d = (int(s) for s in Q.shape)
    mask = _mask_code(mask_mode)
    if window is None:
        window = 0
    if score_scale is None:
        score_scale = math.log2(math.e) / math.sqrt(d)
    ptrs = [_dev_ptr(t, n, torch.float16, (B, L, H, d)) for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (dO, "dO"))]
    lib = load_library()
    nbytes = ctypes.c_size_t(0)
    st = lib.iha_attention_backward_workspace(B, L, H, d, ctypes.byref(nbytes))
    if st != IHA_OK:
        raise IHAError(st, "iha_attention_backward_workspace")
    if workspace is None:
        workspace = torch.empty(max(int(nbytes.value), 1), dtype=torch.uint8, device=Q.device)
    grads = [torch.empty((B, L, H, d), dtype=torch.float32, device=Q.device) for _ in range(3)]
    stream = ctypes.c_void_p(torch.cuda.current_stream(Q.device).cuda_stream)
    st = lib.iha_attention_backward(B, L, H, d, mask, int(window), float(score_scale), *ptrs,
                                    *[ctypes.c_void_p(g.data_ptr()) for g in grads],
                                    ctypes.c_void_p(workspace.data_ptr()), int(workspace.numel()), stream)
    if st != IHA_OK:
        raise IHAError(st, "iha_attention_backward")
    return tuple(grads)


def load_library() -> ctypes.CDLL:
    """Load libiha.so (built in-tree by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                              "(run __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
        P = ctypes.POINTER(iha_problem)
        lib.iha_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        lib.iha_workspace_bytes.restype = ctypes.c_int
        fwd = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.iha_plan.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
        lib.iha_plan.restype = ctypes.c_int
        lib.iha_forward.argtypes = fwd
        lib.iha_forward.restype = ctypes.c_int
        lib.iha_forward_timed.argtypes = fwd + [ctypes.POINTER(vp)]
        lib.iha_forward_timed.restype = ctypes.c_int
        lib.iha_forward_static.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.iha_forward_static.restype = ctypes.c_int
        lib.iha_attention.argtypes = [i64, i64, i64, i64, i32, i64, ctypes.c_float, vp, vp, vp, vp,
                                      u32, vp, vp]
        lib.iha_attention.restype = ctypes.c_int
        lib.iha_nexus_inner_workspace.argtypes = [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.iha_nexus_inner_workspace.restype = ctypes.c_int
        lib.iha_nexus_inner.argtypes = [i64, i64, i64, i64, i32, i64, ctypes.c_float, vp, vp, u32, vp,
                                        ctypes.c_size_t, vp]
        lib.iha_nexus_inner.restype = ctypes.c_int
        lib.iha_attention_backward_workspace.argtypes = [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
        lib.iha_attention_backward_workspace.restype = ctypes.c_int
        lib.iha_attention_backward.argtypes = [i64, i64, i64, i64, i32, i64, ctypes.c_float, vp, vp, vp, vp,
                                               vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.iha_attention_backward.restype = ctypes.c_int
        lib.iha_backward_workspace.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
        lib.iha_backward_workspace.restype = ctypes.c_int
        lib.iha_backward.argtypes = [P] + [vp] * 18 + [ctypes.c_size_t, vp]
        lib.iha_backward.restype = ctypes.c_int
        lib.iha_status_str.argtypes = [ctypes.c_int]
        lib.iha_status_str.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def iha_status_str(status: int) -> str:
    return load_library().iha_status_str(int(status)).decode()


def _mask_code(mask_mode) -> int:
    if isinstance(mask_mode, str):
        return _MASKS[mask_mode]
    return int(mask_mode)


def make_problem(B, N, D, H, P, mask_mode, window=None, dtype=IHA_BF16, flags=0) -> iha_problem:
    """Fill an iha_problem.  In window mode the default window is N // (2P) stacked
    positions (figure 1 of the IHA page)."""
    mask = _mask_code(mask_mode)
    if window is None:
        window = N // (2 * P) if mask == IHA_MASK_WINDOW else 0
    return iha_problem(B, N, D, H, P, window, mask, dtype, flags, 0)


def iha_workspace_bytes(prob: iha_problem) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().iha_workspace_bytes(ctypes.byref(prob), ctypes.byref(n))
    if st != IHA_OK:
        raise IHAError(st, "iha_workspace_bytes")
    return n.value


def iha_plan(prob: iha_problem) -> int:
    """IHA_PLAN_* bits: which kernel path iha_forward takes for `prob`."""
    n = ctypes.c_uint32(0)
    st = load_library().iha_plan(ctypes.byref(prob), ctypes.byref(n))
    if st != IHA_OK:
        raise IHAError(st, "iha_plan")
    return n.value


def _dev_ptr(t, name, dtype=None, shape: Optional[Sequence[int]] = None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def iha_forward(X, W_Q, W_K, W_V, alpha_Q, alpha_K, alpha_V, R, H: int, P: int, mask_mode,
                window: Optional[int] = None, flags: int = 0, out=None, workspace=None,
                events=None):
    """IHA forward (Algorithm 1).  X [B, N, D] bf16 or fp32 on the GPU; W_* [D, D] same dtype;
    alpha_* [H, H, P] and R [H, H*P] fp32.  Returns X~ [B, N, D] fp32.

    ``events``: optional list of TIMED_EVENTS (7) torch.cuda.Event(enable_timing=True),
    recorded on the current stream at: start, after the weight preparation, after the
    projection GEMMs, after the mixing (empty when the mixing runs in the GEMM), after the
    attention launch (which also computes the fp32 first rows), again right after it (kept
    for a stable count), after the collapse.  Each record adds a gap of about 10 us."""
    import torch
    if X.dim() != 3:
        raise ValueError("X must be [B, N, D]")
    B, N, D = (int(s) for s in X.shape)
    dtype = {torch.bfloat16: IHA_BF16, torch.float32: IHA_F32}.get(X.dtype)
    if dtype is None:
        raise TypeError("X must be bfloat16 or float32")
    prob = make_problem(B, N, D, int(H), int(P), mask_mode, window, dtype, flags)
    args = [_dev_ptr(X, "X")]
    for n, w in (("W_Q", W_Q), ("W_K", W_K), ("W_V", W_V)):
        args.append(_dev_ptr(w, n, X.dtype, (D, D)))
    for n, a in (("alpha_Q", alpha_Q), ("alpha_K", alpha_K), ("alpha_V", alpha_V)):
        args.append(_dev_ptr(a, n, torch.float32, (H, H, P)))
    args.append(_dev_ptr(R, "R", torch.float32, (H, H * P)))
    if out is None:
        out = torch.empty((B, N, D), dtype=torch.float32, device=X.device)
    args.append(_dev_ptr(out, "out", torch.float32, (B, N, D)))
    need = iha_workspace_bytes(prob)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    args += [_dev_ptr(workspace, "workspace", torch.uint8), ctypes.c_size_t(workspace.numel())]
    stream = ctypes.c_void_p(torch.cuda.current_stream(X.device).cuda_stream)
    lib = load_library()
    if events is None:
        st = lib.iha_forward(ctypes.byref(prob), *args, stream)
    else:
        if len(events) != TIMED_EVENTS:
            raise ValueError(f"events must hold {TIMED_EVENTS} torch.cuda.Event objects")
        for e in events:
            if e.cuda_event == 0:     # create the underlying event
                e.record()
        evs = (ctypes.c_void_p * TIMED_EVENTS)(*[e.cuda_event for e in events])
        st = lib.iha_forward_timed(ctypes.byref(prob), *args, stream, evs)
    if st != IHA_OK:
        raise IHAError(st, "iha_forward")
    return out


def iha_forward_static(X, W_Q, W_K, W_V, alpha_Q, alpha_K, alpha_V, R, H: int, P: int, mask_mode,
                       out, window: Optional[int] = None, flags: int = 0):
    """iha_forward with the library's static per-device workspace (iha_forward_static): no
    device memory is allocated, here or in the library; the caller supplies `out`
    ([B, N, D] fp32).  Problems needing more than STATIC_WORKSPACE_BYTES raise
    IHAError(IHA_ERR_WORKSPACE); calls that overlap on one device race."""
    import torch
    if X.dim() != 3:
        raise ValueError("X must be [B, N, D]")
    B, N, D = (int(s) for s in X.shape)
    dtype = {torch.bfloat16: IHA_BF16, torch.float32: IHA_F32}.get(X.dtype)
    if dtype is None:
        raise TypeError("X must be bfloat16 or float32")
    prob = make_problem(B, N, D, int(H), int(P), mask_mode, window, dtype, flags)
    args = [_dev_ptr(X, "X")]
    for n, w in (("W_Q", W_Q), ("W_K", W_K), ("W_V", W_V)):
        args.append(_dev_ptr(w, n, X.dtype, (D, D)))
    for n, a in (("alpha_Q", alpha_Q), ("alpha_K", alpha_K), ("alpha_V", alpha_V)):
        args.append(_dev_ptr(a, n, torch.float32, (H, H, P)))
    args.append(_dev_ptr(R, "R", torch.float32, (H, H * P)))
    args.append(_dev_ptr(out, "out", torch.float32, (B, N, D)))
    stream = ctypes.c_void_p(torch.cuda.current_stream(X.device).cuda_stream)
    st = load_library().iha_forward_static(ctypes.byref(prob), *args, stream)
    if st != IHA_OK:
        raise IHAError(st, "iha_forward_static")
    return out


def iha_backward_workspace_bytes(prob: iha_problem) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().iha_backward_workspace(ctypes.byref(prob), ctypes.byref(n))
    if st != IHA_OK:
        raise IHAError(st, "iha_backward_workspace")
    return n.value


def iha_backward(X, W_Q, W_K, W_V, alpha_Q, alpha_K, alpha_V, R, G, H: int, P: int, mask_mode,
                 window: Optional[int] = None, flags: int = 0, workspace=None):
    """Gradients of the IHA layer for the loss sum(G * X~) (iha_backward): X [B, N, D] and
    W_* [D, D] bf16, alpha_* [H, H, P], R [H, H*P] and G [B, N, D] fp32, all on the GPU.
    Returns a dict of fp32 tensors {"X", "WQ", "WK", "WV", "aQ", "aK", "aV", "R"}."""
    import torch
    if X.dim() != 3 or X.dtype != torch.bfloat16:
        raise TypeError("X must be a bfloat16 [B, N, D] tensor")
    B, N, D = (int(s) for s in X.shape)
    H, P = int(H), int(P)
    prob = make_problem(B, N, D, H, P, mask_mode, window, IHA_BF16, flags)
    args = [_dev_ptr(X, "X")]
    for n, w in (("W_Q", W_Q), ("W_K", W_K), ("W_V", W_V)):
        args.append(_dev_ptr(w, n, torch.bfloat16, (D, D)))
    for n, a in (("alpha_Q", alpha_Q), ("alpha_K", alpha_K), ("alpha_V", alpha_V)):
        args.append(_dev_ptr(a, n, torch.float32, (H, H, P)))
    args.append(_dev_ptr(R, "R", torch.float32, (H, H * P)))
    args.append(_dev_ptr(G, "G", torch.float32, (B, N, D)))
    dev = X.device
    shapes = {"X": (B, N, D), "WQ": (D, D), "WK": (D, D), "WV": (D, D), "aQ": (H, H, P),
              "aK": (H, H, P), "aV": (H, H, P), "R": (H, H * P)}
    grads = {k: torch.empty(v, dtype=torch.float32, device=dev) for k, v in shapes.items()}
    args += [ctypes.c_void_p(grads[k].data_ptr()) for k in shapes]
    need = iha_backward_workspace_bytes(prob)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    args += [_dev_ptr(workspace, "workspace", torch.uint8), ctypes.c_size_t(workspace.numel())]
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = load_library().iha_backward(ctypes.byref(prob), *args, stream)
    if st != IHA_OK:
        raise IHAError(st, "iha_backward")
    return grads


def iha_nexus_inner(Q, mask_mode="none", window: Optional[int] = None, score_scale: Optional[float] = None,
                    flags: int = 0, out=None, workspace=None):
    """Nexus inner attention softmax(Q Q^T / sqrt(d)) Q per head (keys and values are the
    queries): Q fp16 [B, L, H, d] -> fp32 [B, L, H, d].  score_scale defaults to
    log2(e)/sqrt(d) (base-2 scores)."""
    import torch
    B, L, H, d = (int(s) for s in Q.shape)
    mask = _mask_code(mask_mode)
    if window is None:
        window = 0
    if score_scale is None:
        score_scale = math.log2(math.e) / math.sqrt(d)
    q = _dev_ptr(Q, "Q", torch.float16, (B, L, H, d))
    lib = load_library()
    nbytes = ctypes.c_size_t(0)
    st = lib.iha_nexus_inner_workspace(B, L, H, d, ctypes.byref(nbytes))
    if st != IHA_OK:
        raise IHAError(st, "iha_nexus_inner_workspace")
    if workspace is None:
        workspace = torch.empty(int(nbytes.value), dtype=torch.uint8, device=Q.device)
    if out is None:
        out = torch.empty((B, L, H, d), dtype=torch.float32, device=Q.device)
    o = _dev_ptr(out, "out", torch.float32, (B, L, H, d))
    stream = ctypes.c_void_p(torch.cuda.current_stream(Q.device).cuda_stream)
    st = lib.iha_nexus_inner(B, L, H, d, mask, int(window), float(score_scale), q, o, flags,
                             ctypes.c_void_p(workspace.data_ptr()), int(workspace.numel()), stream)
    if st != IHA_OK:
        raise IHAError(st, "iha_nexus_inner")
    return out


def iha_attention(Q, K, Vt, mask_mode, window: Optional[int] = None,
                  score_scale: Optional[float] = None, flags: int = 0, out=None):
    """Attention step alone on stacked tensors: Q, K fp16 [B, L, H, d]; Vt fp16 [B, H, d, L].
    Returns O fp32 [B, L, H, d].  score_scale defaults to log2(e)/sqrt(d)."""
    import torch
    B, L, H, d = (int(s) for s in Q.shape)
    mask = _mask_code(mask_mode)
    if window is None:
        window = 0
    if score_scale is None:
        score_scale = math.log2(math.e) / math.sqrt(d)
    q = _dev_ptr(Q, "Q", torch.float16)
    k = _dev_ptr(K, "K", torch.float16, (B, L, H, d))
    v = _dev_ptr(Vt, "Vt", torch.float16, (B, H, d, L))
    if out is None:
        out = torch.empty((B, L, H, d), dtype=torch.float32, device=Q.device)
    o = _dev_ptr(out, "out", torch.float32, (B, L, H, d))
    flag = torch.zeros(64, dtype=torch.int32, device=Q.device) if flags else None
    stream = ctypes.c_void_p(torch.cuda.current_stream(Q.device).cuda_stream)
    st = load_library().iha_attention(B, L, H, d, mask, int(window), float(score_scale), q, k, v, o,
                                      flags, None if flag is None else ctypes.c_void_p(flag.data_ptr()),
                                      stream)
    if st != IHA_OK:
        raise IHAError(st, "iha_attention")
    return out
