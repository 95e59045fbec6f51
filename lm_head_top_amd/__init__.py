"""Fused chunked top-K KL distillation loss on AMD MI355X (gfx950).

A thin ctypes binding over ``libkdtopk.so`` (declared in ``include/kdtopk.h``).
Every step of the loss runs in the library's HIP kernels; this module only
marshals arguments.  PyTorch provides device memory and the current stream.

There is no fallback: if the library is missing, importing the entry points
raises, so nothing can silently run elsewhere.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "lib_path", "debug_lib_path", "load_library", "swap_library", "workspace_size", "forward", "forward_noalloc", "backward", "validate",
    "KDTopKKL", "profile_enable", "profile_read", "KERNELS", "KDError", "topk_select",
    "keep_workspace_size", "forward_keep", "backward_keep",
    "keep_logits_workspace_size", "forward_keep_logits", "backward_keep_logits",
    "dense_workspace_size", "dense_forward", "dense_backward", "forward_ex", "backward_ex",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libkdtopk.so"
_lib = None

KERNELS = {
    "teacher": 0, "logits_fwd": 1, "combine": 2, "finalize": 3,
    "logits_bwd": 4, "dh": 5, "dh_reduce": 6, "dw": 7, "bucket": 8, "topk_select": 9, "keep_grad": 10,
}

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported problem size",
           3: "workspace too small", 4: "HIP launch failed", 5: "cached id outside [0, V)",
           6: "device bounds check failed"}


class KDError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: str = ""):
        detail = f", {hip_error}" if hip_error else ""
        super().__init__(f"{what}: {_STATUS.get(status, 'unknown')} (status {status}{detail})")
        self.status = status
        self.hip_error = hip_error


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def debug_lib_path() -> str:
    """libkdtopk_debug.so: the same exports, with device-side bounds checks on
    the cache-entry scatters and gathers (built beside libkdtopk.so)."""
    return os.path.join(_HERE, "libkdtopk_debug.so")


def _open(path: str):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m lm_head_top_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    # The library finds libamdhip64 by soname.  Loading torch first makes it
    # bind to the HIP runtime torch has already loaded, so the device pointers
    # and streams torch hands over belong to the same runtime (loaded the other
    # way round, the process would hold two HIP runtimes).
    import torch  # noqa: F401
    return _configure(ctypes.CDLL(path))


def load_library():
    """Loads libkdtopk.so (built by ``python -m lm_head_top_amd.build``)."""
    global _lib
    if _lib is None:
        _lib = _open(lib_path())
    return _lib


def swap_library(lib):
    """Points the entry points at another build of the library: a path (say
    debug_lib_path()) or a handle an earlier call returned.  Returns the
    handle in use before, so a caller can switch back."""
    global _lib
    prev = load_library()
    _lib = _open(lib) if isinstance(lib, str) else lib
    return prev


def _configure(lib):
    c_i64, c_i32, c_f, c_vp, c_sz = (ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                                     ctypes.c_void_p, ctypes.c_size_t)
    lib.kd_topk_kl_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_i32, c_i64]
    lib.kd_topk_kl_workspace_size.restype = c_sz
    lib.kd_topk_kl_forward.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_f,
                                       c_i64, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
    lib.kd_topk_kl_forward.restype = ctypes.c_int
    lib.kd_topk_kl_forward_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_f,
                                               c_i64, c_vp, c_vp, c_vp, c_vp]
    lib.kd_topk_kl_forward_noalloc.restype = ctypes.c_int
    lib.kd_topk_kl_backward.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64,
                                        c_i32, c_f, c_i64, c_vp, c_vp, c_vp, c_sz, c_vp]
    lib.kd_topk_kl_backward.restype = ctypes.c_int
    lib.kd_topk_kl_forward_ex.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_f, c_i64,
                                          c_vp, c_vp, c_f, c_f, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
    lib.kd_topk_kl_forward_ex.restype = ctypes.c_int
    lib.kd_topk_kl_backward_ex.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32,
                                           c_f, c_i64, c_vp, c_vp, c_f, c_f, c_i32, c_vp, c_vp, c_vp, c_sz,
                                           c_vp]
    lib.kd_topk_kl_backward_ex.restype = ctypes.c_int
    lib.kd_topk_kl_validate.argtypes = [c_vp, c_i64, c_i32, c_i64, c_vp, c_vp]
    lib.kd_topk_kl_validate.restype = ctypes.c_int
    lib.kd_status_string.argtypes = [ctypes.c_int]
    lib.kd_status_string.restype = ctypes.c_char_p
    lib.kd_topk_kl_keep_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_i32, c_i64]
    lib.kd_topk_kl_keep_workspace_size.restype = c_sz
    lib.kd_topk_kl_forward_keep.argtypes = lib.kd_topk_kl_forward.argtypes
    lib.kd_topk_kl_forward_keep.restype = ctypes.c_int
    lib.kd_topk_kl_backward_keep.argtypes = [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_f, c_i64,
                                             c_vp, c_vp, c_vp, c_sz, c_vp]
    lib.kd_topk_kl_backward_keep.restype = ctypes.c_int
    lib.kd_topk_kl_keep_logits_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_i32, c_i64]
    lib.kd_topk_kl_keep_logits_workspace_size.restype = c_sz
    lib.kd_topk_kl_forward_keep_logits.argtypes = lib.kd_topk_kl_forward.argtypes
    lib.kd_topk_kl_forward_keep_logits.restype = ctypes.c_int
    lib.kd_topk_kl_backward_keep_logits.argtypes = lib.kd_topk_kl_backward.argtypes
    lib.kd_topk_kl_backward_keep_logits.restype = ctypes.c_int
    lib.kd_dense_kl_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_i64]
    lib.kd_dense_kl_workspace_size.restype = c_sz
    lib.kd_dense_kl_forward.argtypes = [c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i64, c_f, c_i64,
                                        c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
    lib.kd_dense_kl_forward.restype = ctypes.c_int
    lib.kd_dense_kl_backward.argtypes = [c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64,
                                         c_f, c_i64, c_vp, c_vp, c_vp, c_sz, c_vp]
    lib.kd_dense_kl_backward.restype = ctypes.c_int
    lib.kd_topk_select.argtypes = [c_vp, c_i32, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp]
    lib.kd_topk_select.restype = ctypes.c_int
    lib.kd_last_hip_error.argtypes = []
    lib.kd_last_hip_error.restype = ctypes.c_char_p
    lib.kd_profile_enable.argtypes = [ctypes.c_uint32]
    lib.kd_profile_enable.restype = ctypes.c_int
    lib.kd_profile_read.argtypes = [c_i32, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64)]
    lib.kd_profile_read.restype = ctypes.c_int
    return lib


def _check(status: int, what: str):
    if status != 0:
        hip = _lib.kd_last_hip_error().decode() if status == 4 and _lib is not None else ""
        raise KDError(status, what, hip)


def workspace_size(N: int, D: int, V: int, K: int, chunk: int) -> int:
    return int(load_library().kd_topk_kl_workspace_size(N, D, V, K, chunk))


def _torch():
    import torch
    return torch


def _stream_ptr(torch, device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev_tensor(torch, x, name, dtype, shape=None, device=None, numel=None):
    """Checks one pointer argument before anything is launched: a contiguous
    tensor of `dtype` on the GPU `device` (or any GPU when None), of exactly
    `shape` (a tuple) or `numel` elements.  Raises TypeError for a wrong type
    or dtype and ValueError for the rest."""
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {x.dtype})")
    if not x.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got one on {x.device})")
    if device is not None and x.device != device:
        raise ValueError(f"{name} is on {x.device}, the other arguments on {device}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(x.shape)})")
    if numel is not None and x.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements (got {x.numel()})")
    return x


def _check_inputs(torch, H, W, idx, t):
    for name, x in (("H", H), ("W", W), ("topk_idx", idx), ("topk_logit", t)):
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError(f"{name} must be a 2-D tensor")
    N, D = H.shape
    V = W.shape[0]
    K = idx.shape[1]
    dev = H.device
    _dev_tensor(torch, H, "H", torch.bfloat16, (N, D))
    _dev_tensor(torch, W, "W", torch.bfloat16, (V, D), dev)
    _dev_tensor(torch, idx, "topk_idx", torch.int32, (N, K), dev)
    _dev_tensor(torch, t, "topk_logit", torch.float32, (N, K), dev)
    return N, D, V, K


def _check_lse(torch, lse, N, dev, name="lse"):
    _dev_tensor(torch, lse, name, torch.float32, device=dev, numel=N)


def _check_grad_loss(torch, grad_loss, dev):
    if grad_loss is not None:
        _dev_tensor(torch, grad_loss, "grad_loss", torch.float32, device=dev, numel=1)


def _out_dW(torch, dW, V, D, dev):
    if dW is None:
        return torch.zeros((V, D), dtype=torch.float32, device=dev)
    return _dev_tensor(torch, dW, "dW", torch.float32, (V, D), dev)


def _given_workspace(torch, workspace, need, dev, name="workspace"):
    _dev_tensor(torch, workspace, name, torch.uint8, device=dev)
    if workspace.dim() != 1 or workspace.numel() < need:
        raise ValueError(f"{name} must be a 1-D uint8 tensor of at least {need} bytes "
                         f"(got {workspace.numel()})")
    return workspace


def _workspace(torch, N, D, V, K, chunk, device, workspace):
    need = workspace_size(N, D, V, K, chunk)
    if need == 0:
        raise KDError(1, "workspace_size")
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    return _given_workspace(torch, workspace, need, device)


def forward(H, W, topk_idx, topk_logit, T: float = 1.0, chunk: int = 1024,
            want_row_kl: bool = False, workspace=None):
    """Loss (device fp32 [1]), lse (fp32 [N]) and optionally row_kl (fp32 [N])."""
    torch = _torch()
    N, D, V, K = _check_inputs(torch, H, W, topk_idx, topk_logit)
    dev = H.device
    ws = _workspace(torch, N, D, V, K, chunk, dev, workspace)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    row_kl = torch.empty(N, dtype=torch.float32, device=dev) if want_row_kl else None
    st = load_library().kd_topk_kl_forward(
        _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit), N, D, V, K, float(T), int(chunk),
        _ptr(loss), _ptr(lse), _ptr(row_kl), _ptr(ws), ws.numel(), _stream_ptr(torch, dev))
    _check(st, "kd_topk_kl_forward")
    return (loss, lse, row_kl) if want_row_kl else (loss, lse)


def forward_noalloc(H, W, topk_idx, topk_logit, T: float = 1.0, chunk: int = 1024,
                    want_row_kl: bool = False, loss=None, lse=None, row_kl=None):
    """kd_topk_kl_forward_noalloc: the forward with the library's own device
    scratch instead of a workspace (the library allocates nothing).  Outputs
    may be passed in (loss fp32 [1], lse fp32 [N], row_kl fp32 [N]) so the
    call allocates nothing here either; missing ones are created."""
    torch = _torch()
    N, D, V, K = _check_inputs(torch, H, W, topk_idx, topk_logit)
    dev = H.device
    loss = torch.empty(1, dtype=torch.float32, device=dev) if loss is None else \
        _dev_tensor(torch, loss, "loss", torch.float32, device=dev, numel=1)
    lse = torch.empty(N, dtype=torch.float32, device=dev) if lse is None else \
        _dev_tensor(torch, lse, "lse", torch.float32, device=dev, numel=N)
    if want_row_kl and row_kl is None:
        row_kl = torch.empty(N, dtype=torch.float32, device=dev)
    elif row_kl is not None:
        _dev_tensor(torch, row_kl, "row_kl", torch.float32, device=dev, numel=N)
    st = load_library().kd_topk_kl_forward_noalloc(
        _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit), N, D, V, K, float(T), int(chunk),
        _ptr(loss), _ptr(lse), _ptr(row_kl), _stream_ptr(torch, dev))
    _check(st, "kd_topk_kl_forward_noalloc")
    return (loss, lse, row_kl) if row_kl is not None else (loss, lse)


def backward(H, W, topk_idx, topk_logit, lse, grad_loss=None, T: float = 1.0,
             chunk: int = 1024, dW=None, workspace=None):
    """dH (bf16 [N, D], overwritten) and dW (fp32 [V, D], accumulated; zeros if None)."""
    torch = _torch()
    N, D, V, K = _check_inputs(torch, H, W, topk_idx, topk_logit)
    dev = H.device
    _check_lse(torch, lse, N, dev)
    _check_grad_loss(torch, grad_loss, dev)
    dW = _out_dW(torch, dW, V, D, dev)
    ws = _workspace(torch, N, D, V, K, chunk, dev, workspace)
    dH = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    gl = grad_loss
    st = load_library().kd_topk_kl_backward(
        _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit), _ptr(lse), _ptr(gl), N, D, V, K,
        float(T), int(chunk), _ptr(dH), _ptr(dW), _ptr(ws), ws.numel(), _stream_ptr(torch, dev))
    _check(st, "kd_topk_kl_backward")
    return dH, dW


KD_SCALE_T2 = 1


def _ext_args(torch, N, row_weight, labels, dev):
    if row_weight is not None:
        _dev_tensor(torch, row_weight, "row_weight", torch.float32, device=dev, numel=N)
    if labels is not None:
        _dev_tensor(torch, labels, "labels", torch.int32, device=dev, numel=N)


def forward_ex(H, W, topk_idx, topk_logit, T: float = 1.0, chunk: int = 1024, row_weight=None,
               labels=None, kd_weight: float = 1.0, ce_weight: float = 0.0, scale_T2: bool = False,
               want_row_loss: bool = False, workspace=None):
    """Loss with the extensions: per-position weights, a hard-label
    cross-entropy term and T^2 scaling.  Returns loss, lse [, row_loss]."""
    torch = _torch()
    N, D, V, K = _check_inputs(torch, H, W, topk_idx, topk_logit)
    dev = H.device
    _ext_args(torch, N, row_weight, labels, dev)
    ws = _workspace(torch, N, D, V, K, chunk, dev, workspace)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    row_loss = torch.empty(N, dtype=torch.float32, device=dev) if want_row_loss else None
    st = load_library().kd_topk_kl_forward_ex(
        _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit), N, D, V, K, float(T), int(chunk),
        _ptr(row_weight), _ptr(labels), float(kd_weight), float(ce_weight),
        KD_SCALE_T2 if scale_T2 else 0, _ptr(loss), _ptr(lse), _ptr(row_loss), _ptr(ws), ws.numel(),
        _stream_ptr(torch, dev))
    _check(st, "kd_topk_kl_forward_ex")
    return (loss, lse, row_loss) if want_row_loss else (loss, lse)


def backward_ex(H, W, topk_idx, topk_logit, lse, grad_loss=None, T: float = 1.0, chunk: int = 1024,
                row_weight=None, labels=None, kd_weight: float = 1.0, ce_weight: float = 0.0,
                scale_T2: bool = False, dW=None, workspace=None):
    """dH (overwritten) and dW (accumulated) of the extended loss."""
    torch = _torch()
    N, D, V, K = _check_inputs(torch, H, W, topk_idx, topk_logit)
    dev = H.device
    _ext_args(torch, N, row_weight, labels, dev)
    _check_lse(torch, lse, N, dev)
    _check_grad_loss(torch, grad_loss, dev)
    dW = _out_dW(torch, dW, V, D, dev)
    ws = _workspace(torch, N, D, V, K, chunk, dev, workspace)
    dH = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    gl = grad_loss
    st = load_library().kd_topk_kl_backward_ex(
        _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit), _ptr(lse), _ptr(gl), N, D, V, K,
        float(T), int(chunk), _ptr(row_weight), _ptr(labels), float(kd_weight), float(ce_weight),
        KD_SCALE_T2 if scale_T2 else 0, _ptr(dH), _ptr(dW), _ptr(ws), ws.numel(), _stream_ptr(torch, dev))
    _check(st, "kd_topk_kl_backward_ex")
    return dH, dW


def keep_workspace_size(N: int, D: int, V: int, K: int, chunk: int) -> int:
    return int(load_library().kd_topk_kl_keep_workspace_size(N, D, V, K, chunk))


def forward_keep(H, W, topk_idx, topk_logit, T: float = 1.0, chunk: int = 1024,
                 want_row_kl: bool = False, workspace=None):
    """Kept-gradient comparator: the forward's outputs plus the workspace
    holding G for every position, which backward_keep consumes.  Returns
    (loss, lse[, row_kl], workspace)."""
    torch = _torch()
    N, D, V, K = _check_inputs(torch, H, W, topk_idx, topk_logit)
    dev = H.device
    need = keep_workspace_size(N, D, V, K, chunk)
    if need == 0:
        raise KDError(1, "keep_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    else:
        _given_workspace(torch, workspace, need, dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    row_kl = torch.empty(N, dtype=torch.float32, device=dev) if want_row_kl else None
    st = load_library().kd_topk_kl_forward_keep(
        _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit), N, D, V, K, float(T), int(chunk),
        _ptr(loss), _ptr(lse), _ptr(row_kl), _ptr(workspace), workspace.numel(),
        _stream_ptr(torch, dev))
    _check(st, "kd_topk_kl_forward_keep")
    return ((loss, lse, row_kl) if want_row_kl else (loss, lse)) + (workspace,)


def backward_keep(H, W, K: int, workspace, grad_loss=None, T: float = 1.0, chunk: int = 1024,
                  dW=None):
    """dH (overwritten) and dW (accumulated) from a forward_keep workspace."""
    torch = _torch()
    for name, x in (("H", H), ("W", W)):
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError(f"{name} must be a 2-D tensor")
    N, D = H.shape
    V = W.shape[0]
    dev = H.device
    _dev_tensor(torch, H, "H", torch.bfloat16, (N, D))
    _dev_tensor(torch, W, "W", torch.bfloat16, (V, D), dev)
    _check_grad_loss(torch, grad_loss, dev)
    need = keep_workspace_size(N, D, V, int(K), chunk)
    if need == 0:
        raise KDError(1, "keep_workspace_size")
    _given_workspace(torch, workspace, need, dev)
    dW = _out_dW(torch, dW, V, D, dev)
    dH = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    gl = grad_loss
    st = load_library().kd_topk_kl_backward_keep(
        _ptr(H), _ptr(W), _ptr(gl), N, D, V, int(K), float(T), int(chunk), _ptr(dH), _ptr(dW),
        _ptr(workspace), workspace.numel(), _stream_ptr(torch, dev))
    _check(st, "kd_topk_kl_backward_keep")
    return dH, dW


def keep_logits_workspace_size(N: int, D: int, V: int, K: int, chunk: int) -> int:
    return int(load_library().kd_topk_kl_keep_logits_workspace_size(N, D, V, K, chunk))


def forward_keep_logits(H, W, topk_idx, topk_logit, T: float = 1.0, chunk: int = 1024,
                        want_row_kl: bool = False, workspace=None):
    """Kept-logits comparator: the forward's outputs plus the workspace holding
    every chunk's fp32 logits, which backward_keep_logits consumes.  Returns
    (loss, lse[, row_kl], workspace)."""
    torch = _torch()
    N, D, V, K = _check_inputs(torch, H, W, topk_idx, topk_logit)
    dev = H.device
    need = keep_logits_workspace_size(N, D, V, K, chunk)
    if need == 0:
        raise KDError(1, "keep_logits_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    else:
        _given_workspace(torch, workspace, need, dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    row_kl = torch.empty(N, dtype=torch.float32, device=dev) if want_row_kl else None
    st = load_library().kd_topk_kl_forward_keep_logits(
        _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit), N, D, V, K, float(T), int(chunk),
        _ptr(loss), _ptr(lse), _ptr(row_kl), _ptr(workspace), workspace.numel(), _stream_ptr(torch, dev))
    _check(st, "kd_topk_kl_forward_keep_logits")
    return ((loss, lse, row_kl) if want_row_kl else (loss, lse)) + (workspace,)


def backward_keep_logits(H, W, topk_idx, topk_logit, lse, workspace, grad_loss=None, T: float = 1.0,
                         chunk: int = 1024, dW=None):
    """dH (overwritten) and dW (accumulated) from a forward_keep_logits
    workspace (its kept logits are consumed)."""
    torch = _torch()
    N, D, V, K = _check_inputs(torch, H, W, topk_idx, topk_logit)
    dev = H.device
    _check_lse(torch, lse, N, dev)
    _check_grad_loss(torch, grad_loss, dev)
    need = keep_logits_workspace_size(N, D, V, K, chunk)
    if need == 0:
        raise KDError(1, "keep_logits_workspace_size")
    _given_workspace(torch, workspace, need, dev)
    dW = _out_dW(torch, dW, V, D, dev)
    dH = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    st = load_library().kd_topk_kl_backward_keep_logits(
        _ptr(H), _ptr(W), _ptr(topk_idx), _ptr(topk_logit), _ptr(lse), _ptr(grad_loss), N, D, V, K,
        float(T), int(chunk), _ptr(dH), _ptr(dW), _ptr(workspace), workspace.numel(), _stream_ptr(torch, dev))
    _check(st, "kd_topk_kl_backward_keep_logits")
    return dH, dW


def _teacher_dtype(torch, teacher):
    if not isinstance(teacher, torch.Tensor):
        raise TypeError("teacher logits must be a torch.Tensor")
    if teacher.dtype == torch.float32:
        return 0
    if teacher.dtype == torch.bfloat16:
        return 1
    raise TypeError("teacher logits must be float32 or bfloat16")


def _check_dense(torch, H, W, teacher):
    for name, x in (("H", H), ("W", W), ("teacher", teacher)):
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError(f"{name} must be a 2-D tensor")
    N, D = H.shape
    V = W.shape[0]
    dev = H.device
    _dev_tensor(torch, H, "H", torch.bfloat16, (N, D))
    _dev_tensor(torch, W, "W", torch.bfloat16, (V, D), dev)
    _dev_tensor(torch, teacher, "teacher", teacher.dtype, (N, V), dev)
    return N, D, V, _teacher_dtype(torch, teacher)


def dense_workspace_size(N: int, D: int, V: int, chunk: int) -> int:
    return int(load_library().kd_dense_kl_workspace_size(N, D, V, chunk))


def _dense_workspace(torch, N, D, V, chunk, device, workspace):
    need = dense_workspace_size(N, D, V, chunk)
    if need == 0:
        raise KDError(1, "dense_workspace_size")
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    return _given_workspace(torch, workspace, need, device)


def dense_forward(H, W, teacher, T: float = 1.0, chunk: int = 1024, want_row_kl: bool = False,
                  workspace=None):
    """Dense-teacher KL over the full vocabulary: loss, lse, lse_t [, row_kl]."""
    torch = _torch()
    N, D, V, tdt = _check_dense(torch, H, W, teacher)
    dev = H.device
    ws = _dense_workspace(torch, N, D, V, chunk, dev, workspace)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    lse_t = torch.empty(N, dtype=torch.float32, device=dev)
    row_kl = torch.empty(N, dtype=torch.float32, device=dev) if want_row_kl else None
    st = load_library().kd_dense_kl_forward(
        _ptr(H), _ptr(W), _ptr(teacher), tdt, N, D, V, float(T), int(chunk),
        _ptr(loss), _ptr(lse), _ptr(lse_t), _ptr(row_kl), _ptr(ws), ws.numel(), _stream_ptr(torch, dev))
    _check(st, "kd_dense_kl_forward")
    return (loss, lse, lse_t, row_kl) if want_row_kl else (loss, lse, lse_t)


def dense_backward(H, W, teacher, lse, lse_t, grad_loss=None, T: float = 1.0, chunk: int = 1024,
                   dW=None, workspace=None):
    """dH (overwritten) and dW (accumulated) of the dense-teacher KL."""
    torch = _torch()
    N, D, V, tdt = _check_dense(torch, H, W, teacher)
    dev = H.device
    _check_lse(torch, lse, N, dev)
    _check_lse(torch, lse_t, N, dev, "lse_t")
    _check_grad_loss(torch, grad_loss, dev)
    dW = _out_dW(torch, dW, V, D, dev)
    ws = _dense_workspace(torch, N, D, V, chunk, dev, workspace)
    dH = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    gl = grad_loss
    st = load_library().kd_dense_kl_backward(
        _ptr(H), _ptr(W), _ptr(teacher), tdt, _ptr(lse), _ptr(lse_t), _ptr(gl),
        N, D, V, float(T), int(chunk), _ptr(dH), _ptr(dW), _ptr(ws), ws.numel(), _stream_ptr(torch, dev))
    _check(st, "kd_dense_kl_backward")
    return dH, dW


def topk_select(logits, K: int):
    """Teacher top-K cache of fp32 or bf16 logits [N, V]: (ids int32 [N, K],
    logits fp32 [N, K]), best first, equal logits by lower id."""
    torch = _torch()
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError("logits must be a 2-D tensor [N, V]")
    if logits.dtype == torch.float32:
        dtype = 0
    elif logits.dtype == torch.bfloat16:
        dtype = 1
    else:
        raise TypeError("logits must be float32 or bfloat16")
    _dev_tensor(torch, logits, "logits", logits.dtype)
    N, V = logits.shape
    idx = torch.empty((N, K), dtype=torch.int32, device=logits.device)
    val = torch.empty((N, K), dtype=torch.float32, device=logits.device)
    st = load_library().kd_topk_select(_ptr(logits), dtype, N, V, int(K), _ptr(idx), _ptr(val),
                                       _stream_ptr(torch, logits.device))
    _check(st, "kd_topk_select")
    return idx, val


def validate(topk_idx, V: int) -> int:
    """Bit 0: an id outside [0, V); bit 1: a repeated id within a row."""
    torch = _torch()
    if not isinstance(topk_idx, torch.Tensor) or topk_idx.dim() != 2:
        raise ValueError("topk_idx must be a 2-D tensor [N, K]")
    _dev_tensor(torch, topk_idx, "topk_idx", torch.int32)
    N, K = topk_idx.shape
    flags = torch.empty(1, dtype=torch.int32, device=topk_idx.device)
    st = load_library().kd_topk_kl_validate(_ptr(topk_idx), N, K, V, _ptr(flags),
                                            _stream_ptr(torch, topk_idx.device))
    _check(st, "kd_topk_kl_validate")
    return int(flags.item())


def profile_enable(kernels=None):
    """Times every launch of the named kernel classes with HIP events (None: off)."""
    mask = 0
    for k in ([kernels] if isinstance(kernels, str) else (kernels or [])):
        mask |= 1 << KERNELS[k]
    _check(load_library().kd_profile_enable(mask), "kd_profile_enable")


def profile_read(kernel: str):
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(load_library().kd_profile_read(KERNELS[kernel], ctypes.byref(ms), ctypes.byref(n)),
           "kd_profile_read")
    return ms.value, n.value


class KDTopKKL:
    """autograd.Function wrapper: loss = KDTopKKL.apply(H, W, topk_idx, topk_logit, T, chunk)."""

    _fn = None

    @classmethod
    def apply(cls, H, W, topk_idx, topk_logit, T: float = 1.0, chunk: int = 1024):
        if cls._fn is None:
            torch = _torch()

            class _F(torch.autograd.Function):
                @staticmethod
                def forward(ctx, H, W, idx, t, T, chunk):
                    loss, lse = forward(H, W, idx, t, T, chunk)
                    ctx.save_for_backward(H, W, idx, t, lse)
                    ctx.T, ctx.chunk = T, chunk
                    return loss[0]

                @staticmethod
                def backward(ctx, g):
                    H, W, idx, t, lse = ctx.saved_tensors
                    gl = g.reshape(1).to(torch.float32).contiguous()
                    dH, dW = backward(H, W, idx, t, lse, gl, ctx.T, ctx.chunk)
                    return dH, dW.to(W.dtype), None, None, None, None

            cls._fn = _F
        return cls._fn.apply(H, W, topk_idx, topk_logit, T, chunk)
