"""Python binding of libfab (the FlashAttention-2 backward for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libfab.so`` behind its C ABI (``include/fab.h``).  PyTorch provides device memory and the
current stream; there is no CPU or framework fallback -- if the library is missing or a
tensor is not on the GPU, the call raises.

    o, lse = fwd(q, k, v, causal=True)                       # supporting forward
    dq, dk, dv = bwd(do, q, k, v, o, lse, causal=True)       # the backward

Layouts: q, o, do ``[B, H, Sq, D]``; k, v ``[B, H_kv, Sk, D]`` (H % H_kv == 0, query head h
uses kv head h // (H / H_kv)); lse ``[B, H, Sq]`` float32.  One dtype (float32, float16 or
bfloat16) for all element tensors of a call.  ``scale`` defaults to 1/sqrt(D), the value
boostr's flash_bwd.rs launch block hard-codes; here it is a parameter.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = ["fwd", "bwd", "bwd_noalloc", "bwd_preprocess", "bwd_workspace_bytes", "bwd_plan", "lib", "FabError",
           "LIB_PATH", "DTYPE_CODES", "STATUS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfab.so")
STATUS = {0: "FAB_OK", 1: "FAB_ERR_INVALID_ARGUMENT", 2: "FAB_ERR_UNSUPPORTED",
          3: "FAB_ERR_DEVICE", 4: "FAB_ERR_LAUNCH"}
DTYPE_CODES = {"float32": 0, "float16": 1, "bfloat16": 2}

_lib = None
_lock = threading.Lock()


class FabError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfab.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m flashattention_backward_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
            L.fab_version.restype = ctypes.c_char_p
            L.fab_last_error.restype = ctypes.c_char_p
            L.fab_bwd_workspace_bytes.restype = sz
            L.fab_bwd_workspace_bytes.argtypes = [i] * 7
            L.fab_bwd_workspace_bytes_min.restype = sz
            L.fab_bwd_workspace_bytes_min.argtypes = [i] * 7
            L.fab_bwd_workspace_bytes_ds.restype = sz
            L.fab_bwd_workspace_bytes_ds.argtypes = [i] * 7
            L.fab_bwd_plan.restype = i
            L.fab_bwd_plan.argtypes = [i] * 7 + [sz]
            L.fab_fwd.restype = i
            L.fab_fwd.argtypes = [vp] * 5 + [i] * 7 + [i, i, f, vp]
            L.fab_bwd_preprocess.restype = i
            L.fab_bwd_preprocess.argtypes = [vp] * 4 + [sz] + [i] * 5 + [vp]
            L.fab_bwd.restype = i
            L.fab_bwd.argtypes = [vp] * 10 + [sz] + [i] * 7 + [i, i, f, vp]
            L.fab_bwd_noalloc.restype = i
            L.fab_bwd_noalloc.argtypes = [vp] * 9 + [i] * 7 + [i, i, f, vp]
            L.fab_bwd_dkdv.restype = i
            L.fab_bwd_dkdv.argtypes = [vp] * 5 + [sz] + [vp] * 2 + [i] * 7 + [i, i, f, vp]
            L.fab_bwd_dq.restype = i
            L.fab_bwd_dq.argtypes = [vp] * 5 + [sz] + [vp] + [i] * 7 + [i, i, f, vp]
            _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        msg = lib().fab_last_error().decode()
        if status in (1, 2):
            raise ValueError(f"{STATUS[status]}: {msg}")
        raise FabError(status, msg)


def _dtype_code(t) -> int:
    name = str(t.dtype).replace("torch.", "")
    if name not in DTYPE_CODES:
        raise ValueError(f"dtype: unsupported dtype {t.dtype} (float32, float16, bfloat16)")
    return DTYPE_CODES[name]


def _stream_handle(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(cond: bool, arg: str, reason: str):
    if not cond:
        raise ValueError(f"{arg}: {reason}")


def _check_tensor(t, name, shape, dtype, device):
    _require(t.is_cuda, name, "must be a GPU tensor")
    _require(t.device == device, name, f"on {t.device}, expected {device}")
    _require(tuple(t.shape) == tuple(shape), name, f"expected shape {tuple(shape)}, got {tuple(t.shape)}")
    _require(t.dtype == dtype, name, f"expected dtype {dtype}, got {t.dtype}")
    _require(t.is_contiguous(), name, "must be contiguous")


def bwd_workspace_bytes(B, H, H_kv, Sq, Sk, D, dtype_code, store_ds: bool | None = None) -> int:
    """Workspace bytes that select a mode of the backward: the recommended one (store_ds=None),
    stored dS (True; where that mode cannot run, the recompute size) or recompute (False)."""
    L = lib()
    args = (B, H, H_kv, Sq, Sk, D, dtype_code)
    if store_ds is None:
        return int(L.fab_bwd_workspace_bytes(*args))
    if store_ds:
        n = int(L.fab_bwd_workspace_bytes_ds(*args))
        if n:
            return n
    return int(L.fab_bwd_workspace_bytes_min(*args))


PLANS = {0: "recompute", 1: "recompute_one_launch", 2: "stored_ds", 3: "f32"}


def bwd_plan(B, H, H_kv, Sq, Sk, D, dtype_code, workspace_bytes) -> str:
    """The launch sequence fab_bwd takes for these sizes and workspace size (see fab.h)."""
    code = int(lib().fab_bwd_plan(B, H, H_kv, Sq, Sk, D, dtype_code, workspace_bytes))
    if code < 0:
        raise ValueError("invalid sizes or workspace too small")
    return PLANS[code]


def _window(window_size) -> int:
    w = int(window_size)
    _require(w >= 0, "window_size", f"{w} is negative (0 = no window)")
    return min(w, 2**31 - 1)


def fwd(q, k, v, causal: bool = False, scale: float | None = None, window_size: int = 0):
    """Supporting forward: returns (o [B,H,Sq,D] in q's dtype, lse [B,H,Sq] float32).

    window_size = W > 0 keeps W keys per query row i: keys j > i - W (and j < i + W without
    the causal mask).  A row left without keys gets o = 0 and lse = -inf."""
    import torch
    _require(q.dim() == 4, "q", f"must be 4-D [B, H, Sq, D], got {tuple(q.shape)}")
    _require(k.dim() == 4, "k", f"must be 4-D [B, H_kv, Sk, D], got {tuple(k.shape)}")
    B, H, Sq, D = q.shape
    H_kv, Sk = k.shape[1], k.shape[2]
    dev = q.device
    _check_tensor(q, "q", q.shape, q.dtype, dev)
    _check_tensor(k, "k", (B, H_kv, Sk, D), q.dtype, dev)
    _check_tensor(v, "v", (B, H_kv, Sk, D), q.dtype, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    _check(lib().fab_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         B, H, H_kv, Sq, Sk, D, _dtype_code(q), int(bool(causal)),
                         _window(window_size), float(scale), _stream_handle(dev)))
    return o, lse


STATS_ROWS = 64  # the workspace pads each (b, h) to a multiple of this many rows


def bwd_preprocess(do, o, lse):
    """Step 1 alone.  Returns (delta [B, H, Sq] float32 = rowsum(do * o), workspace); the
    workspace holds the per-row statistics the step-2 kernels read."""
    import torch
    _require(o.dim() == 4, "o", f"must be 4-D, got {tuple(o.shape)}")
    B, H, Sq, D = o.shape
    dev = o.device
    _check_tensor(o, "o", o.shape, o.dtype, dev)
    _check_tensor(do, "dO", o.shape, o.dtype, dev)
    _check_tensor(lse, "lse", (B, H, Sq), torch.float32, dev)
    code = _dtype_code(o)
    nb = bwd_workspace_bytes(B, H, H, Sq, 1, D, code)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    _check(lib().fab_bwd_preprocess(do.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(), nb,
                                    B, H, Sq, D, code, _stream_handle(dev)))
    sq_pad = (Sq + STATS_ROWS - 1) // STATS_ROWS * STATS_ROWS
    stats = ws[: B * H * sq_pad * 8].view(torch.float32).view(B, H, sq_pad, 2)
    return stats[:, :, :Sq, 1], ws


def bwd(do, q, k, v, o, lse, num_heads: int | None = None, num_kv_heads: int | None = None,
        causal: bool = False, scale: float | None = None, workspace=None, window_size: int = 0,
        store_ds: bool | None = None):
    """The backward: returns (dq, dk, dv) with the shapes and dtype of (q, k, v).  `causal`,
    `scale` and `window_size` must be those the forward ran with.  Without a `workspace`, one is
    allocated for the recommended mode (store_ds=None), the stored-dS mode (True, where it can
    run) or the recompute mode (False); a given workspace selects the mode by its size."""
    import torch
    _require(q.dim() == 4, "q", f"must be 4-D [B, H, Sq, D], got {tuple(q.shape)}")
    _require(k.dim() == 4, "k", f"must be 4-D [B, H_kv, Sk, D], got {tuple(k.shape)}")
    B, H, Sq, D = q.shape
    H_kv, Sk = k.shape[1], k.shape[2]
    if num_heads is not None:
        _require(num_heads == H, "num_heads", f"{num_heads} does not match q's {H} heads")
    if num_kv_heads is not None:
        _require(num_kv_heads == H_kv, "num_kv_heads", f"{num_kv_heads} does not match k's {H_kv} heads")
    dev = q.device
    dt = q.dtype
    _check_tensor(q, "q", (B, H, Sq, D), dt, dev)
    _check_tensor(k, "k", (B, H_kv, Sk, D), dt, dev)
    _check_tensor(v, "v", (B, H_kv, Sk, D), dt, dev)
    _check_tensor(o, "output", (B, H, Sq, D), dt, dev)
    _check_tensor(do, "dout", (B, H, Sq, D), dt, dev)
    _check_tensor(lse, "lse", (B, H, Sq), torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    code = _dtype_code(q)
    need = bwd_workspace_bytes(B, H, H_kv, Sq, Sk, D, code, store_ds=False)
    if workspace is None:
        nb = bwd_workspace_bytes(B, H, H_kv, Sq, Sk, D, code, store_ds=store_ds)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _require(workspace.is_cuda and workspace.numel() * workspace.element_size() >= need,
             "workspace", f"needs {need} bytes on {dev}")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    _check(lib().fab_bwd(do.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                         lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                         workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                         B, H, H_kv, Sq, Sk, D, code, int(bool(causal)), _window(window_size),
                         float(scale), _stream_handle(dev)))
    return dq, dk, dv


def bwd_noalloc(do, q, k, v, o, lse, causal: bool = False, scale: float | None = None,
                window_size: int = 0, out=None):
    """The backward through fab_bwd_noalloc: no workspace; the library keeps the per-row
    statistics in its static per-GPU scratch (at most 2^21 padded query rows, B * H * Sq
    rounded up to 64).  ``out`` = (dq, dk, dv) preallocated tensors to write into (so that the
    call itself allocates nothing); by default they are allocated here.  Calls that overlap on
    one GPU race on the shared scratch."""
    import torch
    _require(q.dim() == 4, "q", f"must be 4-D [B, H, Sq, D], got {tuple(q.shape)}")
    _require(k.dim() == 4, "k", f"must be 4-D [B, H_kv, Sk, D], got {tuple(k.shape)}")
    B, H, Sq, D = q.shape
    H_kv, Sk = k.shape[1], k.shape[2]
    dev, dt = q.device, q.dtype
    _check_tensor(q, "q", (B, H, Sq, D), dt, dev)
    _check_tensor(k, "k", (B, H_kv, Sk, D), dt, dev)
    _check_tensor(v, "v", (B, H_kv, Sk, D), dt, dev)
    _check_tensor(o, "output", (B, H, Sq, D), dt, dev)
    _check_tensor(do, "dout", (B, H, Sq, D), dt, dev)
    _check_tensor(lse, "lse", (B, H, Sq), torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    _check_tensor(dq, "dq", (B, H, Sq, D), dt, dev)
    _check_tensor(dk, "dk", (B, H_kv, Sk, D), dt, dev)
    _check_tensor(dv, "dv", (B, H_kv, Sk, D), dt, dev)
    _check(lib().fab_bwd_noalloc(do.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 o.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                 dv.data_ptr(), B, H, H_kv, Sq, Sk, D, _dtype_code(q),
                                 int(bool(causal)), _window(window_size), float(scale),
                                 _stream_handle(dev)))
    return dq, dk, dv
