"""Thin Python binding over libwkv7.so (argument marshalling only).

Torch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  The names mirror the C ABI in
include/wkv7.h: wkv7_forward (which calls wkv7_forward_ws when the two-pass
form runs), wkv7_decode_step, wkv7_resolve_algo, wkv7_workspace_bytes.

If the library is missing, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "wkv7_forward", "wkv7_forward_noalloc", "wkv7_backward", "wkv7_decode_step", "wkv7_resolve_algo", "wkv7_workspace_bytes",
    "wkv7_backward_workspace_bytes", "wkv4_forward", "wkv4_workspace_bytes", "wkv4_wait_status", "Wkv7Error",
    "lib_path", "load_library",
    "WKV7_OK", "WKV7_EINVAL", "WKV7_EUNSUPPORTED", "WKV7_EDEVICE", "WKV7_ELAUNCH", "WKV7_ETIMEOUT",
    "ALGOS", "W_MODES", "AB_MODES", "Desc", "EXPORTED_SYMBOLS",
]

WKV7_OK, WKV7_EINVAL, WKV7_EUNSUPPORTED, WKV7_EDEVICE, WKV7_ELAUNCH, WKV7_ETIMEOUT = 0, 1, 2, 3, 4, 5
_DTYPES = {"f32": 0, "bf16": 1}
W_MODES = {"decay": 0, "logneglog": 1}
ALGOS = {"auto": 0, "scan": 1, "chunked": 2, "two_pass": 3}
AB_MODES = {"given": 0, "from_k": 1}
EXPORTED_SYMBOLS = ("wkv7_forward", "wkv7_forward_ws", "wkv7_forward_noalloc", "wkv7_workspace_bytes", "wkv7_decode_step",
                    "wkv7_backward", "wkv7_backward_workspace_bytes", "wkv4_forward", "wkv4_workspace_bytes",
                    "wkv4_wait_status", "wkv7_resolve_algo", "wkv7_strerror", "wkv7_last_error", "wkv7_abi_version")


class Wkv7Error(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__(f"{where}: {_status_name(code)} ({code}): {detail}")
        self.code = code


class Desc(ctypes.Structure):
    """Mirror of struct wkv7_desc."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("H_kv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32),
        ("w_mode", ctypes.c_int32), ("algo", ctypes.c_int32), ("chunk_len", ctypes.c_int32),
        ("y_scale", ctypes.c_float), ("ab_mode", ctypes.c_int32), ("r_k", ctypes.c_void_p),
        ("mask", ctypes.c_void_p),
    ]


class Wkv4Desc(ctypes.Structure):
    """Mirror of struct wkv4_desc."""
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("C", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32), ("spin_limit", ctypes.c_int32)]


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwkv7.so")


_LIB = None


def load_library():
    """Load libwkv7.so (once) and declare the C signatures.  Raises if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m linear_rnn_sequence_wkv7_amd.build`")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    sig = [ctypes.POINTER(Desc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    for name in ("wkv7_forward", "wkv7_decode_step", "wkv7_forward_noalloc"):
        fn = getattr(lib, name)
        fn.argtypes = sig
        fn.restype = ctypes.c_int
    lib.wkv7_forward_ws.argtypes = sig[:-1] + [vp, ctypes.c_int64, vp]
    lib.wkv7_forward_ws.restype = ctypes.c_int
    lib.wkv7_workspace_bytes.argtypes = [ctypes.POINTER(Desc)]
    lib.wkv7_workspace_bytes.restype = ctypes.c_int64
    lib.wkv7_backward.argtypes = [ctypes.POINTER(Desc)] + [vp] * 18 + [ctypes.c_int64, vp]
    lib.wkv7_backward.restype = ctypes.c_int
    lib.wkv7_backward_workspace_bytes.argtypes = [ctypes.POINTER(Desc)]
    lib.wkv7_backward_workspace_bytes.restype = ctypes.c_int64
    lib.wkv4_forward.argtypes = [ctypes.POINTER(Wkv4Desc)] + [vp] * 8 + [ctypes.c_int64, vp]
    lib.wkv4_forward.restype = ctypes.c_int
    lib.wkv4_workspace_bytes.argtypes = [ctypes.POINTER(Wkv4Desc)]
    lib.wkv4_workspace_bytes.restype = ctypes.c_int64
    lib.wkv4_wait_status.argtypes = [ctypes.POINTER(Wkv4Desc), vp, ctypes.c_int64, vp]
    lib.wkv4_wait_status.restype = ctypes.c_int
    lib.wkv7_resolve_algo.argtypes = [ctypes.POINTER(Desc)]
    lib.wkv7_resolve_algo.restype = ctypes.c_int
    lib.wkv7_strerror.argtypes = [ctypes.c_int]
    lib.wkv7_strerror.restype = ctypes.c_char_p
    lib.wkv7_last_error.argtypes = []
    lib.wkv7_last_error.restype = ctypes.c_char_p
    lib.wkv7_abi_version.argtypes = []
    lib.wkv7_abi_version.restype = ctypes.c_int
    _LIB = lib
    return lib


def _status_name(code: int) -> str:
    try:
        return load_library().wkv7_strerror(code).decode()
    except Exception:  # pragma: no cover - only while reporting another failure
        return "status"


def make_desc(B, T, H, D, *, H_kv=None, in_dtype="bf16", y_dtype="bf16", w_mode="decay",
              algo="auto", chunk_len=0, y_scale=1.0, r_k_ptr=None, ab_mode="given", mask_ptr=None) -> Desc:
    return Desc(B=B, T=T, H=H, H_kv=H if H_kv is None else H_kv, D=D,
                in_dtype=_DTYPES[in_dtype], y_dtype=_DTYPES[y_dtype], w_mode=W_MODES[w_mode],
                algo=ALGOS[algo], chunk_len=chunk_len, y_scale=float(y_scale), ab_mode=AB_MODES[ab_mode],
                r_k=r_k_ptr, mask=mask_ptr)


def _torch():
    import torch
    return torch


def _dtype_name(t) -> str:
    torch = _torch()
    if t.dtype == torch.float32:
        return "f32"
    if t.dtype == torch.bfloat16:
        return "bf16"
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_inputs(r, w, k, v, a, b, state, r_k, mask=None, ab_mode="given"):
    torch = _torch()
    if r.dim() != 4:
        raise ValueError("r must be [B, T, H, D]")
    B, T, H, D = r.shape
    dev = r.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    dt = r.dtype
    if ab_mode not in AB_MODES:
        raise ValueError(f"ab_mode must be one of {sorted(AB_MODES)}")
    if b is None and ab_mode != "from_k":
        raise ValueError("b is required unless ab_mode='from_k'")
    for name, x in (("w", w), ("a", a), ("b", b)):
        if x is None:
            continue
        if tuple(x.shape) != (B, T, H, D):
            raise ValueError(f"{name} must have shape {(B, T, H, D)}, got {tuple(x.shape)}")
    if k.dim() != 4 or tuple(k.shape[:2]) != (B, T) or k.shape[3] != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, T, H_kv, D] with matching shapes")
    for name, x in (("r", r), ("w", w), ("k", k), ("v", v), ("a", a), ("b", b)):
        if x is None:
            continue
        if x.dtype != dt:
            raise TypeError(f"{name} has dtype {x.dtype}, expected {dt} like r")
        if x.device != dev or not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous and on {dev}")
    if state is not None:
        if tuple(state.shape) != (B, H, D, D) or state.dtype != torch.float32:
            raise ValueError(f"state must be float32 [B, H, D, D] = {(B, H, D, D)}")
        if state.device != dev or not state.is_contiguous():
            raise ValueError(f"state must be contiguous and on {dev}")
    if r_k is not None:
        if tuple(r_k.shape) != (H, D) or r_k.dtype != torch.float32 or r_k.device != dev or not r_k.is_contiguous():
            raise ValueError(f"r_k must be contiguous float32 [H, D] = {(H, D)} on {dev}")
    if mask is not None:
        if (tuple(mask.shape) != (B, T) or mask.dtype not in (torch.uint8, torch.bool)
                or mask.device != dev or not mask.is_contiguous()):
            raise ValueError(f"mask must be a contiguous uint8 or bool [B, T] = {(B, T)} tensor on {dev}")
    return B, T, H, int(k.shape[2]), D


def _call(fn_name, desc, r, w, k, v, a, b, state, y, state_out, workspace=None):
    torch = _torch()
    lib = load_library()
    stream = torch.cuda.current_stream(r.device).cuda_stream
    args = [ctypes.byref(desc), _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
            _ptr(state), _ptr(y), _ptr(state_out)]
    if fn_name == "wkv7_forward_ws":
        args += [_ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size()]
    with torch.cuda.device(r.device):
        rc = getattr(lib, fn_name)(*args, stream)
    if rc != WKV7_OK:
        raise Wkv7Error(rc, fn_name, lib.wkv7_last_error().decode())


def wkv7_workspace_bytes(B, T, H, D, *, H_kv=None, algo="auto", **kw) -> int:
    """Workspace bytes wkv7_forward_ws uses for these sizes (0: none)."""
    n = load_library().wkv7_workspace_bytes(ctypes.byref(make_desc(B, T, H, D, H_kv=H_kv, algo=algo, **kw)))
    if n < 0:
        raise Wkv7Error(int(-n), "wkv7_workspace_bytes", load_library().wkv7_last_error().decode())
    return int(n)


def wkv7_forward(r, w, k, v, a, b, state=None, *, w_mode: str = "decay", y_dtype: Optional[str] = None,
                 algo: str = "auto", chunk_len: int = 0, y_scale: float = 1.0, r_k=None,
                 ab_mode: str = "given", mask=None,
                 y=None, state_out=None, return_state: bool = True, workspace=None) -> Tuple[object, object]:
    """Run the forward on torch GPU tensors.

    r, w, a, b: [B, T, H, D]; k, v: [B, T, H_kv, D]; all float32 or all bfloat16, contiguous.
    state: [B, H, D, D] float32 or None (zeros).  r_k: [H, D] float32 or None.
    ab_mode "from_k": a holds alpha and b is unused (may be None); the kernel
    forms kk = normalize(k), a = -kk, b = kk * alpha, k * (1 - decay + alpha).
    mask: [B, T] uint8 / bool device tensor (0 = token masked) or None.
    y_dtype: "f32" | "bf16" (default: the input dtype).  Outputs are allocated
    unless `y` / `state_out` are given (state_out may equal state: in place).
    algo "auto" and "two_pass" go through wkv7_forward_ws: when the library
    reports a workspace size for the descriptor, `workspace` (a contiguous
    device tensor of at least that many bytes) is used, or allocated here.
    Returns (y, state_out); state_out is None when return_state is False.
    """
    torch = _torch()
    B, T, H, H_kv, D = _check_inputs(r, w, k, v, a, b, state, r_k, mask, ab_mode)
    ydt = y_dtype or _dtype_name(r)
    if y is None:
        y = torch.empty((B, T, H, D), dtype=torch.float32 if ydt == "f32" else torch.bfloat16, device=r.device)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=r.device)
    desc = make_desc(B, T, H, D, H_kv=H_kv, in_dtype=_dtype_name(r), y_dtype=ydt, w_mode=w_mode, algo=algo,
                     chunk_len=chunk_len, y_scale=y_scale, r_k_ptr=_ptr(r_k), ab_mode=ab_mode,
                     mask_ptr=_ptr(mask))
    if algo in ("auto", "two_pass"):
        need = load_library().wkv7_workspace_bytes(ctypes.byref(desc))
        if need < 0:
            raise Wkv7Error(int(-need), "wkv7_workspace_bytes", load_library().wkv7_last_error().decode())
        if need > 0 and workspace is None:
            workspace = torch.empty(int(need), dtype=torch.uint8, device=r.device)
        if workspace is not None and (workspace.device != r.device or not workspace.is_contiguous()):
            raise ValueError(f"workspace must be a contiguous tensor on {r.device}")
        _call("wkv7_forward_ws", desc, r, w, k, v, a, b, state, y, state_out, workspace)
    else:
        _call("wkv7_forward", desc, r, w, k, v, a, b, state, y, state_out)
    return y, state_out


def wkv7_forward_noalloc(r, w, k, v, a, b, state=None, *, w_mode: str = "decay", y_dtype: Optional[str] = None,
                         algo: str = "auto", chunk_len: int = 0, y_scale: float = 1.0, r_k=None,
                         ab_mode: str = "given", mask=None, y=None, state_out=None,
                         return_state: bool = True) -> Tuple[object, object]:
    """wkv7_forward through the allocation-free entry point: no workspace, the
    two-pass form runs in the library's static device scratch.  Arguments as in
    wkv7_forward; `y` and `state_out` are allocated here unless given."""
    torch = _torch()
    B, T, H, H_kv, D = _check_inputs(r, w, k, v, a, b, state, r_k, mask, ab_mode)
    ydt = y_dtype or _dtype_name(r)
    if y is None:
        y = torch.empty((B, T, H, D), dtype=torch.float32 if ydt == "f32" else torch.bfloat16, device=r.device)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=r.device)
    desc = make_desc(B, T, H, D, H_kv=H_kv, in_dtype=_dtype_name(r), y_dtype=ydt, w_mode=w_mode, algo=algo,
                     chunk_len=chunk_len, y_scale=y_scale, r_k_ptr=_ptr(r_k), ab_mode=ab_mode,
                     mask_ptr=_ptr(mask))
    _call("wkv7_forward_noalloc", desc, r, w, k, v, a, b, state, y, state_out)
    return y, state_out


NOALLOC_SCRATCH_BYTES = 64 << 20


def wkv7_decode_step(r, w, k, v, a, b, state, *, w_mode: str = "decay", y_dtype: Optional[str] = None,
                     y_scale: float = 1.0, r_k=None, ab_mode: str = "given", mask=None,
                     y=None, state_out=None) -> Tuple[object, object]:
    """One token per sequence: inputs [B, 1, H, D] (k, v [B, 1, H_kv, D]); state [B, H, D, D] or None.
    ab_mode and mask ([B, 1]) as in wkv7_forward."""
    torch = _torch()
    B, T, H, H_kv, D = _check_inputs(r, w, k, v, a, b, state, r_k, mask, ab_mode)
    if T != 1:
        raise ValueError("decode_step takes exactly one token per sequence (T == 1)")
    ydt = y_dtype or _dtype_name(r)
    if y is None:
        y = torch.empty((B, 1, H, D), dtype=torch.float32 if ydt == "f32" else torch.bfloat16, device=r.device)
    if state_out is None:
        state_out = torch.empty((B, H, D, D), dtype=torch.float32, device=r.device)
    desc = make_desc(B, 1, H, D, H_kv=H_kv, in_dtype=_dtype_name(r), y_dtype=ydt, w_mode=w_mode,
                     y_scale=y_scale, r_k_ptr=_ptr(r_k), ab_mode=ab_mode, mask_ptr=_ptr(mask))
    _call("wkv7_decode_step", desc, r, w, k, v, a, b, state, y, state_out)
    return y, state_out


def wkv7_resolve_algo(B, T, H, D, *, H_kv=None, algo="auto", **kw) -> str:
    """Which algorithm the C wkv7_forward runs for these sizes ("scan" or "chunked";
    an explicit "two_pass" is returned as is)."""
    rc = load_library().wkv7_resolve_algo(ctypes.byref(make_desc(B, T, H, D, H_kv=H_kv, algo=algo, **kw)))
    if rc < 0:
        raise Wkv7Error(-rc, "wkv7_resolve_algo", load_library().wkv7_last_error().decode())
    return {1: "scan", 2: "chunked", 3: "two_pass"}[rc]


def wkv7_backward_workspace_bytes(B, T, H, D, *, H_kv=None, **kw) -> int:
    """Workspace bytes wkv7_backward uses for these sizes."""
    n = load_library().wkv7_backward_workspace_bytes(ctypes.byref(make_desc(B, T, H, D, H_kv=H_kv, **kw)))
    if n < 0:
        raise Wkv7Error(int(-n), "wkv7_backward_workspace_bytes", load_library().wkv7_last_error().decode())
    return int(n)


def wkv7_backward(r, w, k, v, a, b, dy, state=None, dstate=None, *, w_mode: str = "decay",
                  y_scale: float = 1.0, r_k=None, mask=None, workspace=None, grads=None,
                  return_dstate: bool = True) -> dict:
    """Gradients of <dy, y> + <dstate, state_out> for wkv7_forward with the same arguments.

    dy: [B, T, H, D] float32 or bfloat16 (the y dtype); dstate: [B, H, D, D] float32 or None.
    Returns a dict of float32 tensors: r, w, a, b [B, T, H, D], k, v [B, T, H_kv, D],
    state [B, H, D, D] (None when return_dstate is False) and r_k [H, D] (None without r_k).
    `grads` may supply preallocated output tensors under the same keys.
    """
    torch = _torch()
    B, T, H, H_kv, D = _check_inputs(r, w, k, v, a, b, state, r_k, mask)
    dev = r.device
    if tuple(dy.shape) != (B, T, H, D) or dy.device != dev or not dy.is_contiguous():
        raise ValueError(f"dy must be a contiguous [B, T, H, D] = {(B, T, H, D)} tensor on {dev}")
    if dstate is not None:
        if tuple(dstate.shape) != (B, H, D, D) or dstate.dtype != torch.float32 or dstate.device != dev \
                or not dstate.is_contiguous():
            raise ValueError(f"dstate must be contiguous float32 [B, H, D, D] = {(B, H, D, D)} on {dev}")
    out = dict(grads or {})
    f32 = dict(dtype=torch.float32, device=dev)
    for key in ("r", "w", "a", "b"):
        out.setdefault(key, torch.empty((B, T, H, D), **f32))
    for key in ("k", "v"):
        out.setdefault(key, torch.empty((B, T, H_kv, D), **f32))
    if return_dstate:
        out.setdefault("state", torch.empty((B, H, D, D), **f32))
    else:
        out["state"] = None
    out["r_k"] = out.get("r_k", torch.empty((H, D), **f32)) if r_k is not None else None
    desc = make_desc(B, T, H, D, H_kv=H_kv, in_dtype=_dtype_name(r), y_dtype=_dtype_name(dy), w_mode=w_mode,
                     y_scale=y_scale, r_k_ptr=_ptr(r_k), mask_ptr=_ptr(mask))
    lib = load_library()
    need = lib.wkv7_backward_workspace_bytes(ctypes.byref(desc))
    if need < 0:
        raise Wkv7Error(int(-need), "wkv7_backward_workspace_bytes", lib.wkv7_last_error().decode())
    if need > 0 and workspace is None:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = [ctypes.byref(desc)] + [_ptr(x) for x in (r, w, k, v, a, b, state, dy, dstate)] + \
           [_ptr(out[n]) for n in ("r", "w", "k", "v", "a", "b", "state", "r_k")] + [_ptr(workspace), ws_bytes, stream]
    with torch.cuda.device(dev):
        rc = lib.wkv7_backward(*args)
    if rc != WKV7_OK:
        raise Wkv7Error(rc, "wkv7_backward", lib.wkv7_last_error().decode())
    return out


def wkv4_workspace_bytes(B, T, C, *, in_dtype="bf16", y_dtype="bf16") -> int:
    """Workspace bytes of wkv4_forward for these sizes."""
    d = Wkv4Desc(B=B, T=T, C=C, in_dtype=_DTYPES[in_dtype], y_dtype=_DTYPES[y_dtype], spin_limit=0)
    n = load_library().wkv4_workspace_bytes(ctypes.byref(d))
    if n < 0:
        raise Wkv7Error(int(-n), "wkv4_workspace_bytes", load_library().wkv7_last_error().decode())
    return int(n)


def wkv4_forward(w, u, k, v, state=None, *, y_dtype: Optional[str] = None, y=None, state_out=None,
                 return_state: bool = True, workspace=None, spin_limit: int = 0) -> Tuple[object, object]:
    """RWKV-4 WKV on torch GPU tensors: w, u [C] float32; k, v [B, T, C] float32 or bfloat16;
    state [B, 3, C] float32 (A, Bs, P with a = A e^P, b = Bs e^P) or None.  Returns (y, state_out).
    spin_limit: polls before a look-back wait gives up (0: the library's bound); pass a
    `workspace` to read the count of such waits afterwards with wkv4_wait_status."""
    torch = _torch()
    if k.dim() != 3 or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, T, C] with the same shape")
    B, T, C = k.shape
    dev = k.device
    for name, x in (("w", w), ("u", u)):
        if tuple(x.shape) != (C,) or x.dtype != torch.float32 or x.device != dev or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 [C] = {(C,)} tensor on {dev}")
    if v.dtype != k.dtype or not k.is_contiguous() or not v.is_contiguous() or v.device != dev:
        raise ValueError("k and v must be contiguous, on one device, with one dtype")
    if state is not None and (tuple(state.shape) != (B, 3, C) or state.dtype != torch.float32 or
                              state.device != dev or not state.is_contiguous()):
        raise ValueError(f"state must be contiguous float32 [B, 3, C] = {(B, 3, C)} on {dev}")
    ydt = y_dtype or _dtype_name(k)
    if y is None:
        y = torch.empty((B, T, C), dtype=torch.float32 if ydt == "f32" else torch.bfloat16, device=dev)
    if state_out is None and return_state:
        state_out = torch.empty((B, 3, C), dtype=torch.float32, device=dev)
    d = Wkv4Desc(B=B, T=T, C=C, in_dtype=_DTYPES[_dtype_name(k)], y_dtype=_DTYPES[ydt], spin_limit=spin_limit)
    lib = load_library()
    need = lib.wkv4_workspace_bytes(ctypes.byref(d))
    if need < 0:
        raise Wkv7Error(int(-need), "wkv4_workspace_bytes", lib.wkv7_last_error().decode())
    if need > 0 and workspace is None:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = lib.wkv4_forward(ctypes.byref(d), _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(state), _ptr(y),
                              _ptr(state_out), _ptr(workspace), ws_bytes, stream)
    if rc != WKV7_OK:
        raise Wkv7Error(rc, "wkv4_forward", lib.wkv7_last_error().decode())
    return y, state_out


def wkv4_wait_status(k, workspace, *, y_dtype: Optional[str] = None) -> int:
    """After wkv4_forward(..., workspace=workspace) with this k: WKV7_OK, or WKV7_ETIMEOUT if
    any look-back wait of that call gave up (y is NaN in its chunk).  Waits for the
    current stream."""
    torch = _torch()
    B, T, C = k.shape
    d = Wkv4Desc(B=B, T=T, C=C, in_dtype=_DTYPES[_dtype_name(k)], y_dtype=_DTYPES[y_dtype or _dtype_name(k)],
                 spin_limit=0)
    lib = load_library()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(k.device).cuda_stream
    with torch.cuda.device(k.device):
        rc = lib.wkv4_wait_status(ctypes.byref(d), _ptr(workspace), ws_bytes, stream)
    if rc not in (WKV7_OK, WKV7_ETIMEOUT):
        raise Wkv7Error(rc, "wkv4_wait_status", lib.wkv7_last_error().decode())
    return rc
