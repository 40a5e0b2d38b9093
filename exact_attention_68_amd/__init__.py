"""Python binding of libattn, the fused exact-attention forward for MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libattn.so, reached through its C ABI (include/attn.h). The names
mirror the C entry points. PyTorch supplies device memory and streams.

The first call loads exact_attention_68_amd/libattn.so and raises
ImportError if it has not been built (python -m exact_attention_68_amd.build);
there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_MASK_NONE = 0
ATTN_MASK_CAUSAL = 1
ATTN_MASK_NA2D = 2
ATTN_MASK_NA3D = 3

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_PARAMS = 3
ATTN_ERR_ALIGNMENT = 4
ATTN_ERR_HIP = 5
ATTN_ERR_WORKSPACE = 6
ATTN_ERR_SCRATCH = 7


class attn_na2d_params_t(ctypes.Structure):
    """Mirror of the C struct: 2D neighbourhood window over a row-major grid."""

    _fields_ = [(n, ctypes.c_int32) for n in
                ("grid_h", "grid_w", "kernel_h", "kernel_w", "wrap_h", "wrap_w", "dil_h", "dil_w")]


def na2d_params(grid_h, grid_w, kernel_h, kernel_w, wrap_h=1, wrap_w=1, dil_h=1, dil_w=1) -> attn_na2d_params_t:
    return attn_na2d_params_t(grid_h, grid_w, kernel_h, kernel_w, int(wrap_h), int(wrap_w), dil_h, dil_w)


class attn_na3d_params_t(ctypes.Structure):
    """Mirror of the C struct: 3D neighbourhood window over a row-major volume."""

    _fields_ = [(n, ctypes.c_int32) for n in
                ("grid_d", "grid_h", "grid_w", "kernel_d", "kernel_h", "kernel_w",
                 "wrap_d", "wrap_h", "wrap_w", "dil_d", "dil_h", "dil_w")]


def na3d_params(grid_d, grid_h, grid_w, kernel_d, kernel_h, kernel_w, wrap_d=1, wrap_h=1, wrap_w=1,
                dil_d=1, dil_h=1, dil_w=1) -> attn_na3d_params_t:
    return attn_na3d_params_t(grid_d, grid_h, grid_w, kernel_d, kernel_h, kernel_w,
                              int(wrap_d), int(wrap_h), int(wrap_w), dil_d, dil_h, dil_w)


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {attn_status_string(status)} (status {status})")
        self.status = status


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m exact_attention_68_amd.build`")
    lib = ctypes.CDLL(path)
    i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, vp, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_ws.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, vp, vp, ctypes.c_uint64, vp]
    lib.attn_fwd_ws.restype = i32
    lib.attn_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i32, vp, ctypes.POINTER(ctypes.c_uint64)]
    lib.attn_fwd_workspace_size.restype = i32
    lib.attn_fwd_check.argtypes = [i64, i64, i64, i64, f32, i32, vp]
    lib.attn_fwd_check.restype = i32
    lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, vp, vp, ctypes.c_uint64, vp]
    lib.attn_fwd_ex.restype = i32
    lib.attn_fwd_ex_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, vp, ctypes.POINTER(ctypes.c_uint64)]
    lib.attn_fwd_ex_workspace_size.restype = i32
    lib.attn_fwd_ex_check.argtypes = [i64, i64, i64, i64, i64, f32, i32, vp]
    lib.attn_fwd_ex_check.restype = i32
    lib.attn_fwd_ex_static.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, vp, vp]
    lib.attn_fwd_ex_static.restype = i32
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, vp, vp,
                             ctypes.c_uint64, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, vp, ctypes.POINTER(ctypes.c_uint64)]
    lib.attn_bwd_workspace_size.restype = i32
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = i32
    return lib


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded libattn.so (loaded on first use)."""
    global _lib_handle
    if _lib_handle is None:
        _lib_handle = _load()
    return _lib_handle


def _params_ptr(params):
    if params is None:
        return None
    if not isinstance(params, (attn_na2d_params_t, attn_na3d_params_t)):
        raise TypeError("params must be an attn_na2d_params_t or attn_na3d_params_t (see na2d_params, na3d_params)")
    return ctypes.cast(ctypes.pointer(params), ctypes.c_void_p)


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def attn_abi_version() -> int:
    return int(lib().attn_abi_version())


def attn_fwd_check(B, H, N, d, scale, mask_mode=ATTN_MASK_NONE, params=None) -> int:
    """Status attn_fwd would return for these sizes and options (no device work)."""
    return int(lib().attn_fwd_check(B, H, N, d, scale, mask_mode, _params_ptr(params)))


def _check_tensors(q, k, v, o, same_n=True):
    """Shapes [B, H, Nq, d] for q and o and [B, H, Nkv, d] for k and v (Nq = Nkv when same_n)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError(f"{name} must be a bfloat16 CUDA tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must have four dimensions [B, H, N, d]")
    if o.shape != q.shape or v.shape != k.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("q and o must be [B, H, Nq, d] and k, v [B, H, Nkv, d]")
    if same_n and k.shape != q.shape:
        raise ValueError("q, k, v and o must share one [B, H, N, d] shape")
    return q.shape[0], q.shape[1], q.shape[2], k.shape[2], q.shape[3]


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    return int(stream) or None


def attn_fwd(q, k, v, o, scale, mask_mode=ATTN_MASK_NONE, params=None, stream=None) -> None:
    """o <- softmax(scale * q k^T + mask) v, queued on `stream` (torch's current stream by default).

    q, k, v, o: torch bfloat16 CUDA tensors, contiguous, one [B, H, N, d] shape.
    Raises AttnError with the library's status on any rejected argument.
    """
    B, H, N, _, d = _check_tensors(q, k, v, o)
    rc = lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, d,
                        float(scale), int(mask_mode), _params_ptr(params), _stream_handle(stream, q.device))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd")


def attn_fwd_workspace_size(B, H, N, d, mask_mode=ATTN_MASK_NONE, params=None) -> int:
    """Bytes of workspace attn_fwd_ws needs for this problem on the current device (0: none)."""
    out = ctypes.c_uint64(0)
    rc = lib().attn_fwd_workspace_size(B, H, N, d, int(mask_mode), _params_ptr(params), ctypes.byref(out))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd_workspace_size")
    return int(out.value)


def attn_fwd_ws(q, k, v, o, scale, mask_mode=ATTN_MASK_NONE, params=None, workspace=None, stream=None) -> None:
    """attn_fwd with a device workspace (a uint8 CUDA tensor of at least attn_fwd_workspace_size
    bytes, any content, or None when that size is 0); see include/attn.h."""
    B, H, N, _, d = _check_tensors(q, k, v, o)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = lib().attn_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, d, float(scale),
                           int(mask_mode), _params_ptr(params), ws_ptr, ws_bytes, _stream_handle(stream, q.device))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd_ws")


def attn_fwd_ex_check(B, H, Nq, Nkv, d, scale, mask_mode=ATTN_MASK_NONE, params=None) -> int:
    """Status attn_fwd_ex would return for these sizes and options (no device work)."""
    return int(lib().attn_fwd_ex_check(B, H, Nq, Nkv, d, scale, mask_mode, _params_ptr(params)))


def attn_fwd_ex_workspace_size(B, H, Nq, Nkv, d, mask_mode=ATTN_MASK_NONE, params=None) -> int:
    """Bytes of workspace attn_fwd_ex needs for this problem on the current device (0: none)."""
    out = ctypes.c_uint64(0)
    rc = lib().attn_fwd_ex_workspace_size(B, H, Nq, Nkv, d, int(mask_mode), _params_ptr(params), ctypes.byref(out))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd_ex_workspace_size")
    return int(out.value)


def attn_fwd_ex(q, k, v, o, lse=None, scale=1.0, mask_mode=ATTN_MASK_NONE, params=None, workspace=None,
                stream=None) -> None:
    """o <- softmax(scale * q k^T + mask) v with q, o [B, H, Nq, d] and k, v [B, H, Nkv, d];
    lse, if given (a float32 CUDA tensor [B, H, Nq], contiguous), receives each row's logsumexp.
    See include/attn.h."""
    import torch

    B, H, Nq, Nkv, d = _check_tensors(q, k, v, o, same_n=False)
    lse_ptr = None
    if lse is not None:
        if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or not lse.is_cuda:
            raise TypeError("lse must be a float32 CUDA tensor")
        if not lse.is_contiguous() or tuple(lse.shape) != (B, H, Nq):
            raise ValueError("lse must be a contiguous [B, H, Nq] tensor")
        lse_ptr = lse.data_ptr()
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = lib().attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_ptr, B, H, Nq, Nkv, d,
                           float(scale), int(mask_mode), _params_ptr(params), ws_ptr, ws_bytes,
                           _stream_handle(stream, q.device))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd_ex")


def attn_fwd_ex_static(q, k, v, o, lse=None, scale=1.0, mask_mode=ATTN_MASK_NONE, params=None, stream=None) -> None:
    """attn_fwd_ex with the library's static device scratch as its workspace: allocates nothing.
    Calls that overlap on one device race for the scratch. See include/attn.h."""
    import torch

    B, H, Nq, Nkv, d = _check_tensors(q, k, v, o, same_n=False)
    lse_ptr = None
    if lse is not None:
        if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or not lse.is_cuda:
            raise TypeError("lse must be a float32 CUDA tensor")
        if not lse.is_contiguous() or tuple(lse.shape) != (B, H, Nq):
            raise ValueError("lse must be a contiguous [B, H, Nq] tensor")
        lse_ptr = lse.data_ptr()
    rc = lib().attn_fwd_ex_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_ptr, B, H, Nq, Nkv, d,
                                  float(scale), int(mask_mode), _params_ptr(params), _stream_handle(stream, q.device))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_fwd_ex_static")


def attn_bwd_workspace_size(B, H, Nq, Nkv, d, mask_mode=ATTN_MASK_NONE, params=None) -> int:
    """Bytes of workspace attn_bwd needs (float32 row sums, B * H * Nq * 4)."""
    out = ctypes.c_uint64(0)
    rc = lib().attn_bwd_workspace_size(B, H, Nq, Nkv, d, int(mask_mode), _params_ptr(params), ctypes.byref(out))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_bwd_workspace_size")
    return int(out.value)


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, scale, mask_mode=ATTN_MASK_NONE, params=None, workspace=None,
             stream=None) -> None:
    """Gradients dq, dk, dv (bfloat16 CUDA tensors shaped like q, k, v) of attn_fwd_ex's output o for the
    output gradient dout, from the forward's logsumexp lse (float32 [B, H, Nq]); see include/attn.h."""
    import torch

    B, H, Nq, Nkv, d = _check_tensors(q, k, v, o, same_n=False)
    for name, t, like in (("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bfloat16 CUDA tensor")
        if t.shape != like.shape:
            raise ValueError(f"{name} must be shaped like {'q' if like is q else ('k' if like is k else 'v')}")
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() \
            or tuple(lse.shape) != (B, H, Nq):
        raise TypeError("lse must be a contiguous float32 CUDA tensor [B, H, Nq]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Nq, Nkv, d, float(scale), int(mask_mode),
                        _params_ptr(params), ws_ptr, ws_bytes, _stream_handle(stream, q.device))
    if rc != ATTN_OK:
        raise AttnError(rc, "attn_bwd")


_workspaces: dict = {}


def workspace(nbytes: int, device=None, stream=None):
    """A uint8 device tensor of at least nbytes, cached per (device, stream).

    Calls that use one workspace must not overlap, so each stream gets its own.
    """
    import torch

    if nbytes <= 0:
        return None
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    key = (dev.index, int(s.cuda_stream))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(s):
            ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def attention(q, k, v, scale=None, causal=False, na=None, stream=None, return_lse=False):
    """Allocate the output (and the logsumexp when return_lse) and run attn_fwd_ex with a cached
    workspace. q is [B, H, Nq, d], k and v [B, H, Nkv, d]; scale defaults to 1/sqrt(d).

    na: an attn_na2d_params_t or attn_na3d_params_t for a neighbourhood window.
    """
    import torch

    if causal and na is not None:
        raise ValueError("choose causal or a neighbourhood window, not both")
    o = torch.empty_like(q)
    if na is None:
        mode = ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE
    else:
        mode = ATTN_MASK_NA3D if isinstance(na, attn_na3d_params_t) else ATTN_MASK_NA2D
    s = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device=q.device) if return_lse else None
    with torch.cuda.device(q.device):
        ts = torch.cuda.current_stream(q.device) if stream is None else torch.cuda.ExternalStream(stream)
        ws = workspace(attn_fwd_ex_workspace_size(B, H, Nq, Nkv, d, mode, na), q.device, ts)
        attn_fwd_ex(q, k, v, o, lse, s, mode, na, ws, ts.cuda_stream)
    return (o, lse) if return_lse else o


__all__ = [
    "ATTN_MASK_NONE", "ATTN_MASK_CAUSAL", "ATTN_MASK_NA2D", "ATTN_MASK_NA3D", "attn_na3d_params_t", "na3d_params",
    "attn_fwd_ex", "attn_fwd_ex_workspace_size", "attn_fwd_ex_check", "attn_bwd", "attn_bwd_workspace_size",
    "ATTN_OK", "ATTN_ERR_INVALID_ARG", "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_PARAMS", "ATTN_ERR_ALIGNMENT",
    "ATTN_ERR_HIP", "ATTN_ERR_WORKSPACE", "AttnError", "attn_na2d_params_t", "na2d_params",
    "attn_fwd", "attn_fwd_ws", "attn_fwd_workspace_size", "workspace", "attn_fwd_check", "attn_status_string",
    "attn_abi_version", "attention", "LIB_PATH",
]
