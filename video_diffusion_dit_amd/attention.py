"""Python binding of libattn (include/attn.h): argument marshalling only.

Every step of the attention forward runs in the gfx950 HIP kernels of libattn.so. This
module checks tensor dtype/shape/device/contiguity, picks the current torch stream, and
passes raw device pointers through ctypes. There is no CPU or PyTorch fallback: if the
library is missing, every call raises.

Guard semantics follow the pages' fast-path convention (page "[sglang] SANA-Video 2.0
anchor attention ... FP32 upcast", code analysis item 1: a ``try_*`` call returns ``None``
so the caller can fall back when dtype/shape/device do not fit) and the varlen backend's
hard errors (page "PR #33702 report", risks: ValueError for a head size other than 128,
TypeError for non-BF16 input).
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

from .build import LIB_PATH

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_WORKSPACE = -3
ATTN_ERR_HIP = -4

_lib = None
_lib_lock = threading.Lock()
_workspaces: dict = {}


class AttnError(RuntimeError):
    """A libattn call returned a failure status."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"libattn status {status}: {detail}")
        self.status = status


def library_path() -> str:
    return os.environ.get("ATTN_LIBRARY", LIB_PATH)


def load_library() -> ctypes.CDLL:
    """Load libattn.so (once). Raises if it has not been built -- no fallback exists."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libattn.so not found at {path}; build it first "
                               "(python -m video_diffusion_dit_amd.build)")
        lib = ctypes.CDLL(path)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
        lib.attn_fwd.restype = i32
        lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, sz, vp]
        lib.attn_fwd_varlen.restype = i32
        lib.attn_fwd_varlen_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, sz, vp]
        lib.attn_fwd_varlen_splitkv.restype = i32
        lib.attn_fwd_varlen_splitkv_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.attn_fwd_varlen_splitkv_workspace_bytes.restype = sz
        lib.attn_fwd_varlen_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
        lib.attn_fwd_varlen_noalloc.restype = i32
        lib.attn_fwd_varlen_workspace_bytes.argtypes = [i32, i32, i32]
        lib.attn_fwd_varlen_workspace_bytes.restype = sz
        lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, sz, vp]
        lib.attn_fwd_splitkv.restype = i32
        lib.attn_fwd_splitkv_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.attn_fwd_splitkv_workspace_bytes.restype = sz
        lib.attn_status_string.argtypes = [i32]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_tile_rows.restype = i32
        lib.attn_tile_keys.restype = i32
        lib.attn_qk_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                         f32, f32, vp]
        lib.attn_qk_prologue.restype = i32
        lib.attn_qk_norm_packed.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, vp]
        lib.attn_qk_norm_packed.restype = i32
        lib.attn_linear_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, sz, vp]
        lib.attn_linear_fwd.restype = i32
        lib.attn_linear_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.attn_linear_workspace_bytes.restype = sz
        lib.attn_block_list_stride.argtypes = [i32]
        lib.attn_block_list_stride.restype = i32
        lib.attn_block_route_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.attn_block_route_workspace_bytes.restype = sz
        lib.attn_block_route.argtypes = [vp, vp, i32, i32, i32, i32, f32, f32, i32, vp, vp, vp, vp, sz, vp]
        lib.attn_block_route.restype = i32
        lib.attn_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
        lib.attn_fwd_block_sparse.restype = i32
        lib.attn_block_varlen_tiles.argtypes = [i32, i32]
        lib.attn_block_varlen_tiles.restype = i32
        lib.attn_block_route_varlen_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.attn_block_route_varlen_workspace_bytes.restype = sz
        lib.attn_block_route_varlen.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, f32, i32, vp, vp, vp, vp, sz, vp]
        lib.attn_block_route_varlen.restype = i32
        lib.attn_fwd_block_sparse_varlen_workspace_bytes.argtypes = [i32, i32, i32]
        lib.attn_fwd_block_sparse_varlen_workspace_bytes.restype = sz
        lib.attn_fwd_block_sparse_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, sz,
                                                     vp]
        lib.attn_fwd_block_sparse_varlen.restype = i32
        lib.attn_block_skip_use_dense.argtypes = [i32, i32, i32, ctypes.c_char_p]
        lib.attn_block_skip_use_dense.restype = i32
        _lib = lib
        return lib


def _raise_for(lib, status: int):
    if status == ATTN_OK:
        return
    detail = (lib.attn_last_error() or b"").decode() or lib.attn_status_string(status).decode()
    if status == ATTN_ERR_UNSUPPORTED:
        raise ValueError(f"libattn: unsupported request: {detail}")
    if status == ATTN_ERR_INVALID_ARG:
        raise ValueError(f"libattn: invalid argument: {detail}")
    raise AttnError(status, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensors(q, k, v, ndim: int):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU device")
        if t.dim() != ndim:
            raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")


def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
             return_lse: bool = False, out: torch.Tensor | None = None, split_kv: bool = True,
             slots: int = 0):
    """Dense attention forward: q, k, v BF16 [B, H, N, 128] contiguous on one GPU.

    Returns out (BF16 [B,H,N,128]) or (out, lse FP32 [B,H,N]). Launches on the current
    torch stream of q's device and returns without synchronising. With split_kv (default)
    the query tiles of the device's last, partly filled round of workgroups are split over
    their key range (attn_fwd_splitkv; ``slots`` = concurrent workgroups, 0 = the device's
    compute units); when no tile needs cutting this is the plain attn_fwd call.
    """
    _check_tensors(q, k, v, 4)
    B, H, N, d = q.shape
    if d != 128:
        raise ValueError(f"head dimension {d} is not supported (only 128)")
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's device")
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    if split_kv:
        _launch_dense_splitkv(q, k, v, out, lse, _default_scale(d, scale), slots)
    else:
        _launch_dense(q, k, v, out, lse, _default_scale(d, scale))
    return (out, lse) if return_lse else out


def _launch_dense(q, k, v, out, lse, scale: float):
    """One C-ABI call on already-checked tensors (the library validates again on the host)."""
    lib = load_library()
    B, H, N, d = q.shape
    with torch.cuda.device(q.device):
        st = lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale,
                          _stream_handle(q.device))
    _raise_for(lib, st)


def splitkv_workspace_bytes(B: int, H: int, N: int, slots: int = 0, device=None) -> int:
    """Workspace of attn_fwd_splitkv (0: nothing is split). slots <= 0 queries the device."""
    lib = load_library()
    if slots <= 0:
        with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
            return int(lib.attn_fwd_splitkv_workspace_bytes(B, H, N, 128, slots))
    return int(lib.attn_fwd_splitkv_workspace_bytes(B, H, N, 128, slots))


def _launch_dense_splitkv(q, k, v, out, lse, scale: float, slots: int = 0):
    """One attn_fwd_splitkv call on already-checked tensors, with a cached workspace."""
    lib = load_library()
    B, H, N, d = q.shape
    with torch.cuda.device(q.device):
        nbytes = int(lib.attn_fwd_splitkv_workspace_bytes(B, H, N, d, slots))
        ws = _workspace(q.device, nbytes) if nbytes > 0 else None
        st = lib.attn_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale, slots,
                                  _ptr(ws), 0 if ws is None else ws.numel(), _stream_handle(q.device))
    _raise_for(lib, st)


def try_attn_fwd(q, k, v, scale=None, return_lse=False):
    """attn_fwd, or None when the request is outside what the kernel implements (caller falls back)."""
    try:
        if not all(isinstance(t, torch.Tensor) for t in (q, k, v)):
            return None
        if not (q.is_cuda and q.dtype == k.dtype == v.dtype == torch.bfloat16 and q.dim() == 4
                and q.shape == k.shape == v.shape and q.shape[-1] == 128):
            return None
        if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
            return None
        return attn_fwd(q, k, v, scale=scale, return_lse=return_lse)
    except ValueError:
        return None


def varlen_workspace_bytes(nseg: int, H: int, total_tokens: int) -> int:
    return int(load_library().attn_fwd_varlen_workspace_bytes(nseg, H, total_tokens))


def _workspace(device, nbytes: int) -> torch.Tensor:
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def check_cu_seqlens(cu_host, total_tokens: int):
    """Validate segment offsets on the host: int32, cu[0] = 0, non-decreasing, cu[-1] = T."""
    cu = [int(x) for x in cu_host]
    if len(cu) < 2:
        raise ValueError("cu_seqlens needs at least 2 entries")
    if cu[0] != 0:
        raise ValueError("cu_seqlens[0] must be 0")
    if any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must be non-decreasing")
    if cu[-1] != total_tokens:
        raise ValueError(f"cu_seqlens[-1] = {cu[-1]} must equal the token count {total_tokens}")
    if cu[-1] > 2**31 - 1:
        raise ValueError("token count exceeds int32")
    return cu


def attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                    scale: float | None = None, return_lse: bool = False,
                    out: torch.Tensor | None = None, cu_seqlens_host=None, split_kv: bool = True,
                    slots: int = 0):
    """Packed varlen forward: q, k, v BF16 [T, H, 128] (THD), attention within each segment.

    cu_seqlens: int32 tensor [nseg + 1] on q's device. The offsets are validated on a host
    copy (``cu_seqlens_host`` if given, else copied from the device, which synchronises).
    With split_kv (default) the schedule's tail is split over keys when that shortens it
    (attn_fwd_varlen_splitkv; ``slots`` = concurrent workgroups, 0 = the device's compute
    units); otherwise the plain attn_fwd_varlen call.
    Returns out (BF16 [T,H,128]) or (out, lse FP32 [H,T]).
    """
    _check_tensors(q, k, v, 3)
    T, H, d = q.shape
    if d != 128:
        raise ValueError(f"head dimension {d} is not supported (only 128)")
    if not (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.dtype == torch.int32
            and cu_seqlens.device == q.device and cu_seqlens.dim() == 1 and cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor on q's device")
    host = cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens.cpu().tolist()
    if len(host) != cu_seqlens.numel():
        raise ValueError("cu_seqlens_host does not match cu_seqlens")
    check_cu_seqlens(host, T)
    nseg = cu_seqlens.numel() - 1
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's device")
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if return_lse else None
    if split_kv:
        _launch_varlen_splitkv(q, k, v, cu_seqlens, out, lse, _default_scale(d, scale), slots)
    else:
        _launch_varlen(q, k, v, cu_seqlens, out, lse, _default_scale(d, scale))
    return (out, lse) if return_lse else out


def _launch_varlen_splitkv(q, k, v, cu_seqlens, out, lse, scale: float, slots: int = 0):
    """One attn_fwd_varlen_splitkv call on already-checked tensors, with a cached workspace."""
    lib = load_library()
    T, H, d = q.shape
    nseg = cu_seqlens.numel() - 1
    with torch.cuda.device(q.device):
        nbytes = int(lib.attn_fwd_varlen_splitkv_workspace_bytes(nseg, H, T, d, slots))
        ws = _workspace(q.device, nbytes)
        st = lib.attn_fwd_varlen_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
                                         nseg, H, T, d, scale, slots, _ptr(ws), ws.numel(), _stream_handle(q.device))
    _raise_for(lib, st)


def _launch_varlen(q, k, v, cu_seqlens, out, lse, scale: float, cu_seqlens_host=None):
    """One C-ABI call on already-checked tensors; cu_seqlens_host, if given, is re-validated."""
    lib = load_library()
    T, H, d = q.shape
    nseg = cu_seqlens.numel() - 1
    if cu_seqlens_host is not None:
        check_cu_seqlens(cu_seqlens_host, T)
    nbytes = int(lib.attn_fwd_varlen_workspace_bytes(nseg, H, T))
    with torch.cuda.device(q.device):
        ws = _workspace(q.device, nbytes)
        st = lib.attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
                                 nseg, H, T, d, scale, _ptr(ws), ws.numel(), _stream_handle(q.device))
    _raise_for(lib, st)


def attn_fwd_varlen_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                            out: torch.Tensor, lse: torch.Tensor | None = None, scale: float | None = None):
    """attn_fwd_varlen into caller-given out (and lse), with the tile schedule in the library's
    fixed per-device scratch instead of a workspace: nothing is allocated, so the call can sit
    in code that must not allocate. Arguments are checked as attn_fwd_varlen checks them,
    except the segment offsets, which are not copied to the host here (that would synchronise):
    the caller guarantees cu_seqlens[0] = 0, non-decreasing, cu_seqlens[-1] = T. Calls that may
    overlap on one device share the scratch and must be serialised by the caller."""
    _check_tensors(q, k, v, 3)
    T, H, d = q.shape
    if not (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.dtype == torch.int32
            and cu_seqlens.device == q.device and cu_seqlens.dim() == 1 and cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor on q's device")
    if out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's device")
    if lse is not None and (lse.shape != (H, T) or lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [H, T] tensor on q's device")
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_varlen_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
                                         cu_seqlens.numel() - 1, H, T, d, _default_scale(d, scale),
                                         _stream_handle(q.device))
    _raise_for(lib, st)
    return out


def qk_prologue(xq: torch.Tensor, xk: torch.Tensor, xv: torch.Tensor | None = None, *, grid,
                weight_q: torch.Tensor | None = None, weight_k: torch.Tensor | None = None,
                eps: float = 1e-6, theta: float = 10000.0, out=None):
    """Per-head RMSNorm + interleaved 3-D RoPE of the projected Q and K, BF16, into the
    attention layout (``attn_qk_prologue`` in include/attn.h).

    xq, xk (, xv): bfloat16 [B, N, H, 128] contiguous, token-major. grid = (frames, grid_h,
    grid_w) with frames * grid_h * grid_w == N. weight_q/weight_k: float32 [128] or None.
    Returns (q, k) or (q, k, v), bfloat16 [B, H, N, 128]; `out` may hold preallocated outputs.
    """
    tensors = [("xq", xq), ("xk", xk)] + ([("xv", xv)] if xv is not None else [])
    for name, t in tensors:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor, got {tuple(t.shape)}")
        if t.shape != xq.shape or t.device != xq.device:
            raise ValueError("xq, xk and xv must have the same shape and device")
    B, N, H, d = xq.shape
    for name, w in (("weight_q", weight_q), ("weight_k", weight_k)):
        if w is not None and (w.dtype != torch.float32 or w.device != xq.device or w.numel() != d
                              or not w.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [{d}] tensor on {xq.device}")
    F, gh, gw = (int(g) for g in grid)
    if out is None:
        out = tuple(torch.empty((B, H, N, d), dtype=torch.bfloat16, device=xq.device)
                    for _ in range(len(tensors)))
    q, k = out[0], out[1]
    v = out[2] if xv is not None else None
    for t in out:
        if t.shape != (B, H, N, d) or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != xq.device:
            raise ValueError("out tensors must be contiguous bfloat16 [B, H, N, d] on the input device")
    lib = load_library()
    st = lib.attn_qk_prologue(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(weight_q), _ptr(weight_k), B, N, H, d, F, gh, gw,
                              float(eps), float(theta), _stream_handle(xq.device))
    _raise_for(lib, st)
    return tuple(out)


def qk_norm_packed(xq: torch.Tensor, xk: torch.Tensor, *, weight_q: torch.Tensor | None = None,
                   weight_k: torch.Tensor | None = None, eps: float = 1e-6, in_place: bool = False):
    """Per-head RMSNorm of packed Q and K: xq, xk BF16 [T, H, 128] (THD, the projection's own
    layout, which attn_fwd_varlen reads) -> (q, k) BF16 [T, H, 128], rounded once. Weights: FP32
    [128] or None. in_place writes into xq and xk."""
    for t in (xq, xk):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
            raise TypeError("xq and xk must be bfloat16 tensors")
    if xq.dim() != 3 or xq.shape != xk.shape or xq.shape[-1] != 128:
        raise ValueError("xq and xk must be [T, H, 128] with the same shape")
    if not (xq.is_contiguous() and xk.is_contiguous()) or xq.device != xk.device:
        raise ValueError("xq and xk must be contiguous and on one device")
    for w in (weight_q, weight_k):
        if w is not None and (w.dtype != torch.float32 or w.shape != (128,) or not w.is_contiguous()
                              or w.device != xq.device):
            raise ValueError("weights must be contiguous float32 [128] tensors on the inputs' device")
    T, H, d = xq.shape
    q, k = (xq, xk) if in_place else (torch.empty_like(xq), torch.empty_like(xk))
    lib = load_library()
    with torch.cuda.device(xq.device):
        st = lib.attn_qk_norm_packed(_ptr(xq), _ptr(xk), _ptr(q), _ptr(k), _ptr(weight_q), _ptr(weight_k), T, H, d,
                                     float(eps), _stream_handle(xq.device))
    _raise_for(lib, st)
    return q, k


def linear_attention(q: torch.Tensor, k: torch.Tensor, q_rot: torch.Tensor, k_rot: torch.Tensor,
                     v: torch.Tensor, eps: float = 1e-15, out: torch.Tensor | None = None) -> torch.Tensor:
    """SANA-Video linear attention (``attn_linear_fwd`` in include/attn.h): inputs bfloat16
    [B, N, H, 128] token-major (q, k ReLU'd; q_rot, k_rot rotated); returns bfloat16
    [B, N, H, 128]. The workspace is cached per device."""
    for name, t in (("q", q), ("k", k), ("q_rot", q_rot), ("k_rot", k_rot), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor, got {tuple(t.shape)}")
        if t.shape != q.shape or t.device != q.device:
            raise ValueError("q, k, q_rot, k_rot and v must have the same shape and device")
    B, N, H, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    lib = load_library()
    need = int(lib.attn_linear_workspace_bytes(B, N, H, d))
    ws = _workspace(q.device, need) if need else None
    st = lib.attn_linear_fwd(_ptr(q), _ptr(k), _ptr(q_rot), _ptr(k_rot), _ptr(v), _ptr(out), B, N, H, d,
                             float(eps), _ptr(ws), need, _stream_handle(q.device))
    _raise_for(lib, st)
    return out


# ---------------------------------------------------------------- block-skip attention
# Page "PR #33702 report" (the Sol-Attn backend): KV blocks routed by a threshold tau, sink
# tokens kept, a dense guard over denoising steps and layers. Query tiles are 256 rows, key
# tiles 64 keys; the routing rule is stated in include/attn.h (attn_block_route).

def block_list_stride(N: int) -> int:
    """Row stride (entries) of the kv_idx lists for N tokens: ceil(N/64) + 8."""
    return int(load_library().attn_block_list_stride(N))


def _list_shapes(B: int, H: int, N: int):
    ntq = -(-N // 256)
    return (B, H, ntq, block_list_stride(N)), (B, H, ntq)


def block_route(q: torch.Tensor, k: torch.Tensor, *, tau: float, sink_tokens: int = 0,
                scale: float | None = None, with_order: bool = False):
    """Key-tile lists of block-skip attention for dense BF16 [B, H, N, 128] q and k.

    Returns (kv_idx int32 [B, H, ntq, stride], kv_cnt int32 [B, H, ntq]) on q's device,
    written on the current stream (see attn_block_route for the rule); with with_order, also
    order int32 [B*H*ntq]: for each (b, h) in turn, its items by list length, longest first
    (the dispatch order for attn_fwd_block_sparse)."""
    _check_tensors(q, k, k, 4)
    B, H, N, d = q.shape
    if d != 128:
        raise ValueError(f"head dimension {d} is not supported (only 128)")
    lib = load_library()
    idx_shape, cnt_shape = _list_shapes(B, H, N)
    kv_idx = torch.empty(idx_shape, dtype=torch.int32, device=q.device)
    kv_cnt = torch.empty(cnt_shape, dtype=torch.int32, device=q.device)
    order = torch.empty(kv_cnt.numel(), dtype=torch.int32, device=q.device) if with_order else None
    with torch.cuda.device(q.device):
        nbytes = int(lib.attn_block_route_workspace_bytes(B, H, N, d))
        ws = _workspace(q.device, nbytes)
        st = lib.attn_block_route(_ptr(q), _ptr(k), B, H, N, d, _default_scale(d, scale), float(tau),
                                  int(sink_tokens), _ptr(kv_idx), _ptr(kv_cnt), _ptr(order), _ptr(ws), ws.numel(),
                                  _stream_handle(q.device))
    _raise_for(lib, st)
    return (kv_idx, kv_cnt, order) if with_order else (kv_idx, kv_cnt)


def _check_order(order, n: int, device):
    if order is None:
        return
    if not isinstance(order, torch.Tensor) or order.dtype != torch.int32 or order.numel() != n:
        raise ValueError(f"order must be an int32 tensor of {n} entries")
    if order.device != device or not order.is_contiguous():
        raise ValueError("order must be contiguous on q's device")


def attn_fwd_block_sparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_idx: torch.Tensor,
                          kv_cnt: torch.Tensor, scale: float | None = None, return_lse: bool = False,
                          out: torch.Tensor | None = None, order: torch.Tensor | None = None):
    """Attention of dense BF16 [B, H, N, 128] q, k, v where query tile I of (b, h) sees only
    the key tiles kv_idx[b, h, I, :kv_cnt[b, h, I]] (int32 device tensors shaped as
    block_route returns them; the caller's own lists are accepted: this is the hook). order:
    the dispatch order block_route(with_order=True) returns, or None (item order)."""
    _check_tensors(q, k, v, 4)
    B, H, N, d = q.shape
    if d != 128:
        raise ValueError(f"head dimension {d} is not supported (only 128)")
    idx_shape, cnt_shape = _list_shapes(B, H, N)
    for name, t, shape in (("kv_idx", kv_idx, idx_shape), ("kv_cnt", kv_cnt, cnt_shape)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be an int32 tensor of shape {shape}")
        if t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on q's device")
    _check_order(order, kv_cnt.numel(), q.device)
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's device")
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(kv_idx),
                                       _ptr(kv_cnt), _ptr(order), B, H, N, d, _default_scale(d, scale),
                                       _stream_handle(q.device))
    _raise_for(lib, st)
    return (out, lse) if return_lse else out


def block_skip_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, tau: float,
                         sink_tokens: int = 0, scale: float | None = None, return_lse: bool = False):
    """block_route, then attn_fwd_block_sparse over its lists in the routing's order: head by
    head, the longest lists first (8 % faster than item order on the 720p grid)."""
    kv_idx, kv_cnt, order = block_route(q, k, tau=tau, sink_tokens=sink_tokens, scale=scale, with_order=True)
    return attn_fwd_block_sparse(q, k, v, kv_idx, kv_cnt, scale=scale, return_lse=return_lse, order=order)


def block_skip_use_dense(step: int, layer: int, dense_steps: int = 0, dense_layers: str | None = None) -> bool:
    """The dense guard: True when denoising step `step` of layer `layer` runs dense
    attention (step < dense_steps, or layer in the "a-b,c" list dense_layers)."""
    lib = load_library()
    text = None if dense_layers is None else str(dense_layers).encode()
    st = lib.attn_block_skip_use_dense(int(step), int(layer), int(dense_steps), text)
    if st < 0:
        _raise_for(lib, st)
    return bool(st)


def _check_cu(q, cu_seqlens, cu_seqlens_host):
    if not (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.dtype == torch.int32
            and cu_seqlens.device == q.device and cu_seqlens.dim() == 1 and cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor on q's device")
    host = cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens.cpu().tolist()
    if len(host) != cu_seqlens.numel():
        raise ValueError("cu_seqlens_host does not match cu_seqlens")
    return check_cu_seqlens(host, q.shape[0])


def varlen_list_shapes(nseg: int, T: int, H: int):
    """(kv_idx, kv_cnt) shapes of the packed-batch lists: [tiles, H, stride], [tiles, H], with
    tiles = T // 256 + nseg (an upper bound; tile g of the numbering segment by segment)."""
    lib = load_library()
    tiles = int(lib.attn_block_varlen_tiles(nseg, T))
    return (tiles, H, block_list_stride(max(T, 1))), (tiles, H)


def varlen_tile_offsets(cu_host) -> list:
    """First query tile of each segment in the numbering segment by segment (host lists)."""
    out, acc = [], 0
    for a, e in zip(cu_host[:-1], cu_host[1:]):
        out.append(acc)
        acc += -(-(int(e) - int(a)) // 256)
    return out + [acc]


def block_route_varlen(q: torch.Tensor, k: torch.Tensor, cu_seqlens: torch.Tensor, *, tau: float,
                       sink_tokens: int = 0, scale: float | None = None, cu_seqlens_host=None,
                       with_order: bool = False):
    """Key-tile lists of block-skip attention for a packed batch (THD BF16 [T, H, 128] q, k):
    (kv_idx int32 [tiles, H, stride], kv_cnt int32 [tiles, H]); row g of the lists is query
    tile g of the numbering segment by segment (see varlen_tile_offsets). with_order adds the
    dispatch order (items g * H + h by list length, longest first)."""
    _check_tensors(q, k, k, 3)
    T, H, d = q.shape
    if d != 128:
        raise ValueError(f"head dimension {d} is not supported (only 128)")
    _check_cu(q, cu_seqlens, cu_seqlens_host)
    nseg = cu_seqlens.numel() - 1
    lib = load_library()
    idx_shape, cnt_shape = varlen_list_shapes(nseg, T, H)
    kv_idx = torch.empty(idx_shape, dtype=torch.int32, device=q.device)
    kv_cnt = torch.empty(cnt_shape, dtype=torch.int32, device=q.device)
    order = torch.empty(kv_cnt.numel(), dtype=torch.int32, device=q.device) if with_order else None
    with torch.cuda.device(q.device):
        nbytes = int(lib.attn_block_route_varlen_workspace_bytes(nseg, H, T, d))
        ws = _workspace(q.device, nbytes)
        st = lib.attn_block_route_varlen(_ptr(q), _ptr(k), _ptr(cu_seqlens), nseg, H, T, d, _default_scale(d, scale),
                                         float(tau), int(sink_tokens), _ptr(kv_idx), _ptr(kv_cnt), _ptr(order),
                                         _ptr(ws), ws.numel(), _stream_handle(q.device))
    _raise_for(lib, st)
    return (kv_idx, kv_cnt, order) if with_order else (kv_idx, kv_cnt)


def attn_fwd_block_sparse_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                                 kv_idx: torch.Tensor, kv_cnt: torch.Tensor, scale: float | None = None,
                                 return_lse: bool = False, out: torch.Tensor | None = None, cu_seqlens_host=None,
                                 order: torch.Tensor | None = None):
    """Packed-batch attention where query tile g (numbered segment by segment) of head h sees
    only the key tiles kv_idx[g, h, :kv_cnt[g, h]] of its segment (the caller's own lists are
    accepted: this is the hook). Returns out (BF16 [T, H, 128]) or (out, lse FP32 [H, T])."""
    _check_tensors(q, k, v, 3)
    T, H, d = q.shape
    if d != 128:
        raise ValueError(f"head dimension {d} is not supported (only 128)")
    _check_cu(q, cu_seqlens, cu_seqlens_host)
    nseg = cu_seqlens.numel() - 1
    idx_shape, cnt_shape = varlen_list_shapes(nseg, T, H)
    for name, t, shape in (("kv_idx", kv_idx, idx_shape), ("kv_cnt", kv_cnt, cnt_shape)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be an int32 tensor of shape {shape}")
        if t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on q's device")
    _check_order(order, kv_cnt.numel(), q.device)
    lib = load_library()
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's device")
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if return_lse else None
    with torch.cuda.device(q.device):
        nbytes = int(lib.attn_fwd_block_sparse_varlen_workspace_bytes(nseg, H, T))
        ws = _workspace(q.device, nbytes)
        st = lib.attn_fwd_block_sparse_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens),
                                              _ptr(kv_idx), _ptr(kv_cnt), _ptr(order), nseg, H, T, d,
                                              _default_scale(d, scale), _ptr(ws), ws.numel(), _stream_handle(q.device))
    _raise_for(lib, st)
    return (out, lse) if return_lse else out


def block_skip_attention_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, *,
                                tau: float, sink_tokens: int = 0, scale: float | None = None,
                                cu_seqlens_host=None, return_lse: bool = False):
    """block_route_varlen, then attn_fwd_block_sparse_varlen with the longest lists started
    first: a packed batch mixes segment lengths, so its list lengths spread widely."""
    kv_idx, kv_cnt, order = block_route_varlen(q, k, cu_seqlens, tau=tau, sink_tokens=sink_tokens, scale=scale,
                                               cu_seqlens_host=cu_seqlens_host, with_order=True)
    return attn_fwd_block_sparse_varlen(q, k, v, cu_seqlens, kv_idx, kv_cnt, scale=scale,
                                        cu_seqlens_host=cu_seqlens_host, return_lse=return_lse, order=order)
