"""Fused scaled-dot-product attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/sdpa.h`` (``libsdpa07.so``,
built in-tree by ``scaled_dot_product_07_amd.build``). Every step of the
computation runs in the library's HIP kernels; this module only checks
Python-level shapes, allocates outputs with torch (device memory plumbing),
and passes pointers, strides and the current HIP stream across the ABI.

If the library has not been built, importing works but every call raises
``RuntimeError``: there is no fallback path.

Entry points (same names as the C ABI, minus the ``sdpa_`` prefix; the
``_ex`` variants of the ABI are reached through the keyword options):
  fwd(q, k, v, ...)                       dense forward, returns (o, lse)
  fwd_varlen(q, k, v, cu_q, cu_kv, ...)   packed THD forward, returns (o, lse)
  bwd(q, k, v, o, dout, lse, ...)         dense backward, returns (dq, dk, dv)
  bwd_varlen(q, k, v, o, dout, lse, cu_q, cu_kv, ...)
                                          packed THD backward, returns (dq, dk, dv)
  fwd_fp8(q, k, v, ...), fwd_fp8_varlen(q, k, v, cu_q, cu_kv, ...)
                                          e4m3 inputs with per-tensor descales,
                                          bf16/fp16 output, returns (o, lse)
Options: grouped-query heads (k, v with fewer heads than q), causal,
bottom_right (diagonal aligned to the bottom-right corner), window_left.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = ["fwd", "fwd_varlen", "fwd_fp8", "fwd_fp8_varlen", "bwd", "bwd_noalloc",
           "bwd_varlen", "bwd_workspace_size", "last_error", "version",
           "library_path", "SdpaError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# SDPA07_LIBRARY names another build of the library (e.g. one whose host code
# carries sanitizers); by default the in-tree build next to this file
_LIB_PATH = os.environ.get("SDPA07_LIBRARY") or os.path.join(_HERE, "libsdpa07.so")

SDPA_OK, SDPA_ERR_INVALID_ARG, SDPA_ERR_UNSUPPORTED, SDPA_ERR_LAUNCH = 0, 1, 2, 3
_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_FP8 = torch.float8_e4m3fn

_lib = None


class SdpaError(RuntimeError):
    """A launch failure reported by the library."""


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m scaled_dot_product_07_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    S4 = ctypes.c_int64 * 4
    S3 = ctypes.c_int64 * 3
    lib.sdpa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, S4, S4, S4, S4, F, I, P]
    lib.sdpa_fwd_ex.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, S4, S4, S4, S4, F, I, I, I,
                                P]
    lib.sdpa_fwd_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                    S3, S3, S3, S3, F, I, P]
    lib.sdpa_fwd_varlen_ex.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I,
                                       S3, S3, S3, S3, F, I, I, I, P]
    lib.sdpa_fwd_fp8.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                 S4, S4, S4, S4, F, I, I, I, P]
    lib.sdpa_fwd_fp8_varlen.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                        I, I, S3, S3, S3, S3, F, I, I, I, P]
    lib.sdpa_bwd_workspace_size.argtypes = [I, I, I, I, I]
    lib.sdpa_bwd_workspace_size.restype = Z
    lib.sdpa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, Z, I, I, I, I, I, I,
                             S4, S4, S4, S4, S4, S4, S4, S4, F, I, P]
    lib.sdpa_bwd_ex.argtypes = [P, P, P, P, P, P, P, P, P, P, Z, I, I, I, I, I, I, I,
                                S4, S4, S4, S4, S4, S4, S4, S4, F, I, I, I, P]
    lib.sdpa_bwd_ex_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                        S4, S4, S4, S4, S4, S4, S4, S4, F, I, I, I, P]
    lib.sdpa_bwd_varlen.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, P, Z, I, I,
                                    I, I, S3, S3, S3, S3, S3, S3, S3, S3, F, I, I, I, P]
    for f in ("sdpa_fwd", "sdpa_fwd_ex", "sdpa_fwd_varlen", "sdpa_fwd_varlen_ex", "sdpa_bwd",
              "sdpa_bwd_ex", "sdpa_bwd_ex_noalloc", "sdpa_bwd_varlen", "sdpa_fwd_fp8",
              "sdpa_fwd_fp8_varlen"):
        getattr(lib, f).restype = I
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return _load().sdpa_last_error().decode()


def version() -> str:
    return _load().sdpa_version().decode()


def _check(status: int) -> None:
    if status == SDPA_OK:
        return
    msg = last_error()
    if status == SDPA_ERR_INVALID_ARG:
        raise ValueError(msg)
    if status == SDPA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise SdpaError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(t: torch.Tensor, n: int):
    return (ctypes.c_int64 * n)(*t.stride())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE_CODE:
        raise NotImplementedError(f"dtype {t.dtype} (supported: float32, float16, bfloat16)")
    return _DTYPE_CODE[t.dtype]


def _on_one_gpu(**named) -> None:
    """Every tensor argument (None skipped) must live on one and the same GPU:
    the library dereferences all of them on the device."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (found it on {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _shape_like(name: str, t: Optional[torch.Tensor], ref: torch.Tensor) -> None:
    if t is not None and tuple(t.shape) != tuple(ref.shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(ref.shape)}")


def _same_dtype(*ts):
    dt = ts[0].dtype
    for t in ts[1:]:
        if t is not None and t.dtype != dt:
            raise ValueError(f"all io tensors must share one dtype ({dt} vs {t.dtype})")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
        causal: bool = False, bottom_right: bool = False, window_left: int = -1,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        return_lse: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Dense forward on logical (b, h, s, d) tensors of any strides (d stride 1).

    k, v may have fewer heads than q (grouped-query attention; h a multiple of
    h_kv). Returns (o, lse): o like q (same strides when q is dense), lse fp32
    (b, h, s_q). scale defaults to 1/sqrt(d); causal is top-left unless
    bottom_right; window_left -1 means no left bound.
    """
    lib = _load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("dense path expects 4-D (b, h, s, d) tensors")
    b, h, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (b, h_kv, s_kv, d) or tuple(v.shape) != (b, h_kv, s_kv, d):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    _on_one_gpu(q=q, k=k, v=v, out=out, lse=lse)
    _shape_like("out", out, q)
    _same_dtype(q, k, v, out)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((b, h, s_q), device=q.device, dtype=torch.float32)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (b, h, s_q)):
        raise ValueError("lse must be a contiguous float32 (b, h, s_q) tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.sdpa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q),
                         b, h, h_kv, s_q, s_kv, d, _strides(q, 4), _strides(k, 4),
                         _strides(v, 4), _strides(out, 4), scale, int(bool(causal)),
                         int(bool(bottom_right)), int(window_left), _stream(stream))
    _check(st)
    return out, lse


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
               cu_seqlens_kv: torch.Tensor, max_seqlen_q: int, max_seqlen_kv: int, *,
               total_q: Optional[int] = None, total_kv: Optional[int] = None,
               scale: Optional[float] = None, causal: bool = False, bottom_right: bool = False,
               window_left: int = -1, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, return_lse: bool = True, stream=None):
    """Packed THD forward: q (T_q, h, d), k/v (T_kv, h_kv, d), int32 cu_seqlens on the device.

    total_q / total_kv default to the tensors' first dims (rows beyond them are
    never touched). Returns (o, lse) with lse fp32 (T_q, h) token-major.
    """
    lib = _load()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("packed path expects (T, h, d) tensors")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_kv.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.shape != cu_seqlens_kv.shape or cu_seqlens_q.dim() != 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must be 1-D of the same length")
    if not (cu_seqlens_q.is_contiguous() and cu_seqlens_kv.is_contiguous()):
        raise ValueError("cu_seqlens must be contiguous")
    t_q, h, d = q.shape
    t_kv, h_kv = k.shape[0], k.shape[1]
    if k.shape[2] != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k, v")
    _on_one_gpu(q=q, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_kv=cu_seqlens_kv, out=out,
                lse=lse)
    _shape_like("out", out, q)
    _same_dtype(q, k, v, out)
    total_q = t_q if total_q is None else int(total_q)
    total_kv = t_kv if total_kv is None else int(total_kv)
    if total_q > t_q or total_kv > t_kv:
        raise ValueError("total_q/total_kv exceed the tensors' first dimension")
    n = cu_seqlens_q.shape[0] - 1
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((t_q, h), device=q.device, dtype=torch.float32)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.shape[1:] != (h,) or lse.shape[0] < total_q):
        raise ValueError("lse must be a contiguous float32 (T_q, h) tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.sdpa_fwd_varlen_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), n, total_q, total_kv,
                                int(max_seqlen_q), int(max_seqlen_kv), _dtype_code(q), h, h_kv,
                                d, _strides(q, 3), _strides(k, 3), _strides(v, 3),
                                _strides(out, 3), scale, int(bool(causal)),
                                int(bool(bottom_right)), int(window_left), _stream(stream))
    _check(st)
    return out, lse


def bwd_workspace_size(b: int, h: int, s_q: int, d: int, dtype: torch.dtype) -> int:
    return int(_load().sdpa_bwd_workspace_size(b, h, s_q, d, _DTYPE_CODE[dtype]))


def bwd(q, k, v, o, dout, lse, *, scale: Optional[float] = None, causal: bool = False,
        bottom_right: bool = False, window_left: int = -1, dq=None, dk=None, dv=None,
        workspace=None, stream=None):
    """Dense backward. Returns (dq, dk, dv), each shaped and strided like q, k, v by default.

    The mask options must be those of the forward that produced o and lse; k, v
    may have fewer heads than q (dk, dv then sum over each head group).
    """
    lib = _load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("dense path expects 4-D (b, h, s, d) tensors")
    b, h, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if tuple(k.shape) != (b, h_kv, s_kv, d) or tuple(v.shape) != (b, h_kv, s_kv, d):
        raise ValueError("k/v shape mismatch")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (b, h, s_q):
        raise ValueError("lse must be a contiguous float32 (b, h, s_q) tensor")
    _on_one_gpu(q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, workspace=workspace)
    _shape_like("dq", dq, q)
    _shape_like("dk", dk, k)
    _shape_like("dv", dv, v)
    _same_dtype(q, k, v, o, dout, dq, dk, dv)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = bwd_workspace_size(b, h, s_q, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.sdpa_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                         _ptr(dk), _ptr(dv), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _dtype_code(q), b, h,
                         h_kv, s_q, s_kv, d, _strides(q, 4), _strides(k, 4), _strides(v, 4),
                         _strides(o, 4), _strides(dout, 4), _strides(dq, 4), _strides(dk, 4),
                         _strides(dv, 4), scale, int(bool(causal)), int(bool(bottom_right)),
                         int(window_left), _stream(stream))
    _check(st)
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, *, scale: Optional[float] = None,
                causal: bool = False, bottom_right: bool = False, window_left: int = -1,
                stream=None):
    """Dense backward into the caller's dq, dk, dv, with the library's fixed
    per-device workspace instead of one passed in (sdpa_bwd_ex_noalloc): no
    device memory is allocated, here or in the library. Calls that overlap on
    one device race on that workspace. Returns (dq, dk, dv)."""
    lib = _load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("dense path expects 4-D (b, h, s, d) tensors")
    b, h, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if tuple(k.shape) != (b, h_kv, s_kv, d) or tuple(v.shape) != (b, h_kv, s_kv, d):
        raise ValueError("k/v shape mismatch")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (b, h, s_q):
        raise ValueError("lse must be a contiguous float32 (b, h, s_q) tensor")
    if dq is None or dk is None or dv is None:
        raise ValueError("bwd_noalloc writes into caller-provided dq, dk and dv")
    _on_one_gpu(q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv)
    _shape_like("dq", dq, q)
    _shape_like("dk", dk, k)
    _shape_like("dv", dv, v)
    _same_dtype(q, k, v, o, dout, dq, dk, dv)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.sdpa_bwd_ex_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(q), b, h, h_kv, s_q,
                                 s_kv, d, _strides(q, 4), _strides(k, 4), _strides(v, 4),
                                 _strides(o, 4), _strides(dout, 4), _strides(dq, 4),
                                 _strides(dk, 4), _strides(dv, 4), scale, int(bool(causal)),
                                 int(bool(bottom_right)), int(window_left), _stream(stream))
    _check(st)
    return dq, dk, dv


def bwd_varlen(q, k, v, o, dout, lse, cu_seqlens_q: torch.Tensor, cu_seqlens_kv: torch.Tensor,
               max_seqlen_q: int, max_seqlen_kv: int, *, total_q: Optional[int] = None,
               total_kv: Optional[int] = None, scale: Optional[float] = None,
               causal: bool = False, bottom_right: bool = False, window_left: int = -1,
               dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Packed THD backward: q, o, dout (T_q, h, d), k, v (T_kv, h_kv, d), lse fp32
    (T_q, h) token-major from fwd_varlen, int32 cu_seqlens on the device.

    Returns (dq, dk, dv) shaped like q, k, v; rows past total_q / total_kv are
    left untouched.
    """
    lib = _load()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("packed path expects (T, h, d) tensors")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_kv.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.shape != cu_seqlens_kv.shape or cu_seqlens_q.dim() != 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must be 1-D of the same length")
    if not (cu_seqlens_q.is_contiguous() and cu_seqlens_kv.is_contiguous()):
        raise ValueError("cu_seqlens must be contiguous")
    t_q, h, d = q.shape
    t_kv, h_kv = k.shape[0], k.shape[1]
    if k.shape[2] != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k, v")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    _on_one_gpu(q=q, k=k, v=v, o=o, dout=dout, lse=lse, cu_seqlens_q=cu_seqlens_q,
                cu_seqlens_kv=cu_seqlens_kv, dq=dq, dk=dk, dv=dv, workspace=workspace)
    _shape_like("dq", dq, q)
    _shape_like("dk", dk, k)
    _shape_like("dv", dv, v)
    _same_dtype(q, k, v, o, dout, dq, dk, dv)
    total_q = t_q if total_q is None else int(total_q)
    total_kv = t_kv if total_kv is None else int(total_kv)
    if total_q > t_q or total_kv > t_kv:
        raise ValueError("total_q/total_kv exceed the tensors' first dimension")
    if (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.dim() != 2
            or lse.shape[1] != h or lse.shape[0] < total_q):
        raise ValueError("lse must be a contiguous float32 (T_q, h) tensor")
    n = cu_seqlens_q.shape[0] - 1
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = bwd_workspace_size(1, h, total_q, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.sdpa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens_q),
                             _ptr(cu_seqlens_kv), n, total_q, total_kv, int(max_seqlen_q),
                             int(max_seqlen_kv), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _dtype_code(q), h,
                             h_kv, d, _strides(q, 3), _strides(k, 3), _strides(v, 3),
                             _strides(o, 3), _strides(dout, 3), _strides(dq, 3),
                             _strides(dk, 3), _strides(dv, 3), scale, int(bool(causal)),
                             int(bool(bottom_right)), int(window_left), _stream(stream))
    _check(st)
    return dq, dk, dv


def _scalar_ptr(t, name):
    """A one-element fp32 device tensor (or None) as a pointer."""
    if t is None:
        return None
    if t.dtype != torch.float32 or t.numel() != 1:
        raise ValueError(f"{name} must be a one-element float32 tensor")
    return _ptr(t)


def _fp8_common(q, k, v, out_dtype, descale_q, descale_k, descale_v, scale_o, amax_o):
    for t in (q, k, v):
        if t.dtype != _FP8:
            raise ValueError("fp8 path expects torch.float8_e4m3fn q, k, v")
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise NotImplementedError("fp8 forward writes bfloat16 or float16 output")
    return [_scalar_ptr(descale_q, "descale_q"), _scalar_ptr(descale_k, "descale_k"),
            _scalar_ptr(descale_v, "descale_v"), _scalar_ptr(scale_o, "scale_o"),
            _scalar_ptr(amax_o, "amax_o")]


def fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
            causal: bool = False, bottom_right: bool = False, window_left: int = -1,
            descale_q=None, descale_k=None, descale_v=None, scale_o=None, amax_o=None,
            out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, return_lse: bool = True, stream=None):
    """Dense FP8 forward: q, k, v float8_e4m3fn of logical shape (b, h, s, d).

    descale_* / scale_o: one-element float32 device tensors (None = 1), read by
    the kernel; amax_o: a one-element float32 device tensor that receives
    max |o| before the cast. Returns (o, lse) with o in out_dtype.
    """
    lib = _load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("dense path expects 4-D (b, h, s, d) tensors")
    b, h, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (b, h_kv, s_kv, d) or tuple(v.shape) != (b, h_kv, s_kv, d):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    _on_one_gpu(q=q, k=k, v=v, out=out, lse=lse, descale_q=descale_q, descale_k=descale_k,
                descale_v=descale_v, scale_o=scale_o, amax_o=amax_o)
    extras = _fp8_common(q, k, v, out_dtype, descale_q, descale_k, descale_v, scale_o, amax_o)
    if out is None:
        out = torch.empty(q.shape, device=q.device, dtype=out_dtype)
    if out.dtype != out_dtype or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape and out_dtype")
    if lse is None and return_lse:
        lse = torch.empty((b, h, s_q), device=q.device, dtype=torch.float32)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (b, h, s_q)):
        raise ValueError("lse must be a contiguous float32 (b, h, s_q) tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.sdpa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), *extras,
                          _DTYPE_CODE[out_dtype], b, h, h_kv, s_q, s_kv, d, _strides(q, 4),
                          _strides(k, 4), _strides(v, 4), _strides(out, 4), scale,
                          int(bool(causal)), int(bool(bottom_right)), int(window_left),
                          _stream(stream))
    _check(st)
    return out, lse


def fwd_fp8_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                   cu_seqlens_kv: torch.Tensor, max_seqlen_q: int, max_seqlen_kv: int, *,
                   total_q: Optional[int] = None, total_kv: Optional[int] = None,
                   scale: Optional[float] = None, causal: bool = False,
                   bottom_right: bool = False, window_left: int = -1, descale_q=None,
                   descale_k=None, descale_v=None, scale_o=None, amax_o=None,
                   out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, return_lse: bool = True, stream=None):
    """Packed THD FP8 forward: q (T_q, h, d), k/v (T_kv, h_kv, d) float8_e4m3fn, int32
    cu_seqlens on the device; the fp8 arguments as in fwd_fp8. Returns (o, lse) with lse
    (T_q, h) token-major."""
    lib = _load()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("packed path expects (T, h, d) tensors")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_kv.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.shape != cu_seqlens_kv.shape or cu_seqlens_q.dim() != 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must be 1-D of the same length")
    if not (cu_seqlens_q.is_contiguous() and cu_seqlens_kv.is_contiguous()):
        raise ValueError("cu_seqlens must be contiguous")
    t_q, h, d = q.shape
    t_kv, h_kv = k.shape[0], k.shape[1]
    if k.shape[2] != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k, v")
    _on_one_gpu(q=q, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_kv=cu_seqlens_kv, out=out,
                lse=lse, descale_q=descale_q, descale_k=descale_k, descale_v=descale_v,
                scale_o=scale_o, amax_o=amax_o)
    extras = _fp8_common(q, k, v, out_dtype, descale_q, descale_k, descale_v, scale_o, amax_o)
    total_q = t_q if total_q is None else int(total_q)
    total_kv = t_kv if total_kv is None else int(total_kv)
    if total_q > t_q or total_kv > t_kv:
        raise ValueError("total_q/total_kv exceed the tensors' first dimension")
    n = cu_seqlens_q.shape[0] - 1
    if out is None:
        out = torch.empty(q.shape, device=q.device, dtype=out_dtype)
    if out.dtype != out_dtype or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape and out_dtype")
    if lse is None and return_lse:
        lse = torch.empty((t_q, h), device=q.device, dtype=torch.float32)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.shape[1:] != (h,) or lse.shape[0] < total_q):
        raise ValueError("lse must be a contiguous float32 (T_q, h) tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.sdpa_fwd_fp8_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), *extras,
                                 _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), n, total_q, total_kv,
                                 int(max_seqlen_q), int(max_seqlen_kv), _DTYPE_CODE[out_dtype],
                                 h, h_kv, d, _strides(q, 3), _strides(k, 3), _strides(v, 3),
                                 _strides(out, 3), scale, int(bool(causal)),
                                 int(bool(bottom_right)), int(window_left), _stream(stream))
    _check(st)
    return out, lse
