"""Oracle: plain fp64 CPU scaled-dot-product attention. TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never imports it and
shares no code with it.

The arithmetic lives in ``oracle.cpp`` (see its header for the sources on the
pages and the readings taken). This module only marshals numpy float64
arrays into that library through ctypes and builds it with g++ when it is
missing.

Parity pins (tests/test_oracle_pins*.py) tie every function here to something
other than itself: torch's CPU attention in float64 (the pages' own check),
closed forms, invariants, finite differences and a hand-worked golden case;
the FP8 decoder is pinned to torch's float8_e4m3fn conversion and to the
format's defining values.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
# ORACLE_LIBRARY names another build of oracle.cpp (the sanitizer test uses it)
_LIB = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (IEEE math, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        D = ctypes.c_double
        I = ctypes.c_int
        lib.oracle_hardware_threads.restype = I
        lib.oracle_attn_rows.argtypes = [P, P, I64, P, P, I64, I64, D, I, P, P, I]
        lib.oracle_attn_rows_ex.argtypes = [P, P, I64, I64, P, P, I64, I64, D, I, I, I64, P, P,
                                            I]
        lib.oracle_fwd_ex.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, D, I, I, I64, P, P,
                                      I]
        lib.oracle_fwd_varlen_ex.argtypes = [P, P, P, P, P, I64, I64, I64, I64, D, I, I, I64, P,
                                             P, I]
        lib.oracle_bwd_ex.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, D, I, I, I64, P,
                                      P, P, P, P, I]
        lib.oracle_bwd_varlen_ex.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, D, I, I, I64,
                                             P, P, P, P, P, I]
        lib.oracle_e4m3_decode.argtypes = [P, I64, P]
        for f in ("oracle_e4m3_decode", "oracle_attn_rows", "oracle_attn_rows_ex", "oracle_fwd_ex",
                  "oracle_fwd_varlen_ex", "oracle_bwd_ex", "oracle_bwd_varlen_ex"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def hardware_threads() -> int:
    return int(_load().oracle_hardware_threads())


def _f64(a) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _mask(causal, bottom_right, window_left):
    """Mask options as the oracle takes them (see oracle.cpp for their reading)."""
    return int(bool(causal)), int(bool(bottom_right)), int(-1 if window_left is None else
                                                          window_left)


def fwd(q, k, v, scale: float, causal: bool, threads: int = 0, *, bottom_right: bool = False,
        window_left: int = -1):
    """Dense forward. q [b,h_q,s_q,d], k/v [b,h_kv,s_kv,d] (h_q a multiple of h_kv)
    -> (o [b,h_q,s_q,d], lse [b,h_q,s_q])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, h, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    assert k.shape == (b, h_kv, s_kv, d) and v.shape == k.shape and h % h_kv == 0
    o = np.zeros((b, h, s_q, d))
    lse = np.zeros((b, h, s_q))
    _load().oracle_fwd_ex(_ptr(q), _ptr(k), _ptr(v), b, h, h_kv, s_q, s_kv, d, float(scale),
                          *_mask(causal, bottom_right, window_left), _ptr(o), _ptr(lse),
                          int(threads))
    return o, lse


def attn_rows(q_rows, q_pos, k, v, scale: float, causal: bool, threads: int = 0, *,
              s_q: int = 0, bottom_right: bool = False, window_left: int = -1):
    """Selected rows of one head. q_rows [n,d] at positions q_pos [n] of a problem with
    s_q query rows (needed for bottom-right alignment); k/v [s_kv,d]."""
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    pos = np.ascontiguousarray(np.asarray(q_pos, dtype=np.int64))
    n, d = q_rows.shape
    s_kv = k.shape[0]
    assert pos.shape == (n,) and k.shape == (s_kv, d) and v.shape == (s_kv, d)
    assert not bottom_right or s_q > 0
    o = np.zeros((n, d))
    lse = np.zeros((n,))
    _load().oracle_attn_rows_ex(_ptr(q_rows), _ptr(pos), n, int(s_q), _ptr(k), _ptr(v), s_kv, d,
                                float(scale), *_mask(causal, bottom_right, window_left), _ptr(o),
                                _ptr(lse), int(threads))
    return o, lse


def fwd_varlen(q, k, v, cu_q, cu_kv, scale: float, causal: bool, threads: int = 0, *,
               bottom_right: bool = False, window_left: int = -1):
    """Packed THD forward. q [T_q,h_q,d], k/v [T_kv,h_kv,d], cu_* [n+1]
    -> (o [T_q,h_q,d], lse [T_q,h_q])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu_q, cu_kv = _i32(cu_q), _i32(cu_kv)
    n = cu_q.shape[0] - 1
    t_q, h, d = q.shape
    h_kv = k.shape[1]
    assert cu_kv.shape == cu_q.shape and cu_q[-1] <= t_q and cu_kv[-1] <= k.shape[0]
    assert v.shape == k.shape and h % h_kv == 0
    o = np.zeros((t_q, h, d))
    lse = np.zeros((t_q, h))
    _load().oracle_fwd_varlen_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_q), _ptr(cu_kv), n, h, h_kv,
                                 d, float(scale), *_mask(causal, bottom_right, window_left),
                                 _ptr(o), _ptr(lse), int(threads))
    return o, lse


def bwd(q, k, v, dout, scale: float, causal: bool, threads: int = 0, *,
        bottom_right: bool = False, window_left: int = -1):
    """Dense backward with the oracle's own forward (heads as in fwd).

    Returns (o, lse, dq, dk, dv), all float64, BHSD / [b,h_q,s_q].
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    b, h, s_q, d = q.shape
    h_kv, s_kv = k.shape[1], k.shape[2]
    assert dout.shape == q.shape and k.shape == v.shape == (b, h_kv, s_kv, d) and h % h_kv == 0
    o = np.zeros_like(q)
    lse = np.zeros((b, h, s_q))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    _load().oracle_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), b, h, h_kv, s_q, s_kv, d,
                          float(scale), *_mask(causal, bottom_right, window_left), _ptr(o),
                          _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), int(threads))
    return o, lse, dq, dk, dv


def bwd_varlen(q, k, v, dout, cu_q, cu_kv, scale: float, causal: bool, threads: int = 0, *,
               bottom_right: bool = False, window_left: int = -1):
    """Packed THD backward with the oracle's own forward. Returns (o, lse, dq, dk, dv)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    cu_q, cu_kv = _i32(cu_q), _i32(cu_kv)
    n = cu_q.shape[0] - 1
    t_q, h, d = q.shape
    h_kv = k.shape[1]
    assert v.shape == k.shape and h % h_kv == 0
    o = np.zeros_like(q)
    lse = np.zeros((t_q, h))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    _load().oracle_bwd_varlen_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(cu_q), _ptr(cu_kv),
                                 n, h, h_kv, d, float(scale),
                                 *_mask(causal, bottom_right, window_left), _ptr(o), _ptr(lse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), int(threads))
    return o, lse, dq, dk, dv


def e4m3_decode(codes) -> np.ndarray:
    """FP8 E4M3 codes (uint8, any shape) -> exact float64 values (NaN codes -> NaN)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    _load().oracle_e4m3_decode(_ptr(c), c.size, _ptr(out))
    return out


def _fp8_inputs(q8, k8, v8, descale_q, descale_k, descale_v):
    return (float(descale_q) * e4m3_decode(q8), float(descale_k) * e4m3_decode(k8),
            float(descale_v) * e4m3_decode(v8))


def fwd_fp8(q8, k8, v8, scale: float, causal: bool, threads: int = 0, *, descale_q=1.0,
            descale_k=1.0, descale_v=1.0, scale_o=1.0, bottom_right: bool = False,
            window_left: int = -1):
    """Per-tensor scaled FP8 forward, dense: the attention of the decoded inputs
    times their descales, its output times scale_o (cudnn-frontend PR #554 merge
    log, the per-tensor FP8 forward entry). q8 [b,h_q,s_q,d], k8/v8 [b,h_kv,s_kv,d]
    of e4m3 codes. Returns (o, lse, amax) with amax = max |o| (0 when empty).
    The method's rounding of P to e4m3 is an implementation step, not part of
    this definition."""
    q, k, v = _fp8_inputs(q8, k8, v8, descale_q, descale_k, descale_v)
    o, lse = fwd(q, k, v, scale, causal, threads, bottom_right=bottom_right,
                 window_left=window_left)
    o = o * float(scale_o)
    return o, lse, float(np.max(np.abs(o))) if o.size else 0.0


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 value (round to nearest, ties to the even code) of each
    non-negative float64 in x; values past the largest finite one (448)
    saturate to it. The value set is that of e4m3_decode over all 256 codes
    (OCP FP8 E4M3: bias 7, three mantissa bits, subnormals below 2^-6)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(x < 0) or np.any(np.isnan(x)):
        raise ValueError("e4m3_round takes non-negative finite values")
    codes = np.arange(128, dtype=np.uint8)  # the non-negative codes
    vals = e4m3_decode(codes)
    ok = np.isfinite(vals)
    vals, codes = vals[ok], codes[ok]
    order = np.argsort(vals, kind="stable")
    vals, codes = vals[order], codes[order]
    xc = np.minimum(x, vals[-1])
    hi = np.clip(np.searchsorted(vals, xc, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    dlo, dhi = xc - vals[lo], vals[hi] - xc
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    return np.where(pick_hi, vals[hi], vals[lo])


def fwd_fp8_rounded_p(q8, k8, v8, scale: float, causal: bool, lift: float = 4.0) -> np.ndarray:
    """The FP8 forward with P cast to e4m3 before the P.V product (cudnn-frontend
    PR #554 merge log, the FP8 forward entry that casts P before BMM2), at the
    plainest scale for that cast: each row's P_j = e4m3(2^(log2(e) * scale *
    (s_j - max_j s_j) + lift)), so the row's largest P is 2^lift, and
    O = sum_j P_j V_j / sum_j P_j with both sums over the same rounded P.
    Dense q8 [b,h,s_q,d], k8/v8 [b,h,s_kv,d] e4m3 codes, scale > 0, top-left
    causal band when causal; rows with no visible key are not supported."""
    q, k, v = _fp8_inputs(q8, k8, v8, 1.0, 1.0, 1.0)
    if not scale > 0:
        raise ValueError("scale must be positive")
    s = np.einsum("bhid,bhjd->bhij", q, k) * float(scale)
    if causal:
        sq, skv = s.shape[-2], s.shape[-1]
        vis = np.arange(skv)[None, :] <= np.arange(sq)[:, None]
        s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("every row needs a visible key")
    x = (s - m) * np.log2(np.e) + float(lift)
    p = np.where(np.isfinite(x), e4m3_round(np.exp2(np.where(np.isfinite(x), x, 0.0))), 0.0)
    return np.einsum("bhij,bhjd->bhid", p, v) / np.sum(p, axis=-1, keepdims=True)


def fwd_fp8_varlen(q8, k8, v8, cu_q, cu_kv, scale: float, causal: bool, threads: int = 0, *,
                   descale_q=1.0, descale_k=1.0, descale_v=1.0, scale_o=1.0,
                   bottom_right: bool = False, window_left: int = -1):
    """Packed THD form of fwd_fp8: q8 [T_q,h_q,d], k8/v8 [T_kv,h_kv,d] e4m3 codes."""
    q, k, v = _fp8_inputs(q8, k8, v8, descale_q, descale_k, descale_v)
    o, lse = fwd_varlen(q, k, v, cu_q, cu_kv, scale, causal, threads,
                        bottom_right=bottom_right, window_left=window_left)
    o = o * float(scale_o)
    return o, lse, float(np.max(np.abs(o))) if o.size else 0.0
