"""The C ABI without a GPU: the library loads, exports every declared symbol,
and every validation path returns its status and message before any HIP call.
"""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
FP32, FP16, BF16, FP8 = 0, 1, 2, 3
ALIGNED = 0x10000  # a fake 16-byte aligned device address: never dereferenced


@pytest.fixture(scope="module")
def lib():
    import scaled_dot_product_07_amd as sdpa
    return sdpa._load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(sdpa_\w+)\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("sdpa_fwd", "sdpa_fwd_ex", "sdpa_fwd_varlen", "sdpa_fwd_varlen_ex", "sdpa_bwd",
              "sdpa_bwd_ex", "sdpa_bwd_ex_noalloc", "sdpa_bwd_varlen", "sdpa_fwd_fp8",
              "sdpa_fwd_fp8_varlen", "sdpa_bwd_workspace_size", "sdpa_last_error",
              "sdpa_version"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), f"{s} not exported"


def test_version(lib):
    assert b"gfx950" in lib.sdpa_version()


def S4(*x):
    return (ctypes.c_int64 * 4)(*x)


def S3(*x):
    return (ctypes.c_int64 * 3)(*x)


def dense_st(b, h, s, d):
    return S4(h * s * d, s * d, d, 1)


def fwd(lib, q=ALIGNED, k=ALIGNED, v=ALIGNED, o=ALIGNED, lse=None, dt=BF16, b=1, h=1, sq=8,
        skv=8, d=64, st=None, scale=0.125, causal=1):
    qs = st or dense_st(b, h, sq, d)
    ks = st or dense_st(b, h, skv, d)
    return lib.sdpa_fwd(q, k, v, o, lse, dt, b, h, sq, skv, d, qs, ks, ks, qs, scale, causal,
                        None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dt=7), UNSUPPORTED, "dtype"),
    (dict(b=-1), INVALID, "negative"),
    (dict(d=96), UNSUPPORTED, "head dim"),
    (dict(d=32), UNSUPPORTED, "head dim"),
    (dict(scale=math.inf), INVALID, "scale"),
    (dict(scale=math.nan), INVALID, "scale"),
    (dict(causal=2), INVALID, "causal"),
    (dict(q=None), INVALID, "q: NULL"),
    (dict(o=None), INVALID, "o: NULL"),
    (dict(k=ALIGNED + 2), UNSUPPORTED, "16-byte"),
    (dict(st=S4(64 * 8, 64 * 8, 64, 2)), UNSUPPORTED, "innermost"),
    (dict(st=S4(64 * 8, 64 * 8, 68, 1)), UNSUPPORTED, "alignment"),
    (dict(lse=ALIGNED + 1), UNSUPPORTED, "lse"),
    (dict(b=100000, h=100000, sq=1000), INVALID, "int32"),
])
def test_fwd_validation(lib, kw, status, msg):
    assert fwd(lib, **kw) == status
    assert msg in lib.sdpa_last_error().decode()


def test_fwd_zero_sizes_return_ok_without_launch(lib):
    for kw in (dict(b=0), dict(h=0), dict(sq=0)):
        assert fwd(lib, q=None, k=None, v=None, o=None, **kw) == OK
        assert lib.sdpa_last_error() == b""


def test_fwd_fp32_needs_4_element_strides(lib):
    # fp32 rows of d=64 floats: a row stride of 68 floats keeps 16-byte alignment
    assert fwd(lib, dt=FP32, b=1, h=1, sq=0, st=S4(0, 0, 68, 1)) == OK


def varlen(lib, cu_q=ALIGNED, cu_kv=ALIGNED, n=2, tq=16, tkv=16, maxq=8, maxkv=8, dt=BF16, h=2,
           d=64, st=None, scale=0.1, causal=1, q=ALIGNED):
    s = st or S3(h * d, d, 1)
    return lib.sdpa_fwd_varlen(q, ALIGNED, ALIGNED, ALIGNED, None, cu_q, cu_kv, n, tq, tkv, maxq,
                               maxkv, dt, h, d, s, s, s, s, scale, causal, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(cu_q=None), INVALID, "cu_seqlens"),
    (dict(cu_kv=None), INVALID, "cu_seqlens"),
    (dict(maxq=0), INVALID, "max_seqlen"),
    (dict(maxkv=0), INVALID, "max_seqlen"),
    (dict(maxq=17), INVALID, "exceeds total_q"),
    (dict(n=-1), INVALID, "negative"),
    (dict(d=80), UNSUPPORTED, "head dim"),
    (dict(st=S3(2 * 64, 64, 3)), UNSUPPORTED, "innermost"),
    (dict(q=None), INVALID, "q: NULL"),
])
def test_varlen_validation(lib, kw, status, msg):
    assert varlen(lib, **kw) == status
    assert msg in lib.sdpa_last_error().decode()


def test_varlen_empty_batch_ok(lib):
    assert varlen(lib, cu_q=None, cu_kv=None, n=0) == OK
    assert varlen(lib, tq=0, maxq=0) == OK


def fwd_ex(lib, h=2, h_kv=2, causal=1, br=0, window=-1, b=1, sq=8, skv=8, d=64, q=ALIGNED,
           k=ALIGNED):
    qs = dense_st(b, h, sq, d)
    ks = dense_st(b, h_kv, skv, d)
    return lib.sdpa_fwd_ex(q, k, ALIGNED, ALIGNED, None, BF16, b, h, h_kv, sq, skv, d, qs, ks, ks,
                           qs, 0.125, causal, br, window, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(h=4, h_kv=3), INVALID, "multiple of h_kv"),
    (dict(h=2, h_kv=0), INVALID, "multiple of h_kv"),
    (dict(h_kv=-1), INVALID, "negative h_kv"),
    (dict(h=2, h_kv=4), INVALID, "multiple of h_kv"),
    (dict(br=1, causal=0, window=-1), INVALID, "bottom_right needs"),
    (dict(br=2), INVALID, "bottom_right"),
    (dict(window=-2), INVALID, "window_left"),
    (dict(causal=3), INVALID, "causal"),
])
def test_fwd_ex_validation(lib, kw, status, msg):
    assert fwd_ex(lib, **kw) == status
    assert msg in lib.sdpa_last_error().decode()


@pytest.mark.parametrize("kw", [dict(h=8, h_kv=2), dict(h=3, h_kv=1), dict(br=1, causal=1),
                                dict(br=1, causal=0, window=4), dict(window=0),
                                dict(causal=0, window=16)])
def test_fwd_ex_accepts_valid_options_without_work(lib, kw):
    # s_q = 0: every check passes and nothing is launched
    assert fwd_ex(lib, sq=0, q=None, **kw) == OK


def test_fwd_ex_checks_kv_shape_with_h_kv(lib):
    # k is validated with h_kv heads: a NULL k with keys present is reported
    assert fwd_ex(lib, h=4, h_kv=2, k=None) == INVALID
    assert "k: NULL" in lib.sdpa_last_error().decode()


def test_varlen_ex_validation(lib):
    s = S3(2 * 64, 64, 1)
    st = lib.sdpa_fwd_varlen_ex(ALIGNED, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, ALIGNED, 2, 16,
                                16, 8, 8, BF16, 4, 3, 64, s, s, s, s, 0.1, 1, 0, -1, None)
    assert st == INVALID and "multiple of h_kv" in lib.sdpa_last_error().decode()
    st = lib.sdpa_fwd_varlen_ex(ALIGNED, ALIGNED, ALIGNED, ALIGNED, None, ALIGNED, ALIGNED, 2, 16,
                                16, 8, 8, BF16, 2, 2, 64, s, s, s, s, 0.1, 0, 1, -1, None)
    assert st == INVALID and "bottom_right needs" in lib.sdpa_last_error().decode()


def test_bwd_workspace_size(lib):
    lib.sdpa_bwd_workspace_size.restype = ctypes.c_size_t
    n = lib.sdpa_bwd_workspace_size(4, 16, 2048, 128, BF16)
    assert n >= 4 * 16 * 2048 * 4 and n % 256 == 0


def bwd(lib, dt=BF16, lse=ALIGNED, ws=ALIGNED, ws_bytes=1 << 20, d=64, b=1, h=1, s=8,
        causal=1, scale=0.1):
    st = dense_st(b, h, s, d)
    P = ALIGNED
    return lib.sdpa_bwd(P, P, P, P, P, lse, P, P, P, ws, ws_bytes, dt, b, h, s, s, d,
                        st, st, st, st, st, st, st, st, scale, causal, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dt=FP32), UNSUPPORTED, "fp16 and bf16"),
    (dict(lse=None), INVALID, "lse"),
    (dict(ws=None), INVALID, "workspace"),
    (dict(ws=ALIGNED + 16), INVALID, "256-byte"),
    (dict(ws_bytes=8), INVALID, "smaller"),
    (dict(d=256), UNSUPPORTED, "head dim"),
    (dict(scale=math.inf), INVALID, "scale"),
])
def test_bwd_validation(lib, kw, status, msg):
    assert bwd(lib, **kw) == status
    assert msg in lib.sdpa_last_error().decode()


def bwd_ex(lib, h=2, h_kv=2, causal=1, br=0, window=-1, b=1, sq=8, skv=8, d=64, k=ALIGNED,
           dk=ALIGNED, ws_bytes=1 << 20, kstride=None):
    qs = dense_st(b, h, sq, d)
    ks = kstride or dense_st(b, h_kv, skv, d)
    P = ALIGNED
    return lib.sdpa_bwd_ex(P, k, P, P, P, ALIGNED, P, dk, P, ALIGNED, ws_bytes, BF16, b, h, h_kv,
                           sq, skv, d, qs, ks, ks, qs, qs, qs, ks, ks, 0.1, causal, br, window,
                           None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(h=4, h_kv=3), INVALID, "multiple of h_kv"),
    (dict(h_kv=-1), INVALID, "negative h_kv"),
    (dict(br=1, causal=0), INVALID, "bottom_right needs"),
    (dict(window=-5), INVALID, "window_left"),
    (dict(h=8, h_kv=2, k=None), INVALID, "k: NULL"),
    (dict(h=8, h_kv=2, dk=None), INVALID, "dk: NULL"),
    (dict(kstride=S4(0, 0, 1 << 24, 1)), UNSUPPORTED, "32-bit tile offsets"),
    (dict(h=4, sq=100, ws_bytes=4 * 100 * 4), INVALID, "smaller"),
])
def test_bwd_ex_validation(lib, kw, status, msg):
    assert bwd_ex(lib, **kw) == status
    assert msg in lib.sdpa_last_error().decode()


@pytest.mark.parametrize("kw", [dict(h=8, h_kv=2), dict(br=1), dict(causal=0, br=1, window=3),
                                dict(window=0)])
def test_bwd_ex_accepts_valid_options_without_work(lib, kw):
    assert bwd_ex(lib, b=0, **kw) == OK


def bwd_noalloc(lib, h=2, h_kv=2, causal=1, br=0, window=-1, b=1, sq=8, skv=8, d=64,
                dt=BF16):
    qs = dense_st(b, h, sq, d)
    ks = dense_st(b, h_kv, skv, d)
    P = ALIGNED
    return lib.sdpa_bwd_ex_noalloc(P, P, P, P, P, ALIGNED, P, P, P, dt, b, h, h_kv, sq, skv, d,
                                   qs, ks, ks, qs, qs, qs, ks, ks, 0.1, causal, br, window, None)


def test_bwd_noalloc_fixed_workspace_size_matches_the_header(lib):
    text = open(HEADER).read()
    assert "#define SDPA_BWD_FIXED_WORKSPACE_BYTES (16u << 20)" in text
    assert "#define SDPA_BWD_FIXED_WORKSPACE_ROWS (1 << 21)" in text
    # two fp32 values per query row: the largest accepted problem fills it exactly
    assert lib.sdpa_bwd_workspace_size(1, 32, 1 << 16, 64, BF16) == 16 << 20


@pytest.mark.parametrize("kw,status,msg", [
    # one 64-row group past 2^21 query rows
    (dict(h=32, sq=(1 << 16) + 2), UNSUPPORTED, "exceed the fixed workspace"),
    (dict(b=3, h=16, sq=1 << 16), UNSUPPORTED, "exceed the fixed workspace"),
    (dict(h=4, h_kv=3), INVALID, "multiple of h_kv"),
    (dict(window=-5), INVALID, "window_left"),
    (dict(dt=FP32), UNSUPPORTED, "fp16 and bf16"),
    (dict(d=96), UNSUPPORTED, "head dim"),
])
def test_bwd_noalloc_validation(lib, kw, status, msg):
    assert bwd_noalloc(lib, **kw) == status
    assert msg in lib.sdpa_last_error().decode()


@pytest.mark.parametrize("kw", [dict(b=0), dict(h=0, h_kv=0), dict(sq=0, skv=0)])
def test_bwd_noalloc_without_work_is_ok(lib, kw):
    """Nothing to compute: OK before any device lookup."""
    assert bwd_noalloc(lib, **kw) == OK


def bwd_varlen(lib, cu_q=ALIGNED, cu_kv=ALIGNED, n=2, tq=16, tkv=16, maxq=8, maxkv=8, h=2, h_kv=2,
               d=64, dt=BF16, lse=ALIGNED, ws=ALIGNED, ws_bytes=1 << 20, causal=1, br=0,
               window=-1, qst=None):
    qs = qst or S3(h * d, d, 1)
    ks = S3(h_kv * d, d, 1)
    P = ALIGNED
    return lib.sdpa_bwd_varlen(P, P, P, P, P, lse, P, P, P, cu_q, cu_kv, n, tq, tkv, maxq, maxkv,
                               ws, ws_bytes, dt, h, h_kv, d, qs, ks, ks, qs, qs, qs, ks, ks, 0.1,
                               causal, br, window, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dt=FP32), UNSUPPORTED, "fp16 and bf16"),
    (dict(cu_q=None), INVALID, "cu_seqlens"),
    (dict(cu_kv=None), INVALID, "cu_seqlens"),
    (dict(maxq=0), INVALID, "max_seqlen"),
    (dict(maxkv=0), INVALID, "max_seqlen"),
    (dict(maxq=17), INVALID, "exceeds the totals"),
    (dict(maxkv=17), INVALID, "exceeds the totals"),
    (dict(lse=None), INVALID, "lse"),
    (dict(lse=ALIGNED + 2), UNSUPPORTED, "4-byte"),
    (dict(ws=None), INVALID, "workspace"),
    (dict(ws_bytes=16 * 2 * 4), INVALID, "smaller"),
    (dict(h=6, h_kv=4), INVALID, "multiple of h_kv"),
    (dict(br=1, causal=0), INVALID, "bottom_right needs"),
    (dict(d=96), UNSUPPORTED, "head dim"),
    (dict(qst=S3(2 * 64, 64, 2)), UNSUPPORTED, "innermost"),
    (dict(n=-1), INVALID, "negative"),
])
def test_bwd_varlen_validation(lib, kw, status, msg):
    assert bwd_varlen(lib, **kw) == status
    assert msg in lib.sdpa_last_error().decode()


def test_bwd_varlen_without_work_is_ok(lib):
    assert bwd_varlen(lib, n=0, cu_q=None, cu_kv=None) == OK
    assert bwd_varlen(lib, tq=0, tkv=0, maxq=0, maxkv=0) == OK


def test_bwd_varlen_workspace_uses_token_rows(lib):
    lib.sdpa_bwd_workspace_size.restype = ctypes.c_size_t
    # (1, h, total_q) rows: 2 * 16 rows here; one 256-byte block short is refused
    need = lib.sdpa_bwd_workspace_size(1, 2, 16, 64, BF16)
    assert need == lib.sdpa_bwd_workspace_size(2, 1, 16, 64, BF16)
    assert bwd_varlen(lib, ws_bytes=need - 256) == INVALID
    assert "smaller" in lib.sdpa_last_error().decode()


def fwd_fp8(lib, out=BF16, h=2, h_kv=2, b=1, sq=8, skv=8, d=64, dq=None, amax=None, qst=None,
            causal=1, br=0, window=-1, q=ALIGNED):
    qs = qst or dense_st(b, h, sq, d)
    ks = dense_st(b, h_kv, skv, d)
    return lib.sdpa_fwd_fp8(q, ALIGNED, ALIGNED, ALIGNED, None, dq, None, None, None, amax, out,
                            b, h, h_kv, sq, skv, d, qs, ks, ks, dense_st(b, h, sq, d), 0.1,
                            causal, br, window, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(out=FP32), UNSUPPORTED, "bf16 or fp16 output"),
    (dict(out=FP8), UNSUPPORTED, "bf16 or fp16 output"),
    (dict(dq=ALIGNED + 2), UNSUPPORTED, "descale_q"),
    (dict(amax=ALIGNED + 1), UNSUPPORTED, "amax_o"),
    (dict(qst=S4(0, 0, 72, 1)), UNSUPPORTED, "16-byte"),
    (dict(h=4, h_kv=3), INVALID, "multiple of h_kv"),
    (dict(br=1, causal=0), INVALID, "bottom_right needs"),
    (dict(d=256), UNSUPPORTED, "head dim"),
    (dict(q=None), INVALID, "q: NULL"),
])
def test_fwd_fp8_validation(lib, kw, status, msg):
    assert fwd_fp8(lib, **kw) == status
    assert msg in lib.sdpa_last_error().decode()


def test_fwd_fp8_accepts_byte_strides_without_work(lib):
    # e4m3 rows of 64 bytes satisfy the 16-byte rule that would refuse 64
    # bf16 elements at a stride of 72; zero queries launch nothing
    assert fwd_fp8(lib, sq=0, q=None, h=8, h_kv=2) == OK
    assert fwd_fp8(lib, sq=0, q=None, out=FP16, qst=S4(0, 0, 80, 1)) == OK


def test_fwd_fp8_varlen_validation(lib):
    s = S3(2 * 64, 64, 1)
    st = lib.sdpa_fwd_fp8_varlen(ALIGNED, ALIGNED, ALIGNED, ALIGNED, None, None, None, None, None,
                                 None, None, ALIGNED, 2, 16, 16, 8, 8, BF16, 2, 2, 64, s, s, s, s,
                                 0.1, 1, 0, -1, None)
    assert st == INVALID and "cu_seqlens" in lib.sdpa_last_error().decode()
    st = lib.sdpa_fwd_fp8_varlen(ALIGNED, ALIGNED, ALIGNED, ALIGNED, None, None, None, None, None,
                                 None, ALIGNED, ALIGNED, 2, 16, 16, 17, 8, BF16, 2, 2, 64, s, s, s,
                                 s, 0.1, 1, 0, -1, None)
    assert st == INVALID and "exceeds total_q" in lib.sdpa_last_error().decode()
    st = lib.sdpa_fwd_fp8_varlen(ALIGNED, ALIGNED, ALIGNED, ALIGNED, None, None, None, None, None,
                                 None, None, None, 0, 0, 0, 0, 0, BF16, 2, 2, 64, s, s, s, s, 0.1, 1,
                                 0, -1, None)
    assert st == OK


def test_python_binding_maps_statuses(lib):
    import scaled_dot_product_07_amd as sdpa
    assert sdpa._check(OK) is None
    lib.sdpa_fwd(None, None, None, None, None, BF16, 1, 1, 8, 8, 96, dense_st(1, 1, 8, 96),
                 dense_st(1, 1, 8, 96), dense_st(1, 1, 8, 96), dense_st(1, 1, 8, 96), 0.1, 0, None)
    with pytest.raises(NotImplementedError):
        sdpa._check(UNSUPPORTED)
    with pytest.raises(ValueError):
        sdpa._check(INVALID)


# ---- the Python binding rejects bad tensor arguments before any launch -------

def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


def _binding_calls():
    import torch
    q, k = _cpu(1, 2, 8, 64), _cpu(1, 2, 8, 64)
    lse = _cpu(1, 2, 8, dtype=torch.float32)
    tq = _cpu(8, 2, 64)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    tl = _cpu(8, 2, dtype=torch.float32)
    f8 = torch.zeros(1, 2, 8, 64, dtype=torch.float8_e4m3fn)
    t8 = torch.zeros(8, 2, 64, dtype=torch.float8_e4m3fn)
    return {
        "fwd": lambda s: s.fwd(q, k, k),
        "fwd_varlen": lambda s: s.fwd_varlen(tq, tq, tq, cu, cu, 8, 8),
        "bwd": lambda s: s.bwd(q, k, k, q, q, lse),
        "bwd_varlen": lambda s: s.bwd_varlen(tq, tq, tq, tq, tq, tl, cu, cu, 8, 8),
        "fwd_fp8": lambda s: s.fwd_fp8(f8, f8, f8),
        "fwd_fp8_varlen": lambda s: s.fwd_fp8_varlen(t8, t8, t8, cu, cu, 8, 8),
    }


@pytest.mark.parametrize("name", sorted(_binding_calls()))
def test_binding_rejects_host_tensors(lib, name):
    """Host (CPU) tensors would be dereferenced as device addresses: refused."""
    import scaled_dot_product_07_amd as sdpa
    with pytest.raises(ValueError, match="GPU tensor"):
        _binding_calls()[name](sdpa)


def test_binding_shape_checks():
    import scaled_dot_product_07_amd as sdpa
    q = _cpu(1, 2, 8, 64)
    sdpa._shape_like("out", None, q)
    sdpa._shape_like("out", _cpu(1, 2, 8, 64), q)
    with pytest.raises(ValueError, match="out has shape"):
        sdpa._shape_like("out", _cpu(1, 2, 7, 64), q)
    with pytest.raises(ValueError, match="must be a torch.Tensor"):
        sdpa._on_one_gpu(q=3)


def test_bwd_varlen_without_keys_needs_no_forward_outputs(lib):
    """A packed batch with no keys: O, dO, the statistic and the workspace are
    not read, so NULL passes validation (the kernels only zero dQ); on a host
    without a GPU the launch itself then fails with SDPA_ERR_LAUNCH."""
    s = S3(2 * 64, 64, 1)
    st = lib.sdpa_bwd_varlen(ALIGNED, None, None, None, None, None, ALIGNED, None, None, ALIGNED,
                             ALIGNED, 2, 16, 0, 9, 0, None, 0, BF16, 2, 2, 64, s, s, s, s, s, s, s,
                             s, 0.1, 1, 0, -1, None)
    assert st in (OK, 3), lib.sdpa_last_error()
