"""GPU parity of the FP8 (e4m3) forward (sdpa_fwd_fp8, sdpa_fwd_fp8_varlen)
against the fp64 oracle on the same input codes. Tolerances and their
derivation are in tests/parity.py (the P rounding to e4m3 is the only
approximation the method adds); rows whose P is exact are checked to the
output rounding.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import announce, check_lse, check_lse_fp8, check_o_fp8, f64

pytestmark = pytest.mark.gpu

OUT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def e4m3(shape, seed, spread=1.0, layout="bhsd"):
    """float8_e4m3fn CPU tensor of rounded N(0, spread) values (logical b, h, s, d)."""
    g = torch.Generator().manual_seed(seed)
    if layout == "bhsd":
        return (torch.randn(*shape, generator=g) * spread).to(torch.float8_e4m3fn)
    b, h, s, d = shape
    return (torch.randn(b, s, h, d, generator=g) * spread).to(torch.float8_e4m3fn).transpose(1, 2)


def codes(t):
    return t.contiguous().view(torch.uint8).numpy()


def scalar(x, dev):
    return torch.tensor([x], dtype=torch.float32, device=dev)


CASES = [
    # out, b, h, h_kv, s_q, s_kv, d, causal, bottom_right, window, scale, dq, dk, dv, so
    ("bf16", 1, 2, 2, 200, 200, 64, True, False, -1, 0.125, 1.0, 1.0, 1.0, 1.0),
    ("bf16", 2, 2, 2, 300, 300, 128, False, False, -1, 0.088, 1.0, 1.0, 1.0, 1.0),
    ("fp16", 1, 2, 2, 257, 257, 128, True, False, -1, 0.088, 0.5, 2.0, 0.25, 4.0),
    ("bf16", 1, 4, 4, 190, 130, 64, True, False, -1, -0.125, 1.5, 0.75, 1.0, 1.0),
    ("bf16", 1, 2, 2, 200, 520, 64, True, True, -1, 0.125, 1.0, 1.0, 2.0, 0.5),
    ("bf16", 1, 2, 2, 520, 200, 128, True, True, -1, 0.088, 1.0, 1.0, 1.0, 1.0),
    ("fp16", 1, 2, 2, 400, 400, 64, True, False, 37, 0.125, 1.0, 1.0, 1.0, 1.0),
    ("bf16", 1, 8, 2, 333, 600, 64, True, True, 90, 0.125, 1.0, 1.0, 1.0, 1.0),
    ("bf16", 2, 6, 1, 130, 330, 128, False, False, -1, 0.088, 1.0, 1.0, 1.0, 1.0),
    ("bf16", 1, 2, 2, 300, 500, 64, False, False, 70, 0.125, 1.0, 1.0, 1.0, 1.0),
    ("bf16", 1, 1, 1, 1, 1, 64, True, False, -1, 0.125, 1.0, 1.0, 1.0, 1.0),
    # more tile pairs than compute units (rounds, a partial last one; 3 tiles
    # per head leave one pair of each head without its second tile)
    ("bf16", 1, 150, 150, 384, 384, 64, True, False, -1, 0.125, 1.0, 1.0, 1.0, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:10])))
def test_dense_vs_oracle(gpu, case):
    import scaled_dot_product_07_amd as sdpa
    out, b, h, h_kv, sq, skv, d, causal, br, window, scale, dq, dk, dv, so = case
    announce(f"fwd_fp8 {case}")
    seed = sq * 5 + skv + d + h
    q, k, v = e4m3((b, h, sq, d), seed), e4m3((b, h_kv, skv, d), seed + 1), \
        e4m3((b, h_kv, skv, d), seed + 2)
    amax = scalar(-1.0, gpu)
    o, lse = sdpa.fwd_fp8(q.to(gpu), k.to(gpu), v.to(gpu), scale=scale, causal=causal,
                          bottom_right=br, window_left=window, descale_q=scalar(dq, gpu),
                          descale_k=scalar(dk, gpu), descale_v=scalar(dv, gpu),
                          scale_o=scalar(so, gpu), amax_o=amax, out_dtype=OUT[out])
    torch.cuda.synchronize()
    assert o.dtype == OUT[out]
    o_ref, lse_ref, amax_ref = oracle.fwd_fp8(codes(q), codes(k), codes(v), scale, causal,
                                              descale_q=dq, descale_k=dk, descale_v=dv,
                                              scale_o=so, bottom_right=br, window_left=window)
    check_o_fp8(f64(o), o_ref)
    check_lse_fp8(f64(lse), lse_ref)
    a = float(amax.item())
    assert abs(a - amax_ref) <= 2.0 ** -3 * amax_ref + 1e-30
    # amax is taken before the cast: it bounds the stored values within one rounding
    assert float(o.float().abs().max()) <= a * (1 + 2.0 ** -7)


def test_bshd_and_no_factors(gpu):
    """Strided (BSHD) inputs and no factor pointers (all 1)."""
    import scaled_dot_product_07_amd as sdpa
    announce("fwd_fp8 bshd")
    q, k, v = (e4m3((2, 4, 300, 128), 40 + i, layout="bshd") for i in range(3))
    o, lse = sdpa.fwd_fp8(q.to(gpu), k.to(gpu), v.to(gpu), scale=0.09, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = oracle.fwd_fp8(codes(q), codes(k), codes(v), 0.09, True)
    check_o_fp8(f64(o), o_ref)
    check_lse_fp8(f64(lse), lse_ref)


def test_one_visible_key_is_exact(gpu):
    """window_left = 0 with causal: every row sees only its diagonal key, P is
    exactly 2^4 and O is that V row times descale_v * scale_o (to the output
    rounding); LSE is the scaled score of that key."""
    import scaled_dot_product_07_amd as sdpa
    announce("fwd_fp8 window 0")
    q, k, v = e4m3((1, 2, 150, 64), 50), e4m3((1, 2, 150, 64), 51), e4m3((1, 2, 150, 64), 52)
    o, lse = sdpa.fwd_fp8(q.to(gpu), k.to(gpu), v.to(gpu), scale=0.125, causal=True,
                          window_left=0, descale_v=scalar(0.5, gpu), scale_o=scalar(3.0, gpu))
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = oracle.fwd_fp8(codes(q), codes(k), codes(v), 0.125, True, descale_v=0.5,
                                       scale_o=3.0, window_left=0)
    np.testing.assert_allclose(f64(o), o_ref, rtol=2.0 ** -8, atol=0)
    check_lse(f64(lse), lse_ref)


def test_constant_v_rows_are_exact(gpu):
    """V rows identical over the keys: any normalised weights give that row, so
    O equals it to the output rounding whatever the rounding of P."""
    import scaled_dot_product_07_amd as sdpa
    announce("fwd_fp8 constant V")
    q, k = e4m3((1, 2, 300, 128), 60), e4m3((1, 2, 400, 128), 61)
    v = e4m3((1, 2, 1, 128), 62).float().expand(1, 2, 400, 128).to(torch.float8_e4m3fn)
    o, _ = sdpa.fwd_fp8(q.to(gpu), k.to(gpu), v.contiguous().to(gpu), scale=0.088,
                        causal=True, bottom_right=True)
    torch.cuda.synchronize()
    ref = v[:, :, :1].float().expand(1, 2, 300, 128).double().numpy()
    np.testing.assert_allclose(f64(o), ref, rtol=2.0 ** -8, atol=0)


def test_varlen_vs_oracle(gpu):
    """Packed THD with grouped heads, a band, an empty key side and NaN codes
    in the capacity tails (keys past the packed total never reach P.V)."""
    import scaled_dot_product_07_amd as sdpa
    announce("fwd_fp8_varlen")
    lens_q, lens_kv = [70, 1, 300, 129, 0, 64, 5], [100, 7, 260, 129, 40, 0, 1]
    cu_q = W.cu_seqlens(lens_q)
    cu_kv = W.cu_seqlens(lens_kv)
    tq, tkv = int(cu_q[-1]), int(cu_kv[-1])
    q = e4m3((tq + 64, 8, 64), 70).reshape(tq + 64, 8, 64)
    k = e4m3((tkv + 64, 2, 64), 71).reshape(tkv + 64, 2, 64)
    v = e4m3((tkv + 64, 2, 64), 72).reshape(tkv + 64, 2, 64)
    for t, n in ((q, tq), (k, tkv), (v, tkv)):
        t.view(torch.uint8)[n:] = 0x7F  # e4m3 NaN
    o, lse = sdpa.fwd_fp8_varlen(q.to(gpu), k.to(gpu), v.to(gpu), cu_q.to(gpu), cu_kv.to(gpu),
                                 max(lens_q), max(lens_kv), total_q=tq, total_kv=tkv, scale=0.125,
                                 causal=True, bottom_right=True, window_left=80,
                                 descale_k=scalar(0.5, gpu), out_dtype=torch.float16)
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = oracle.fwd_fp8_varlen(codes(q[:tq]), codes(k[:tkv]), codes(v[:tkv]),
                                              cu_q.numpy(), cu_kv.numpy(), 0.125, True,
                                              descale_k=0.5, bottom_right=True, window_left=80)
    check_o_fp8(f64(o[:tq]), o_ref)
    check_lse_fp8(f64(lse[:tq]), lse_ref)


@pytest.mark.parametrize("shape", ["b4h16s1024d64-causal", "b2h16s4096d128-bshd"])
def test_workload_shapes_sampled(gpu, shape):
    """The two forward workload shapes in e4m3: whole heads (causal) or sampled
    rows (non-causal) against the oracle."""
    import scaled_dot_product_07_amd as sdpa
    announce(f"fwd_fp8 workload {shape}")
    if shape.startswith("b4"):
        b, h, s, d, causal, layout = 4, 16, 1024, 64, True, "bhsd"
    else:
        b, h, s, d, causal, layout = 2, 16, 4096, 128, False, "bshd"
    q, k, v = (e4m3((b, h, s, d), 80 + i, layout=layout) for i in range(3))
    scale = 1.0 / np.sqrt(d)
    o, lse = sdpa.fwd_fp8(q.to(gpu), k.to(gpu), v.to(gpu), scale=scale, causal=causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for bi, hi in [(0, 0), (b - 1, h - 1), (1, 7)]:
        if causal:
            qb, kb, vb = (codes(x[bi:bi + 1, hi:hi + 1]) for x in (q, k, v))
            o_ref, lse_ref, _ = oracle.fwd_fp8(qb, kb, vb, scale, True, threads=8)
            check_o_fp8(f64(o[bi, hi]), o_ref[0, 0], f"O[b{bi},h{hi}]")
            check_lse_fp8(f64(lse[bi, hi]), lse_ref[0, 0], f"LSE[b{bi},h{hi}]")
        else:
            rows = np.sort(rng.choice(s, 96, replace=False))
            qd = oracle.e4m3_decode(codes(q[bi, hi]))[rows]
            kd = oracle.e4m3_decode(codes(k[bi, hi]))
            vd = oracle.e4m3_decode(codes(v[bi, hi]))
            o_ref, lse_ref = oracle.attn_rows(qd, rows, kd, vd, scale, False, threads=8)
            check_o_fp8(f64(o[bi, hi])[rows], o_ref, f"O[b{bi},h{hi}]")
            check_lse_fp8(f64(lse[bi, hi])[rows], lse_ref, f"LSE[b{bi},h{hi}]")


@pytest.mark.parametrize("d,causal", [(64, True), (64, False), (128, True)])
def test_p_cast_at_row_max_matches_rounded_p_oracle(gpu, d, causal):
    """A tighter pin of the cast of P to e4m3. Q >= 0, key 0 = 1.0 in every
    column and the other keys in [0, 1]: key 0 holds every row's largest score
    and lies in the first key tile, so the kernel's offset is that row max from
    its first tile on and never rises, and its P is the e4m3 cast of
    2^(c (s - rowmax) + 4), which the oracle's fwd_fp8_rounded_p computes in
    float64. What may differ: the bf16 rounding of O (2^-9 relative) and, for
    a P within about 2^-20 of a midpoint of the cast, the other side of it
    (the kernel's exponent is fp32 arithmetic), which moves the outputs of
    that row by up to one e4m3 step of that P over the row's sum."""
    import scaled_dot_product_07_amd as sdpa
    b, h, s = 1, 4, 320
    announce(f"fwd_fp8 rounded-P pin d={d} causal={causal}")
    rng = np.random.default_rng(40 + d + int(causal))
    enc = lambda a: torch.from_numpy(a).to(torch.float32).to(torch.float8_e4m3fn).view(
        torch.uint8)
    qv = rng.uniform(0, 1, (b, h, s, d))
    kv = rng.uniform(0, 1, (b, h, s, d))
    kv[:, :, 0, :] = 1.0
    vv = rng.uniform(-1, 1, (b, h, s, d))
    q8, k8, v8 = enc(qv), enc(kv), enc(vv)
    scale = d ** -0.5
    f8 = lambda t: t.view(torch.float8_e4m3fn).to(gpu)
    o, _ = sdpa.fwd_fp8(f8(q8), f8(k8), f8(v8), scale=scale, causal=causal,
                        out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.fwd_fp8_rounded_p(q8.numpy(), k8.numpy(), v8.numpy(), scale, causal)
    err = np.abs(f64(o) - ref)
    m = float(np.abs(ref).max())
    # (measured on MI355X: rms 2^-12.6 .. 2^-10.9, max 2^-9 .. 2^-8 of max|O|,
    # no output past the bf16 level; against the exact forward the same
    # outputs differ by up to 2^-4.6)
    assert float(np.sqrt(np.mean(err ** 2))) <= 2.0 ** -10 * m
    off = err > 2.0 ** -8 * m + 2.0 ** -8 * np.abs(ref)
    assert float(np.mean(off)) <= 0.005, f"{np.mean(off):.4f} of outputs off"
    assert float(err.max()) <= 2.0 ** -4 * m
