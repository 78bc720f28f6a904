"""Pins for the oracle's FP8 (e4m3) forward.

The per-tensor FP8 forward of cudnn-frontend pull request #554's merge log
runs attention on e4m3 inputs with per-tensor descales, folds descale_q *
descale_k into the softmax scale and descale_v * scale_o into the output, and
reports the amax of the output before its cast. What pins what:
  * the decoder: torch's float8_e4m3fn -> float64 conversion for all 256
    codes (an independent implementation of the same format), and the
    format's defining values (1.0, the smallest subnormal, the smallest
    normal, the largest finite value, the NaN codes, signed zeros);
  * the forward: torch's scaled_dot_product_attention in float64 on the
    decoded inputs times their descales (torch's own decode), with the
    output times scale_o, under a negative scale, the band options and
    grouped heads; amax = max |stored O|;
  * the descales act only through the products they scale: doubling
    descale_q and halving descale_k changes nothing;
  * packed batches equal the per-sequence dense result.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def codes(shape, seed, spread=1.0):
    """e4m3 codes of N(0, spread) values (torch's rounding), as uint8 numpy."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g) * spread
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_value(c):
    return torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).to(torch.float64)


def test_decode_matches_torch_on_every_code():
    c = np.arange(256, dtype=np.uint8)
    x = oracle.e4m3_decode(c)
    t = torch_value(c).numpy()
    assert np.array_equal(np.isnan(x), np.isnan(t))
    live = ~np.isnan(t)
    assert np.array_equal(x[live], t[live])
    assert np.array_equal(np.signbit(x[live]), np.signbit(t[live]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0xB8, -1.0), (0x40, 2.0), (0x01, 2.0 ** -9),
    (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x7E, 448.0), (0xFE, -448.0),
    (0x3C, 1.5), (0x77, 240.0),
])
def test_decode_defining_values(code, value):
    assert oracle.e4m3_decode(np.array([code], np.uint8))[0] == value


def test_decode_nan_codes_and_negative_zero():
    x = oracle.e4m3_decode(np.array([0x7F, 0xFF, 0x80], np.uint8))
    assert np.isnan(x[0]) and np.isnan(x[1])
    assert x[2] == 0.0 and np.signbit(x[2])


def _torch_ref(q8, k8, v8, scale, dq, dk, dv, so, mask=None, gqa=False):
    q, k, v = dq * torch_value(q8), dk * torch_value(k8), dv * torch_value(v8)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale, enable_gqa=gqa)
    s = scale * torch.matmul(q, k.repeat_interleave(q.shape[1] // k.shape[1], 1).transpose(-1, -2))
    if mask is not None:
        s = s.masked_fill(~mask, float("-inf"))
    return (so * o).numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("scale,dq,dk,dv,so", [(0.125, 1.0, 1.0, 1.0, 1.0),
                                               (0.09, 0.5, 2.0, 0.25, 3.0),
                                               (-0.2, 1.5, 0.75, 4.0, 0.5)])
def test_fwd_fp8_matches_torch_on_decoded_inputs(scale, dq, dk, dv, so):
    q8, k8, v8 = codes((2, 4, 37, 64), 1), codes((2, 4, 53, 64), 2), codes((2, 4, 53, 64), 3)
    o, lse, amax = oracle.fwd_fp8(q8, k8, v8, scale, False, descale_q=dq, descale_k=dk,
                                  descale_v=dv, scale_o=so)
    ref_o, ref_lse = _torch_ref(q8, k8, v8, scale, dq, dk, dv, so)
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12 * max(1.0, np.abs(ref_o).max()))
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-10)
    assert amax == np.abs(o).max() and amax == pytest.approx(np.abs(ref_o).max(), rel=1e-12)


def test_fwd_fp8_band_and_gqa_match_torch():
    sq, skv, w = 40, 70, 12
    q8, k8, v8 = codes((1, 6, sq, 128), 4), codes((1, 2, skv, 128), 5), codes((1, 2, skv, 128), 6)
    shift = skv - sq
    mask = torch.ones(sq, skv, dtype=torch.bool).tril(shift).triu(shift - w)
    o, lse, _ = oracle.fwd_fp8(q8, k8, v8, 0.1, True, descale_q=0.7, descale_k=1.3,
                               descale_v=0.9, scale_o=2.0, bottom_right=True, window_left=w)
    ref_o, ref_lse = _torch_ref(q8, k8, v8, 0.1, 0.7, 1.3, 0.9, 2.0, mask=mask, gqa=True)
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12 * np.abs(ref_o).max())
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-10)


def test_fwd_fp8_dead_rows_and_amax():
    # bottom-right with more queries than keys: the first rows see no key
    q8, k8, v8 = codes((1, 1, 9, 64), 7), codes((1, 1, 4, 64), 8), codes((1, 1, 4, 64), 9)
    o, lse, amax = oracle.fwd_fp8(q8, k8, v8, 0.125, True, bottom_right=True, scale_o=2.0)
    assert np.all(o[0, 0, :5] == 0) and np.all(np.isneginf(lse[0, 0, :5]))
    assert np.all(np.isfinite(lse[0, 0, 5:]))
    assert amax == np.abs(o).max()
    # with no query rows at all the amax is 0
    assert oracle.fwd_fp8(q8[:, :, :0], k8, v8, 0.1, False)[2] == 0.0


def test_descales_act_through_their_products():
    q8, k8, v8 = codes((1, 2, 30, 64), 10), codes((1, 2, 30, 64), 11), codes((1, 2, 30, 64), 12)
    a = oracle.fwd_fp8(q8, k8, v8, 0.125, True, descale_q=2.0, descale_k=0.5)
    b = oracle.fwd_fp8(q8, k8, v8, 0.125, True)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    c = oracle.fwd_fp8(q8, k8, v8, 0.125, True, descale_v=4.0)
    d = oracle.fwd_fp8(q8, k8, v8, 0.125, True, scale_o=4.0)
    np.testing.assert_array_equal(c[0], d[0])


def test_fwd_fp8_varlen_equals_dense_per_sequence():
    lens_q, lens_kv = [17, 1, 40], [25, 3, 40]
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(lens_kv)]).astype(np.int32)
    q8, k8, v8 = codes((sum(lens_q), 4, 64), 13), codes((sum(lens_kv), 2, 64), 14), \
        codes((sum(lens_kv), 2, 64), 15)
    o, lse, amax = oracle.fwd_fp8_varlen(q8, k8, v8, cu_q, cu_kv, 0.1, True, descale_q=0.5,
                                         descale_v=2.0, scale_o=0.25, bottom_right=True,
                                         window_left=9)
    peak = 0.0
    for i in range(3):
        qs = q8[cu_q[i]:cu_q[i + 1]].transpose(1, 0, 2)[None]
        ks = k8[cu_kv[i]:cu_kv[i + 1]].transpose(1, 0, 2)[None]
        vs = v8[cu_kv[i]:cu_kv[i + 1]].transpose(1, 0, 2)[None]
        od, ld, ad = oracle.fwd_fp8(qs, ks, vs, 0.1, True, descale_q=0.5, descale_v=2.0,
                                    scale_o=0.25, bottom_right=True, window_left=9)
        np.testing.assert_array_equal(o[cu_q[i]:cu_q[i + 1]], od[0].transpose(1, 0, 2))
        np.testing.assert_array_equal(lse[cu_q[i]:cu_q[i + 1]], ld[0].T)
        peak = max(peak, ad)
    assert amax == peak


# ---- e4m3_round and the rounded-P forward ------------------------------------

def test_e4m3_round_fixes_every_value():
    """Every finite non-negative E4M3 value rounds to itself."""
    v = oracle.e4m3_decode(np.arange(128, dtype=np.uint8))
    v = v[np.isfinite(v)]
    assert np.array_equal(oracle.e4m3_round(v), v)


def test_e4m3_round_ties_to_even_and_nearest():
    """Midpoints of neighbouring values go to the even code; points just off a
    midpoint go to the nearer value; past 448 the value saturates."""
    codes = np.arange(127, dtype=np.uint8)  # 0x00 .. 0x7e: finite, non-negative
    v = oracle.e4m3_decode(codes)
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2
    even_hi = (codes[1:] % 2) == 0
    assert np.array_equal(oracle.e4m3_round(mid), np.where(even_hi, hi, lo))
    eps = (hi - lo) * 1e-6
    assert np.array_equal(oracle.e4m3_round(mid - eps), lo)
    assert np.array_equal(oracle.e4m3_round(mid + eps), hi)
    assert oracle.e4m3_round(np.array([1e4]))[0] == 448.0


def test_e4m3_round_matches_torch_cast():
    """Against torch's own float8_e4m3fn cast (round to nearest even) on random
    values in the finite range, an implementation the oracle does not use."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(0, 448, 20000), rng.uniform(0, 2.0 ** -5, 20000),
                        2.0 ** rng.uniform(-10, 8, 20000)])
    x = x[x <= 448]
    ref = torch.from_numpy(x).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    # float32 first: exact for these draws' rounding except in the last bits,
    # which cannot move an e4m3 decision (3 mantissa bits)
    assert np.array_equal(oracle.e4m3_round(x.astype(np.float32).astype(np.float64)), ref)


def test_fwd_fp8_rounded_p_equals_exact_when_every_p_is_a_power_of_two():
    """scale = ln 2 and integer scores: every P = 2^(s - max + 4) is an
    integer power of two, which e4m3 holds exactly, so the rounded-P forward
    is the exact FP8 forward."""
    b, h, s, d = 1, 2, 40, 16
    rng = np.random.default_rng(3)
    q = np.zeros((b, h, s, d)); q[..., 0] = 1.0
    k = np.zeros((b, h, s, d)); k[..., 0] = rng.integers(0, 6, (b, h, s))
    v = rng.uniform(-2, 2, (b, h, s, d))
    enc = lambda a: torch.from_numpy(a).to(torch.float32).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    q8, k8, v8 = enc(q), enc(k), enc(v)
    for causal in (False, True):
        o_r = oracle.fwd_fp8_rounded_p(q8, k8, v8, float(np.log(2.0)), causal)
        o_e, _, _ = oracle.fwd_fp8(q8, k8, v8, float(np.log(2.0)), causal)
        assert np.allclose(o_r, o_e, rtol=1e-12, atol=1e-12)


def test_fwd_fp8_rounded_p_rounds():
    """With scores that are not integer in log2 units the cast changes P: the
    result moves off the exact forward, by at most the cast's relative error
    (2^-4) times max |V|."""
    b, h, s, d = 1, 2, 48, 32
    rng = np.random.default_rng(5)
    enc = lambda a: torch.from_numpy(a).to(torch.float32).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    q8 = enc(rng.uniform(0, 1, (b, h, s, d)))
    k8 = enc(rng.uniform(0, 1, (b, h, s, d)))
    v8 = enc(rng.uniform(-1, 1, (b, h, s, d)))
    o_r = oracle.fwd_fp8_rounded_p(q8, k8, v8, 0.3, True)
    o_e, _, _ = oracle.fwd_fp8(q8, k8, v8, 0.3, True)
    diff = np.abs(o_r - o_e).max()
    vmax = np.abs(oracle.e4m3_decode(v8)).max()
    assert 0 < diff <= 2 * 2.0 ** -4 * vmax
