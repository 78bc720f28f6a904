"""Pins for the oracle's mask options and grouped-query heads.

The options follow the sdpa API of cudnn-frontend pull request #554
("torch: put torch.sdpa on the cuDNN Python API"): is_causal (top-left),
causal_bottom_right, window_left, and GQA (h_kv < h_q). What pins what:
  * bottom-right causal: torch's lower-right causal bias
    (torch.nn.attention.bias.causal_lower_right) in float64 -- an
    independent statement of the alignment; equal lengths reduce to top-left;
  * window_left: torch attention with a band mask built by torch's tril/triu
    (an independent band construction); window 0 has a closed form (each
    row returns the V row on its aligned diagonal and LSE = scale q.k of that
    key); a window as wide as the keys changes nothing;
  * GQA: torch's scaled_dot_product_attention with enable_gqa in float64, and
    torch autograd through it for dQ, dK, dV (a K/V head's gradient sums over
    its query heads);
  * masked backward: torch autograd through the band-masked attention;
  * packed batches with these options equal the per-sequence dense result.
Rows with no visible key are checked to give O = 0 and LSE = -inf (torch
returns NaN there, so those rows are compared only against that reading).
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def band(s_q, s_kv, causal, bottom_right, window):
    """Boolean [s_q, s_kv] visibility built from torch's tril/triu."""
    shift = s_kv - s_q if bottom_right else 0
    m = torch.ones(s_q, s_kv, dtype=torch.bool)
    if causal:
        m = m.tril(shift)
    if window >= 0:
        m = m.triu(shift - window)
    return m


def torch_masked(q, k, v, scale, mask, gqa=False):
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    return F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                          enable_gqa=gqa).numpy()


def live_rows(mask):
    return mask.any(dim=1).numpy()


@pytest.mark.parametrize("sq,skv", [(5, 9), (9, 5), (8, 8), (1, 6)])
def test_bottom_right_matches_torch_lower_right(sq, skv):
    q, k, v = rnd((2, 3, sq, 16), 1), rnd((2, 3, skv, 16), 2), rnd((2, 3, skv, 16), 3)
    o, lse = oracle.fwd(q, k, v, 0.3, True, bottom_right=True)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=causal_lower_right(sq, skv),
                                         scale=0.3).numpy()
    live = np.arange(sq) + skv - sq >= 0
    np.testing.assert_allclose(o[:, :, live], ref[:, :, live], atol=1e-12)
    assert np.all(o[:, :, ~live] == 0) and np.all(np.isneginf(lse[:, :, ~live]))
    # LSE of the live rows: torch's logsumexp over the same lower-right band
    s = 0.3 * torch.einsum("bhqd,bhkd->bhqk", tq, tk)
    s = s.masked_fill(~causal_lower_right(sq, skv)._materialize(torch.device("cpu")), float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    np.testing.assert_allclose(lse[:, :, live], ref_lse[:, :, live], atol=1e-12)


def test_bottom_right_equal_lengths_is_top_left():
    q, k, v = rnd((1, 2, 13, 8), 4), rnd((1, 2, 13, 8), 5), rnd((1, 2, 13, 8), 6)
    a = oracle.fwd(q, k, v, 0.4, True, bottom_right=True)
    b = oracle.fwd(q, k, v, 0.4, True)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("bottom_right", [False, True])
@pytest.mark.parametrize("sq,skv", [(7, 7), (4, 10), (10, 4)])
def test_window_zero_closed_form(bottom_right, sq, skv):
    """Causal with window_left 0: row i sees only its aligned diagonal key p."""
    q, k, v = rnd((1, 1, sq, 8), 7), rnd((1, 1, skv, 8), 8), rnd((1, 1, skv, 8), 9)
    o, lse = oracle.fwd(q, k, v, 0.7, True, bottom_right=bottom_right, window_left=0)
    shift = skv - sq if bottom_right else 0
    for i in range(sq):
        p = i + shift
        if 0 <= p < skv:
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, p], atol=1e-14)
            np.testing.assert_allclose(lse[0, 0, i], 0.7 * q[0, 0, i] @ k[0, 0, p], atol=1e-13)
        else:
            assert np.all(o[0, 0, i] == 0) and np.isneginf(lse[0, 0, i])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bottom_right", [False, True])
@pytest.mark.parametrize("window", [1, 3, 6])
@pytest.mark.parametrize("sq,skv", [(9, 9), (6, 11), (11, 6)])
def test_window_matches_band_mask(causal, bottom_right, window, sq, skv):
    q, k, v = rnd((1, 2, sq, 8), 10), rnd((1, 2, skv, 8), 11), rnd((1, 2, skv, 8), 12)
    o, lse = oracle.fwd(q, k, v, 0.45, causal, bottom_right=bottom_right, window_left=window)
    m = band(sq, skv, causal, bottom_right, window)
    live = live_rows(m)
    ref = torch_masked(q, k, v, 0.45, m)
    np.testing.assert_allclose(o[:, :, live], ref[:, :, live], atol=1e-12)
    assert np.all(o[:, :, ~live] == 0) and np.all(np.isneginf(lse[:, :, ~live]))


@pytest.mark.parametrize("bottom_right", [False, True])
def test_window_as_wide_as_keys_changes_nothing(bottom_right):
    q, k, v = rnd((1, 2, 12, 8), 13), rnd((1, 2, 12, 8), 14), rnd((1, 2, 12, 8), 15)
    a = oracle.fwd(q, k, v, 0.5, True, bottom_right=bottom_right, window_left=12)
    b = oracle.fwd(q, k, v, 0.5, True, bottom_right=bottom_right)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("h,h_kv", [(4, 2), (6, 1), (8, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_fwd_matches_torch(h, h_kv, causal):
    q, k, v = rnd((2, h, 11, 16), 16), rnd((2, h_kv, 11, 16), 17), rnd((2, h_kv, 11, 16), 18)
    o, lse = oracle.fwd(q, k, v, 0.33, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.33,
                                         enable_gqa=True).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)
    # LSE: aten's CPU flash kernel on K/V heads repeated to h (torch's own repeat)
    g = h // h_kv
    _, ref_lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq, tk.repeat_interleave(g, 1), tv.repeat_interleave(g, 1), 0.0, causal,
        attn_mask=None, scale=0.33)
    np.testing.assert_allclose(lse, ref_lse.numpy(), atol=1e-12)


@pytest.mark.parametrize("h,h_kv", [(4, 2), (3, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_bwd_matches_torch_autograd(h, h_kv, causal):
    q, k, v = rnd((1, h, 9, 8), 19), rnd((1, h_kv, 13, 8), 20), rnd((1, h_kv, 13, 8), 21)
    do = rnd((1, h, 9, 8), 22)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.29,
                                        enable_gqa=True)
    to.backward(torch.from_numpy(do))
    o, lse, dq, dk, dv = oracle.bwd(q, k, v, do, 0.29, causal)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


@pytest.mark.parametrize("causal,bottom_right,window", [(True, True, -1), (True, False, 2),
                                                        (True, True, 3), (False, False, 2),
                                                        (False, True, 4)])
def test_masked_bwd_matches_torch_autograd(causal, bottom_right, window):
    sq, skv = 8, 12
    q, k, v = rnd((1, 2, sq, 8), 23), rnd((1, 2, skv, 8), 24), rnd((1, 2, skv, 8), 25)
    do = rnd((1, 2, sq, 8), 26)
    m = band(sq, skv, causal, bottom_right, window)
    assert m.any(dim=1).all()  # every row live here, so torch has no NaN rows
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=0.5)
    to.backward(torch.from_numpy(do))
    o, lse, dq, dk, dv = oracle.bwd(q, k, v, do, 0.5, causal, bottom_right=bottom_right,
                                    window_left=window)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_dead_rows_in_backward_have_zero_gradient():
    """Bottom-right with s_q > s_kv: the first rows see no key; their dQ is 0 and
    they add nothing to dK, dV (the remaining rows against torch autograd)."""
    sq, skv = 9, 5
    q, k, v = rnd((1, 1, sq, 8), 27), rnd((1, 1, skv, 8), 28), rnd((1, 1, skv, 8), 29)
    do = rnd((1, 1, sq, 8), 30)
    o, lse, dq, dk, dv = oracle.bwd(q, k, v, do, 0.6, True, bottom_right=True)
    dead = sq - skv
    assert np.all(dq[:, :, :dead] == 0)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in
                  (q[:, :, dead:], k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=causal_lower_right(skv, skv),
                                        scale=0.6)
    to.backward(torch.from_numpy(do[:, :, dead:]))
    np.testing.assert_allclose(dq[:, :, dead:], tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def _packed(lens_q, lens_kv, h, h_kv, d, seed):
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(lens_kv)]).astype(np.int32)
    return (cu_q, cu_kv, rnd((int(cu_q[-1]), h, d), seed), rnd((int(cu_kv[-1]), h_kv, d), seed + 1),
            rnd((int(cu_kv[-1]), h_kv, d), seed + 2))


@pytest.mark.parametrize("causal,bottom_right,window", [(True, True, -1), (True, False, 3),
                                                        (True, True, 2), (False, True, 5)])
def test_varlen_options_are_per_sequence_dense(causal, bottom_right, window):
    lens_q, lens_kv = [5, 1, 9, 7], [8, 3, 9, 4]
    h, h_kv, d = 4, 2, 8
    cu_q, cu_kv, q, k, v = _packed(lens_q, lens_kv, h, h_kv, d, 31)
    do = rnd(q.shape, 40)
    kw = dict(bottom_right=bottom_right, window_left=window)
    o, lse = oracle.fwd_varlen(q, k, v, cu_q, cu_kv, 0.35, causal, **kw)
    _, _, dq, dk, dv = oracle.bwd_varlen(q, k, v, do, cu_q, cu_kv, 0.35, causal, **kw)
    for n in range(len(lens_q)):
        sq_, skv_ = slice(cu_q[n], cu_q[n + 1]), slice(cu_kv[n], cu_kv[n + 1])
        dense = lambda x: x.transpose(1, 0, 2)[None]  # noqa: E731
        on, ln = oracle.fwd(dense(q[sq_]), dense(k[skv_]), dense(v[skv_]), 0.35, causal, **kw)
        np.testing.assert_allclose(o[sq_], on[0].transpose(1, 0, 2), atol=1e-13)
        np.testing.assert_allclose(lse[sq_], ln[0].T, atol=1e-13)
        _, _, dqn, dkn, dvn = oracle.bwd(dense(q[sq_]), dense(k[skv_]), dense(v[skv_]),
                                         dense(do[sq_]), 0.35, causal, **kw)
        np.testing.assert_allclose(dq[sq_], dqn[0].transpose(1, 0, 2), atol=1e-12)
        np.testing.assert_allclose(dk[skv_], dkn[0].transpose(1, 0, 2), atol=1e-12)
        np.testing.assert_allclose(dv[skv_], dvn[0].transpose(1, 0, 2), atol=1e-12)
