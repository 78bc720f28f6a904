"""Pins for the oracle: each function is tied to something other than itself.

What pins what (a plausible slip in the oracle fails at least one):
  * torch's CPU attention in float64 (the pages' own check is torch's
    scaled_dot_product_attention): O, and aten's CPU flash kernel for the
    logsumexp statistic -- catches a dropped scale, a transposed operand, a
    wrong mask direction or a wrong LSE base;
  * torch autograd in float64: dQ, dK, dV;
  * central finite differences of the oracle's own forward: the backward;
  * a hand-worked golden case (tests/golden/hand_worked_two_keys.txt);
  * closed forms: causal row 0 returns V[0]; identical keys return the mean of
    the visible V rows; all-ones V returns ones (rows of P sum to 1);
  * invariants: shifting every key by u shifts LSE by scale*q.u and leaves O;
    permuting keys and values jointly (non-causal) leaves O; packed batches
    equal the per-sequence dense result and do not see each other;
  * backward identities: sum_j dV_j = sum_i dO_i and sum_j dK_j = 0.
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_two_keys.txt")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def torch_ref(q, k, v, scale, causal):
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    return o.numpy()


def torch_lse(q, k, v, scale, causal):
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    _, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq, tk, tv, 0.0, causal, attn_mask=None, scale=scale)
    return lse.numpy()


SHAPES = [(1, 1, 1, 1, 4), (2, 3, 17, 17, 8), (1, 2, 33, 33, 64), (1, 1, 70, 70, 128),
          (2, 2, 9, 21, 16)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_matches_torch_fp64(shape, causal):
    b, h, sq, skv, d = shape
    q, k, v = rnd((b, h, sq, d), 1), rnd((b, h, skv, d), 2), rnd((b, h, skv, d), 3)
    scale = 0.37
    o, lse = oracle.fwd(q, k, v, scale, causal)
    np.testing.assert_allclose(o, torch_ref(q, k, v, scale, causal), rtol=0, atol=1e-12)
    if sq == skv:  # aten's CPU flash kernel: same top-left reading when square
        np.testing.assert_allclose(lse, torch_lse(q, k, v, scale, causal), rtol=0, atol=1e-12)


def test_lse_matches_torch_noncausal_rectangular():
    q, k, v = rnd((1, 2, 9, 16), 4), rnd((1, 2, 21, 16), 5), rnd((1, 2, 21, 16), 6)
    _, lse = oracle.fwd(q, k, v, 0.25, False)
    np.testing.assert_allclose(lse, torch_lse(q, k, v, 0.25, False), atol=1e-12)


def test_causal_top_left_when_rectangular():
    """s_q < s_kv: query i sees keys 0..i (top-left), per torch's is_causal."""
    q, k, v = rnd((1, 1, 3, 8), 7), rnd((1, 1, 6, 8), 8), rnd((1, 1, 6, 8), 9)
    o, lse = oracle.fwd(q, k, v, 0.5, True)
    for i in range(3):
        oi, li = oracle.fwd(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.5, False)
        np.testing.assert_allclose(o[0, 0, i], oi[0, 0, 0], atol=1e-13)
        np.testing.assert_allclose(lse[0, 0, i], li[0, 0, 0], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 5, 5, 4), (2, 2, 13, 13, 16), (1, 2, 7, 11, 8)])
def test_bwd_matches_torch_autograd(shape, causal):
    b, h, sq, skv, d = shape
    q, k, v = rnd((b, h, sq, d), 11), rnd((b, h, skv, d), 12), rnd((b, h, skv, d), 13)
    do = rnd((b, h, sq, d), 14)
    scale = 0.41
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.from_numpy(do))
    o, lse, dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,d", [(1, 2), (3, 4), (5, 3)])
def test_bwd_finite_differences(causal, sq, d):
    """dL/dX for L = sum(O * G) by central differences of the oracle forward."""
    q, k, v = rnd((1, 1, sq, d), 21), rnd((1, 1, sq, d), 22), rnd((1, 1, sq, d), 23)
    g = rnd((1, 1, sq, d), 24)
    scale = 0.7
    _, _, dq, dk, dv = oracle.bwd(q, k, v, g, scale, causal)
    eps = 1e-6

    def loss(qq, kk, vv):
        o, _ = oracle.fwd(qq, kk, vv, scale, causal)
        return float(np.sum(o * g))

    for pos, (name, grad) in enumerate((("q", dq), ("k", dk), ("v", dv))):
        x = (q, k, v)[pos]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[pos], args_m[pos] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, atol=1e-7, err_msg=name)


def _parse_golden():
    cases, cur = {}, None
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("["):
                cur = cases.setdefault(line.strip("[]"), {})
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            if key == "scale":
                cur[key] = float(val)
            else:
                cur[key] = np.array([[float(x) for x in row.split(",")] for row in val.split(";")])
    return cases


@pytest.mark.parametrize("name", ["A", "B"])
def test_golden_hand_worked(name):
    c = _parse_golden()[name]
    q, k, v = (c[x][None, None] for x in ("q", "k", "v"))
    for causal, tag in ((False, "noncausal"), (True, "causal")):
        o, lse = oracle.fwd(q, k, v, c["scale"], causal)
        np.testing.assert_allclose(o[0, 0], c["o_" + tag], atol=1e-12)
        np.testing.assert_allclose(lse[0, 0], c["lse_" + tag][:, 0], atol=1e-12)
    if "dout" in c:
        _, _, dq, dk, dv = oracle.bwd(q, k, v, c["dout"][None, None], c["scale"], False)
        np.testing.assert_allclose(dq[0, 0], c["dq_noncausal"], atol=1e-12)
        np.testing.assert_allclose(dk[0, 0], c["dk_noncausal"], atol=1e-12)
        np.testing.assert_allclose(dv[0, 0], c["dv_noncausal"], atol=1e-12)


def test_causal_row0_returns_v0():
    q, k, v = rnd((2, 3, 40, 16), 31), rnd((2, 3, 40, 16), 32), rnd((2, 3, 40, 16), 33)
    o, lse = oracle.fwd(q, k, v, 0.3, True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.sum(q[:, :, 0] * k[:, :, 0], -1), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_v(causal):
    s, d = 23, 8
    q, v = rnd((1, 1, s, d), 41), rnd((1, 1, s, d), 42)
    k = np.broadcast_to(rnd((1, 1, 1, d), 43), (1, 1, s, d)).copy()
    o, lse = oracle.fwd(q, k, v, 0.6, causal)
    for i in range(s):
        n = i + 1 if causal else s
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(0), atol=1e-13)
        np.testing.assert_allclose(lse[0, 0, i], 0.6 * q[0, 0, i] @ k[0, 0, 0] + math.log(n),
                                   atol=1e-12)


def test_rows_of_p_sum_to_one():
    q, k = rnd((2, 2, 31, 16), 51) * 3, rnd((2, 2, 31, 16), 52) * 3
    v = np.ones((2, 2, 31, 16))
    for causal in (False, True):
        o, _ = oracle.fwd(q, k, v, 0.9, causal)
        np.testing.assert_allclose(o, 1.0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    q, k, v = rnd((1, 2, 19, 8), 61), rnd((1, 2, 19, 8), 62), rnd((1, 2, 19, 8), 63)
    u = rnd((8,), 64)
    o1, l1 = oracle.fwd(q, k, v, 0.45, causal)
    o2, l2 = oracle.fwd(q, k + u, v, 0.45, causal)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + 0.45 * (q @ u), atol=1e-12)


def test_key_permutation_invariance_noncausal():
    q, k, v = rnd((1, 1, 12, 8), 71), rnd((1, 1, 15, 8), 72), rnd((1, 1, 15, 8), 73)
    perm = np.random.default_rng(74).permutation(15)
    o1, l1 = oracle.fwd(q, k, v, 0.5, False)
    o2, l2 = oracle.fwd(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, atol=1e-12)


def test_attn_rows_equals_full_rows():
    q, k, v = rnd((1, 1, 50, 16), 81), rnd((1, 1, 50, 16), 82), rnd((1, 1, 50, 16), 83)
    o, lse = oracle.fwd(q, k, v, 0.25, True)
    rows = np.array([0, 7, 31, 49])
    o2, l2 = oracle.attn_rows(q[0, 0, rows], rows, k[0, 0], v[0, 0], 0.25, True)
    assert np.array_equal(o2, o[0, 0, rows]) and np.array_equal(l2, lse[0, 0, rows])


def _packed(lens, h, d, seed):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t = int(cu[-1])
    return cu, rnd((t, h, d), seed), rnd((t, h, d), seed + 1), rnd((t, h, d), seed + 2)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_is_per_sequence_dense(causal):
    lens = [5, 1, 17, 9]
    h, d = 3, 8
    cu, q, k, v = _packed(lens, h, d, 90)
    o, lse = oracle.fwd_varlen(q, k, v, cu, cu, 0.35, causal)
    for n, L in enumerate(lens):
        sl = slice(cu[n], cu[n + 1])
        on, ln = oracle.fwd(*(x[sl].transpose(1, 0, 2)[None] for x in (q, k, v)), 0.35, causal)
        np.testing.assert_allclose(o[sl], on[0].transpose(1, 0, 2), atol=1e-13)
        np.testing.assert_allclose(lse[sl], ln[0].T, atol=1e-13)


def test_varlen_sequences_do_not_see_each_other():
    lens = [6, 11, 4]
    cu, q, k, v = _packed(lens, 2, 8, 100)
    o1, l1 = oracle.fwd_varlen(q, k, v, cu, cu, 0.5, True)
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:cu[2]] += 5.0
    v2[cu[1]:cu[2]] -= 3.0
    o2, l2 = oracle.fwd_varlen(q, k2, v2, cu, cu, 0.5, True)
    for n in (0, 2):
        sl = slice(cu[n], cu[n + 1])
        assert np.array_equal(o1[sl], o2[sl]) and np.array_equal(l1[sl], l2[sl])
    assert not np.allclose(o1[cu[1]:cu[2]], o2[cu[1]:cu[2]])


def test_varlen_dead_rows_and_empty_sequences():
    """Zero-length KV: dead rows (O = 0, LSE = -inf). Zero-length Q: writes nothing."""
    h, d = 2, 4
    cu_q = np.array([0, 3, 3, 7], dtype=np.int32)   # sequence 1 has no queries
    cu_kv = np.array([0, 0, 5, 9], dtype=np.int32)  # sequence 0 has no keys
    q, k, v = rnd((7, h, d), 110), rnd((9, h, d), 111), rnd((9, h, d), 112)
    o, lse = oracle.fwd_varlen(q, k, v, cu_q, cu_kv, 0.5, False)
    assert np.all(o[0:3] == 0) and np.all(np.isneginf(lse[0:3]))
    on, ln = oracle.fwd(q[3:7].transpose(1, 0, 2)[None], k[5:9].transpose(1, 0, 2)[None],
                        v[5:9].transpose(1, 0, 2)[None], 0.5, False)
    np.testing.assert_allclose(o[3:7], on[0].transpose(1, 0, 2), atol=1e-13)


def test_dense_dead_rows_when_no_keys():
    q = rnd((1, 1, 4, 8), 120)
    k = np.zeros((1, 1, 0, 8))
    o, lse = oracle.fwd(q, k, k, 0.5, False)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_identities(causal):
    q, k, v = rnd((2, 2, 29, 16), 131), rnd((2, 2, 29, 16), 132), rnd((2, 2, 29, 16), 133)
    do = rnd((2, 2, 29, 16), 134)
    _, _, dq, dk, dv = oracle.bwd(q, k, v, do, 0.3, causal)
    np.testing.assert_allclose(dv.sum(2), do.sum(2), atol=1e-11)
    np.testing.assert_allclose(dk.sum(2), 0.0, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_is_per_sequence_dense(causal):
    lens = [4, 9, 1]
    h, d = 2, 8
    cu, q, k, v = _packed(lens, h, d, 140)
    do = rnd(q.shape, 150)
    _, _, dq, dk, dv = oracle.bwd_varlen(q, k, v, do, cu, cu, 0.5, causal)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        args = [x[sl].transpose(1, 0, 2)[None] for x in (q, k, v, do)]
        _, _, dqn, dkn, dvn = oracle.bwd(*args, 0.5, causal)
        np.testing.assert_allclose(dq[sl], dqn[0].transpose(1, 0, 2), atol=1e-12)
        np.testing.assert_allclose(dk[sl], dkn[0].transpose(1, 0, 2), atol=1e-12)
        np.testing.assert_allclose(dv[sl], dvn[0].transpose(1, 0, 2), atol=1e-12)


def test_threads_do_not_change_result():
    q, k, v = rnd((1, 2, 64, 32), 160), rnd((1, 2, 64, 32), 161), rnd((1, 2, 64, 32), 162)
    o1, l1 = oracle.fwd(q, k, v, 0.2, True, threads=1)
    o2, l2 = oracle.fwd(q, k, v, 0.2, True, threads=7)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
