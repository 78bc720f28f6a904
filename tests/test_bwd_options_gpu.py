"""GPU parity of the backward with grouped-query heads and the band options
(sdpa_bwd_ex), and of the packed THD backward (sdpa_bwd_varlen), against the
fp64 oracle. The GPU backward consumes the GPU forward's O and LSE; the oracle
runs its own fp64 forward. Tolerances are the shared ones in tests/parity.py.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import announce, check_grad, f64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _dense(b, h, h_kv, sq, skv, d, dt, seed, layout="bhsd"):
    g = torch.Generator().manual_seed(seed)
    out = []
    for nh, s in ((h, sq), (h_kv, skv), (h_kv, skv), (h, sq)):
        if layout == "bhsd":
            out.append(torch.randn(b, nh, s, d, generator=g).to(DT[dt]))
        else:
            out.append(torch.randn(b, s, nh, d, generator=g).to(DT[dt]).transpose(1, 2))
    return out


def _check_all(dq, dk, dv, ref):
    _, _, dq_r, dk_r, dv_r = ref
    check_grad(f64(dq), dq_r, "dQ")
    check_grad(f64(dk), dk_r, "dK")
    check_grad(f64(dv), dv_r, "dV")


CASES = [
    # dtype, b, h, h_kv, s_q, s_kv, d, causal, bottom_right, window
    ("bf16", 1, 2, 2, 200, 520, 64, True, True, -1),    # bottom-right, s_q < s_kv
    ("bf16", 1, 2, 2, 520, 200, 64, True, True, -1),    # bottom-right, dead query rows
    ("bf16", 1, 2, 2, 400, 400, 64, True, False, 0),    # window 0: the diagonal only
    ("fp16", 1, 2, 2, 400, 400, 128, True, False, 37),  # window inside one tile
    ("bf16", 2, 2, 2, 700, 700, 64, True, False, 150),  # window over several tiles
    ("fp16", 1, 2, 2, 333, 600, 64, True, True, 90),    # window + bottom-right
    ("bf16", 1, 2, 2, 300, 500, 128, False, False, 70),  # left bound only
    ("bf16", 1, 2, 2, 450, 300, 64, False, True, 40),   # left bound only, bottom-right
    ("bf16", 1, 8, 2, 260, 260, 64, True, False, -1),   # GQA, group 4
    ("fp16", 2, 6, 1, 200, 330, 128, False, False, -1),  # MQA
    ("bf16", 1, 4, 2, 300, 700, 128, True, True, 200),  # GQA + band
    ("bf16", 1, 3, 3, 1, 1, 64, True, True, 0),         # one query, one key
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_dense_options_vs_oracle(gpu, case):
    import scaled_dot_product_07_amd as sdpa
    dt, b, h, h_kv, sq, skv, d, causal, br, window = case
    announce(f"bwd options {case}")
    q, k, v, do = _dense(b, h, h_kv, sq, skv, d, dt, seed=sq * 3 + skv + d + h + window)
    scale = 1.0 / np.sqrt(d)
    qd, kd, vd, dod = (x.to(gpu) for x in (q, k, v, do))
    o, lse = sdpa.fwd(qd, kd, vd, scale=scale, causal=causal, bottom_right=br,
                      window_left=window)
    dq, dk, dv = sdpa.bwd(qd, kd, vd, o, dod, lse, scale=scale, causal=causal, bottom_right=br,
                          window_left=window)
    torch.cuda.synchronize()
    ref = oracle.bwd(f64(q), f64(k), f64(v), f64(do), scale, causal, bottom_right=br,
                     window_left=window)
    _check_all(dq, dk, dv, ref)


def test_bshd_gqa_window(gpu):
    """Strided (BSHD) tensors with grouped heads, a window and a negative scale."""
    import scaled_dot_product_07_amd as sdpa
    announce("bwd options bshd gqa window")
    q, k, v, do = _dense(2, 8, 2, 300, 300, 128, "bf16", seed=5, layout="bshd")
    qd, kd, vd, dod = (x.to(gpu) for x in (q, k, v, do))
    o, lse = sdpa.fwd(qd, kd, vd, scale=-0.09, causal=True, window_left=100)
    dq, dk, dv = sdpa.bwd(qd, kd, vd, o, dod, lse, scale=-0.09, causal=True, window_left=100)
    torch.cuda.synchronize()
    assert dq.stride() == qd.stride() and dk.stride() == kd.stride()
    ref = oracle.bwd(f64(q), f64(k), f64(v), f64(do), -0.09, True, window_left=100)
    _check_all(dq, dk, dv, ref)


def test_option_defaults_match_plain_backward(gpu):
    """h_kv == h, top-left, no window: bit-identical to the plain backward."""
    import scaled_dot_product_07_amd as sdpa
    announce("bwd options defaults")
    q, k, v, do = (x.to(gpu) for x in _dense(2, 4, 4, 333, 333, 64, "bf16", seed=8))
    o, lse = sdpa.fwd(q, k, v, scale=0.125, causal=True)
    a = sdpa.bwd(q, k, v, o, do, lse, scale=0.125, causal=True)
    b2 = sdpa.bwd(q, k, v, o, do, lse, scale=0.125, causal=True, bottom_right=True)
    b3 = sdpa.bwd(q, k, v, o, do, lse, scale=0.125, causal=True, window_left=1000)
    torch.cuda.synchronize()
    for other in (b2, b3):
        for x, y in zip(a, other):
            assert torch.equal(x, y)


def test_gqa_equals_repeated_heads(gpu):
    """dK, dV of a grouped head equal the group sum of the dK, dV that the same
    problem gives with K, V repeated per query head (fp32 sums of the bf16
    per-head results; the grouped kernel sums in fp32 before rounding once)."""
    import scaled_dot_product_07_amd as sdpa
    announce("bwd gqa vs repeated heads")
    q, k, v, do = (x.to(gpu) for x in _dense(1, 8, 2, 256, 384, 64, "bf16", seed=31))
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o, lse = sdpa.fwd(q, k, v, scale=0.125, causal=True, bottom_right=True, window_left=64)
    o2, lse2 = sdpa.fwd(q, kr, vr, scale=0.125, causal=True, bottom_right=True, window_left=64)
    dq, dk, dv = sdpa.bwd(q, k, v, o, do, lse, scale=0.125, causal=True, bottom_right=True,
                          window_left=64)
    dq2, dk2, dv2 = sdpa.bwd(q, kr, vr, o2, do, lse2, scale=0.125, causal=True,
                             bottom_right=True, window_left=64)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(dq, dq2)
    for g1, g4 in ((dk, dk2), (dv, dv2)):
        summed = g4.float().view(1, 2, 4, 384, 64).sum(2)
        err = (g1.float() - summed).abs().max().item()
        assert err <= 2e-2 * summed.abs().max().item(), err


# ---------------------------------------------------------------------------
# packed THD backward


def _varlen_run(sdpa, vi, h, d, dt, scale, causal, br, window, gpu, fill=None):
    q, k, v, do = (x.to(gpu) for x in (vi.q, vi.k, vi.v, vi.dout))
    cq, ckv = vi.cu_q.to(gpu), vi.cu_kv.to(gpu)
    mq, mkv = int(vi.lens_q.max()), int(vi.lens_kv.max())
    o, lse = sdpa.fwd_varlen(q, k, v, cq, ckv, max(mq, 1), max(mkv, 1), total_q=vi.total_q,
                             total_kv=vi.total_kv, scale=scale, causal=causal, bottom_right=br,
                             window_left=window)
    grads = None
    if fill is not None:
        grads = [torch.full_like(x, fill) for x in (q, k, v)]
    dq, dk, dv = sdpa.bwd_varlen(q, k, v, o, do, lse, cq, ckv, max(mq, 1), max(mkv, 1),
                                 total_q=vi.total_q, total_kv=vi.total_kv, scale=scale,
                                 causal=causal, bottom_right=br, window_left=window,
                                 dq=None if grads is None else grads[0],
                                 dk=None if grads is None else grads[1],
                                 dv=None if grads is None else grads[2])
    torch.cuda.synchronize()
    return dq, dk, dv


VARLEN = [
    # lens_q, lens_kv, h, h_kv, d, dtype, causal, bottom_right, window
    ([70, 1, 300, 129, 64, 5], [70, 1, 300, 129, 64, 5], 2, 2, 64, "bf16", True, False, -1),
    ([70, 1, 300, 129, 64, 5], [100, 7, 260, 129, 190, 1], 4, 2, 64, "bf16", True, True, -1),
    ([200, 33, 0, 150], [200, 90, 50, 0], 2, 2, 128, "fp16", True, True, 40),
    ([257, 128, 3], [300, 128, 200], 6, 1, 128, "bf16", False, False, -1),
    ([190, 64, 77], [190, 250, 30], 4, 4, 64, "bf16", False, True, 30),
    ([500, 131], [500, 131], 8, 2, 64, "fp16", True, False, 100),
]
# Many sequences (more than one wave's 64 lanes, so the workgroups' unit
# search reads cu_seqlens in chunks), some without queries or keys.
_g = np.random.default_rng(91)
_lq = _g.integers(0, 260, size=100)
_lq[_g.random(100) < 0.15] = 0
_lkv = _g.integers(0, 260, size=100)
_lkv[_g.random(100) < 0.15] = 0
VARLEN += [
    (_lq.tolist(), _lq.tolist(), 2, 2, 64, "bf16", True, False, -1),
    (_lq.tolist(), _lkv.tolist(), 4, 2, 64, "bf16", False, False, -1),
    (_lq.tolist(), _lkv.tolist(), 2, 1, 128, "fp16", True, True, 50),
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"{c[5]}-h{c[2]}kv{c[3]}-d{c[4]}-"
                         f"c{int(c[6])}br{int(c[7])}w{c[8]}-n{len(c[0])}")
def test_varlen_vs_oracle(gpu, case):
    import scaled_dot_product_07_amd as sdpa
    lens_q, lens_kv, h, h_kv, d, dt, causal, br, window = case
    announce(f"bwd_varlen {case}")
    vi = W.varlen_inputs(lens_q, lens_kv, h, d, dt, seed=sum(lens_q) + h + d, with_dout=True,
                         h_kv=h_kv)
    scale = 1.0 / np.sqrt(d)
    fill = 3.0  # rows past the packed totals must keep it
    dq, dk, dv = _varlen_run(sdpa, vi, h, d, dt, scale, causal, br, window, gpu, fill=fill)
    tq, tkv = vi.total_q, vi.total_kv
    ref = oracle.bwd_varlen(f64(vi.q[:tq]), f64(vi.k[:tkv]), f64(vi.v[:tkv]),
                            f64(vi.dout[:tq]), vi.cu_q.numpy(), vi.cu_kv.numpy(), scale, causal,
                            bottom_right=br, window_left=window)
    _check_all(dq[:tq], dk[:tkv], dv[:tkv], ref)
    for g, t in ((dq, tq), (dk, tkv), (dv, tkv)):
        assert bool((g[t:] == fill).all()), "rows past the packed total were written"


def test_varlen_single_sequence_equals_dense(gpu):
    """One packed sequence is the dense problem with b = 1 in BSHD order: given
    the same O and LSE, the same kernels on the same addresses give
    bit-identical gradients."""
    import scaled_dot_product_07_amd as sdpa
    announce("bwd_varlen one sequence vs dense")
    vi = W.varlen_inputs([600], [600], 4, 128, "bf16", seed=12, poison_tail=False,
                         with_dout=True, h_kv=2)
    q, k, v, do = (x.to(gpu) for x in (vi.q, vi.k, vi.v, vi.dout))
    cu = vi.cu_q.to(gpu)
    o, lse = sdpa.fwd_varlen(q, k, v, cu, cu, 600, 600, scale=0.088, causal=True,
                             window_left=200)
    gv = sdpa.bwd_varlen(q, k, v, o, do, lse, cu, cu, 600, 600, scale=0.088, causal=True,
                         window_left=200)
    dense = lambda t: t.unsqueeze(0).transpose(1, 2)  # (T, h, d) -> (1, h, T, d) view
    gd = sdpa.bwd(dense(q), dense(k), dense(v), dense(o), dense(do),
                  lse.t().contiguous().unsqueeze(0), scale=0.088, causal=True, window_left=200)
    torch.cuda.synchronize()
    for x, y in zip(gv, gd):
        assert torch.equal(x, y.transpose(1, 2).squeeze(0))


def test_varlen_deterministic(gpu):
    import scaled_dot_product_07_amd as sdpa
    announce("bwd_varlen deterministic")
    vi = W.varlen_inputs([300, 45, 700], [300, 45, 700], 4, 64, "bf16", seed=2, with_dout=True,
                         h_kv=1)
    a = _varlen_run(sdpa, vi, 4, 64, "bf16", 0.125, True, False, -1, gpu)
    b = _varlen_run(sdpa, vi, 4, 64, "bf16", 0.125, True, False, -1, gpu)
    # rows past the packed totals are the callers' (uninitialised here)
    for x, y, t in zip(a, b, (vi.total_q, vi.total_kv, vi.total_kv)):
        assert torch.equal(x[:t], y[:t])


def test_varlen_workload_sampled(gpu):
    """The packed workload's shape (32 sequences, lengths ~U[64, 2048], h16
    d128, causal, bf16) through the backward; three sequences and two heads
    checked against the oracle on their own rows."""
    import scaled_dot_product_07_amd as sdpa
    c = W.VARLEN_BF16_32SEQ_H16D128
    announce(f"bwd_varlen workload {c.name}")
    g = W.generator(c.seed)
    lens = W.lengths(c.n_seqs, c.len_lo, c.len_hi, g)
    vi = W.varlen_inputs(lens, lens, c.h, c.d, c.dtype, c.seed + 100_000, with_dout=True)
    dq, dk, dv = _varlen_run(sdpa, vi, c.h, c.d, c.dtype, c.scale, c.causal, False, -1, gpu)
    cu = vi.cu_q.numpy()
    picks = [int(np.argmax(lens.numpy())), int(np.argmin(lens.numpy())), 7]
    for si in picks:
        a, e = int(cu[si]), int(cu[si + 1])
        for hi in (0, c.h - 1):
            sl = lambda t: f64(t[a:e, hi:hi + 1])
            ref = oracle.bwd_varlen(sl(vi.q), sl(vi.k), sl(vi.v), sl(vi.dout),
                                    np.array([0, e - a], np.int32), np.array([0, e - a], np.int32),
                                    c.scale, c.causal, threads=8)
            _, _, dq_r, dk_r, dv_r = ref
            check_grad(sl(dq), dq_r, f"dQ[seq{si},h{hi}]")
            check_grad(sl(dk), dk_r, f"dK[seq{si},h{hi}]")
            check_grad(sl(dv), dv_r, f"dV[seq{si},h{hi}]")


def test_varlen_without_keys_reads_no_forward_outputs(gpu):
    """A packed batch whose sequences have no keys at all: every dQ row is zero
    and O, dO, the statistic and the workspace may be NULL (they are not read)."""
    import ctypes
    import scaled_dot_product_07_amd as sdpa
    announce("bwd varlen total_kv=0 with NULL forward outputs")
    lib = sdpa._load()
    lens = [40, 3, 0, 90]
    tq, h, d = sum(lens), 2, 64
    cu_q = W.cu_seqlens(lens).to(gpu)
    cu_kv = torch.zeros(len(lens) + 1, dtype=torch.int32, device=gpu)
    q = torch.randn(tq, h, d, dtype=torch.bfloat16, device=gpu)
    dq = torch.full_like(q, 9.0)
    st3 = lambda t: (ctypes.c_int64 * 3)(*t.stride())  # noqa: E731
    z3 = (ctypes.c_int64 * 3)(h * d, d, 1)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.sdpa_bwd_varlen(p(q), None, None, None, None, None, p(dq), None, None, p(cu_q),
                             p(cu_kv), len(lens), tq, 0, max(lens), 0, None, 0, 2, h, h, d,
                             st3(q), z3, z3, z3, z3, st3(dq), z3, z3, 0.125, 1, 0, -1,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, sdpa.last_error()
    torch.cuda.synchronize()
    assert torch.all(dq == 0)
