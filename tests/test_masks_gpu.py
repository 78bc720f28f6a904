"""GPU parity of the forward's band options and grouped-query heads against
the fp64 oracle: bottom-right causal alignment, window_left, and h_kv < h_q
(cudnn-frontend PR #554's sdpa API), dense and packed. Tolerances are the
shared ones in tests/parity.py.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import announce, check_lse, check_o, f64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _inputs(b, h, h_kv, sq, skv, d, dt, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(b, h, sq, d, generator=g).to(DT[dt])
    k = torch.randn(b, h_kv, skv, d, generator=g).to(DT[dt])
    v = torch.randn(b, h_kv, skv, d, generator=g).to(DT[dt])
    return q, k, v


CASES = [
    # dtype, b, h, h_kv, s_q, s_kv, d, causal, bottom_right, window
    ("bf16", 1, 2, 2, 200, 520, 64, True, True, -1),    # bottom-right, s_q < s_kv
    ("bf16", 1, 2, 2, 520, 200, 64, True, True, -1),    # bottom-right, dead rows
    ("fp16", 1, 2, 2, 300, 300, 128, True, True, -1),   # equal lengths = top-left
    ("bf16", 1, 2, 2, 400, 400, 64, True, False, 0),    # window 0: the diagonal only
    ("bf16", 1, 2, 2, 400, 400, 64, True, False, 37),   # window inside one tile
    ("bf16", 2, 2, 2, 700, 700, 128, True, False, 150),  # window over tiles
    ("fp16", 1, 2, 2, 333, 600, 64, True, True, 90),    # window + bottom-right
    ("bf16", 1, 2, 2, 300, 500, 64, False, False, 70),  # left bound only
    ("bf16", 1, 2, 2, 450, 300, 128, False, True, 40),  # left bound only, bottom-right
    ("bf16", 1, 8, 2, 260, 260, 64, True, False, -1),   # GQA, group 4
    ("fp16", 2, 6, 1, 200, 330, 128, False, False, -1),  # MQA
    ("bf16", 1, 4, 2, 300, 700, 64, True, True, 200),   # GQA + band
    ("fp32", 1, 2, 1, 150, 260, 64, True, True, 60),    # fp32 io with every option
    ("fp32", 1, 4, 2, 130, 130, 128, False, False, 20),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_dense_options_vs_oracle(gpu, case):
    import scaled_dot_product_07_amd as sdpa
    dt, b, h, h_kv, sq, skv, d, causal, br, window = case
    announce(f"fwd options {case}")
    q, k, v = _inputs(b, h, h_kv, sq, skv, d, dt, seed=sq * 7 + skv + d + h)
    scale = 1.0 / np.sqrt(d)
    o, lse = sdpa.fwd(q.to(gpu), k.to(gpu), v.to(gpu), scale=scale, causal=causal,
                      bottom_right=br, window_left=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), scale, causal, bottom_right=br,
                                window_left=window)
    check_o(f64(o), o_ref, dt)
    check_lse(f64(lse), lse_ref)


def test_bshd_gqa_window(gpu):
    """Strided (BSHD) tensors with grouped heads and a window."""
    import scaled_dot_product_07_amd as sdpa
    announce("fwd options bshd gqa window")
    q, k, v = _inputs(2, 8, 2, 400, 400, 128, "bf16", seed=77)
    qd, kd, vd = (x.transpose(1, 2).contiguous().transpose(1, 2).to(gpu) for x in (q, k, v))
    o, lse = sdpa.fwd(qd, kd, vd, scale=0.09, causal=True, window_left=100)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), 0.09, True, window_left=100)
    check_o(f64(o), o_ref, "bf16")
    check_lse(f64(lse), lse_ref)


@pytest.mark.parametrize("h,h_kv,causal,br,window", [(4, 2, True, True, -1),
                                                     (4, 4, True, False, 48),
                                                     (8, 1, True, True, 100),
                                                     (2, 2, False, True, 30)])
def test_varlen_options_vs_oracle(gpu, h, h_kv, causal, br, window):
    import scaled_dot_product_07_amd as sdpa
    announce(f"fwd_varlen options h{h} h_kv{h_kv} causal{causal} br{br} w{window}")
    g = torch.Generator().manual_seed(99 + h + h_kv + window)
    lens_q = [70, 1, 300, 129, 64, 5]
    lens_kv = [100, 7, 260, 129, 190, 1]
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(lens_kv)]).astype(np.int32)
    tq, tkv = int(cu_q[-1]), int(cu_kv[-1])
    d = 64
    q = torch.randn(tq + 64, h, d, generator=g).to(torch.bfloat16)
    k = torch.randn(tkv + 64, h_kv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(tkv + 64, h_kv, d, generator=g).to(torch.bfloat16)
    q[tq:] = float("nan")
    k[tkv:] = float("nan")
    v[tkv:] = float("nan")
    cq, ckv = (torch.from_numpy(x).to(gpu) for x in (cu_q, cu_kv))
    o, lse = sdpa.fwd_varlen(q.to(gpu), k.to(gpu), v.to(gpu), cq, ckv, max(lens_q), max(lens_kv),
                             total_q=tq, total_kv=tkv, scale=0.125, causal=causal,
                             bottom_right=br, window_left=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd_varlen(f64(q[:tq]), f64(k[:tkv]), f64(v[:tkv]), cu_q, cu_kv,
                                       0.125, causal, bottom_right=br, window_left=window)
    check_o(f64(o[:tq]), o_ref, "bf16")
    check_lse(f64(lse[:tq]), lse_ref)


def test_option_defaults_match_plain_forward(gpu):
    """Options that change nothing on the headline-shaped workload: bottom-right
    alignment with s_q == s_kv, and a window wider than the keys, describe
    the same band, which the dense forward runs on the same schedule
    (bit-identical results)."""
    import scaled_dot_product_07_amd as sdpa
    announce("fwd options defaults")
    c = W.FWD_BF16_B4H16S1024D64
    q, k, v = (x.to(gpu) for x in W.case_inputs(c))
    a = sdpa.fwd(q, k, v, scale=c.scale, causal=True)
    b2 = sdpa.fwd(q, k, v, scale=c.scale, causal=True, bottom_right=True)  # s_q == s_kv
    b3 = sdpa.fwd(q, k, v, scale=c.scale, causal=True, window_left=4096)   # wider than the keys
    torch.cuda.synchronize()
    assert torch.equal(a[0], b2[0]) and torch.equal(a[1], b2[1])
    assert torch.equal(a[0], b3[0]) and torch.equal(a[1], b3[1])
