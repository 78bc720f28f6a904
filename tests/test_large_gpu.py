"""GPU parity at sizes whose tensors span more than 2 GiB, so that every tile
base, row offset and statistic index past 2^31 bytes is exercised: keys
1,048,576 long in BSHD order (16 heads x 64 d x 2 B per token: K and V are
2 GiB each, their last rows start past 2^31 bytes), a packed batch whose keys
total 1.2M tokens (2.4 GiB), and the backward with 64 heads of 300,000 keys
(2.3 GiB per tensor). Inputs are
drawn on the device from a fixed seed; the oracle runs on the bytes of the
checked heads, copied back: sampled query rows of the forward (non-causal,
so every row reads every key), all of one head's dQ, dK, dV.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import announce, check_grad, check_lse, check_o, f64

pytestmark = pytest.mark.gpu

S_KV = 1 << 20
H, D, S_Q = 16, 64, 256


def _dense_bshd(gpu, seed):
    # (b, s, h, d) allocations viewed as logical (b, h, s, d)
    q = W.device_normal((1, S_Q, H, D), "bf16", seed, gpu).transpose(1, 2)
    k = W.device_normal((1, S_KV, H, D), "bf16", seed + 1, gpu).transpose(1, 2)
    v = W.device_normal((1, S_KV, H, D), "bf16", seed + 2, gpu).transpose(1, 2)
    return q, k, v


def test_forward_keys_past_2gib(gpu):
    import scaled_dot_product_07_amd as sdpa
    announce(f"fwd large: b1 h{H} s_q {S_Q} s_kv {S_KV} d{D} BSHD, K and V 2 GiB each")
    q, k, v = _dense_bshd(gpu, 7001)
    assert k.untyped_storage().nbytes() == 2 << 30
    scale = 1.0 / np.sqrt(D)
    o, lse = sdpa.fwd(q, k, v, scale=scale, causal=False)
    torch.cuda.synchronize()
    rows = [0, 1, 129, 255]
    for hd in (0, 9, 15):
        qh = f64(q[:, hd:hd + 1, rows])
        kh, vh = f64(k[:, hd:hd + 1]), f64(v[:, hd:hd + 1])
        o_ref, lse_ref = oracle.fwd(qh, kh, vh, scale, False)
        check_o(f64(o[:, hd:hd + 1, rows]), o_ref, "bf16")
        check_lse(f64(lse[:, hd:hd + 1, rows]), lse_ref)


def test_packed_forward_keys_past_2gib(gpu):
    import scaled_dot_product_07_amd as sdpa
    lens_q, lens_kv = [128, 200], [700_000, 500_000]
    announce(f"fwd_varlen large: q {lens_q} kv {lens_kv} h{H} d{D}, K and V 2.4 GiB each")
    tq, tkv = sum(lens_q), sum(lens_kv)
    q = W.device_normal((tq, H, D), "bf16", 7101, gpu)
    k = W.device_normal((tkv, H, D), "bf16", 7102, gpu)
    v = W.device_normal((tkv, H, D), "bf16", 7103, gpu)
    cu_q = torch.tensor([0, 128, 328], dtype=torch.int32)
    cu_kv = torch.tensor([0, 700_000, 1_200_000], dtype=torch.int32)
    scale = 0.1
    o, lse = sdpa.fwd_varlen(q, k, v, cu_q.to(gpu), cu_kv.to(gpu), max(lens_q), max(lens_kv),
                             scale=scale, causal=False)
    torch.cuda.synchronize()
    for hd in (0, 15):
        o_ref, lse_ref = oracle.fwd_varlen(f64(q[:, hd:hd + 1]), f64(k[:, hd:hd + 1]),
                                           f64(v[:, hd:hd + 1]), cu_q.numpy(), cu_kv.numpy(),
                                           scale, False)
        check_o(f64(o[:, hd:hd + 1]), o_ref, "bf16")
        check_lse(f64(lse[:, hd:hd + 1]), lse_ref)


def test_backward_keys_past_2gib(gpu):
    """64 heads x 64 d per token (8 KB), 300,000 keys: K, V, dK, dV are 2.3 GiB
    each; all of dQ, dK, dV of the first and the last head against the oracle."""
    import scaled_dot_product_07_amd as sdpa
    h, s_q, s_kv = 64, 128, 300_000
    announce(f"bwd large: b1 h{h} s_q {s_q} s_kv {s_kv} d{D} BSHD, dK and dV 2.3 GiB each")
    q = W.device_normal((1, s_q, h, D), "bf16", 7201, gpu).transpose(1, 2)
    k = W.device_normal((1, s_kv, h, D), "bf16", 7202, gpu).transpose(1, 2)
    v = W.device_normal((1, s_kv, h, D), "bf16", 7203, gpu).transpose(1, 2)
    do = W.device_normal((1, s_q, h, D), "bf16", 7204, gpu).transpose(1, 2)
    scale = 1.0 / np.sqrt(D)
    o, lse = sdpa.fwd(q, k, v, scale=scale, causal=False)
    dq, dk, dv = sdpa.bwd(q, k, v, o, do, lse, scale=scale, causal=False)
    torch.cuda.synchronize()
    assert dk.stride() == k.stride() and dk.untyped_storage().nbytes() > 2 << 30
    for hd in (0, h - 1):
        sl = slice(hd, hd + 1)
        _, _, dq_r, dk_r, dv_r = oracle.bwd(f64(q[:, sl]), f64(k[:, sl]), f64(v[:, sl]),
                                            f64(do[:, sl]), scale, False)
        check_grad(f64(dq[:, sl]), dq_r, "dQ")
        check_grad(f64(dk[:, sl]), dk_r, "dK")
        check_grad(f64(dv[:, sl]), dv_r, "dV")
