"""GPU parity of the dense forward (sdpa_fwd) against the fp64 oracle.

Small cases run the whole oracle (several 128-row query tiles and 64-key
tiles, ragged tails, both dtypes of 16 bits, fp32, both head dims, causal and
not, rectangular s_q != s_kv, BSHD strides, negative and zero scale, no keys).
The workloads at full size run in the same launch configuration as the
benchmark and are checked element by element against the oracle over their
whole outputs.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import announce, check_lse, check_o, f64

pytestmark = pytest.mark.gpu


def _run(q, k, v, scale, causal, dev):
    import scaled_dot_product_07_amd as sdpa
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o, lse = sdpa.fwd(qd, kd, vd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


SMALL = [
    # dtype, b, h, s_q, s_kv, d, causal, layout
    ("bf16", 2, 3, 300, 300, 64, True, "bhsd"),
    ("bf16", 2, 3, 300, 300, 64, False, "bhsd"),
    ("fp16", 1, 2, 257, 257, 128, True, "bhsd"),
    ("fp16", 1, 2, 257, 257, 128, False, "bshd"),
    ("bf16", 1, 2, 200, 333, 128, True, "bshd"),
    ("bf16", 1, 2, 333, 200, 64, True, "bhsd"),
    ("bf16", 1, 1, 1, 1, 64, True, "bhsd"),
    ("bf16", 1, 1, 130, 65, 64, False, "bhsd"),
    ("fp32", 1, 2, 190, 190, 64, True, "bhsd"),
    ("fp32", 1, 2, 150, 170, 128, False, "bshd"),
    ("fp32", 1, 1, 129, 129, 128, True, "bhsd"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_small_vs_oracle(gpu, case):
    dt, b, h, sq, skv, d, causal, layout = case
    announce(f"fwd small {case}")
    q, k, v = W.dense_inputs(b, h, sq, skv, d, dt, layout, seed=7 + sq + d)
    scale = 1.0 / np.sqrt(d)
    o, lse = _run(q, k, v, scale, causal, gpu)
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), scale, causal)
    check_o(f64(o), o_ref, dt)
    check_lse(f64(lse), lse_ref)


# More pair units than compute units: the one-tile workgroups run in rounds
# of twice the CU count with a partial last round, and an odd tile count
# (3 per head here) leaves one pair of each head without its second tile.
ROUNDS = [
    # dtype, b, h, s_q, s_kv, d, causal, layout
    ("bf16", 1, 150, 384, 384, 64, True, "bhsd"),
    ("bf16", 2, 75, 384, 200, 64, False, "bhsd"),
    ("fp16", 1, 130, 384, 384, 128, True, "bshd"),
]


@pytest.mark.parametrize("case", ROUNDS, ids=lambda c: "-".join(map(str, c)))
def test_grid_rounds_vs_oracle(gpu, case):
    dt, b, h, sq, skv, d, causal, layout = case
    announce(f"fwd rounds {case}")
    q, k, v = W.dense_inputs(b, h, sq, skv, d, dt, layout, seed=11 + h + d)
    scale = 1.0 / np.sqrt(d)
    o, lse = _run(q, k, v, scale, causal, gpu)
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), scale, causal)
    check_o(f64(o), o_ref, dt)
    check_lse(f64(lse), lse_ref)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.9])
def test_scale_sign_and_zero(gpu, scale):
    announce(f"fwd scale={scale}")
    q, k, v = W.dense_inputs(1, 2, 150, 150, 64, "bf16", "bhsd", seed=31)
    for causal in (False, True):
        o, lse = _run(q, k, v, scale, causal, gpu)
        o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), scale, causal)
        check_o(f64(o), o_ref, "bf16")
        check_lse(f64(lse), lse_ref)


RISING = [
    # dtype, s_q, s_kv, d, causal
    ("bf16", 300, 300, 64, True),
    ("fp16", 200, 520, 64, False),
    ("bf16", 257, 257, 128, True),
    ("fp16", 130, 390, 128, False),
]


@pytest.mark.parametrize("case", RISING, ids=lambda c: "-".join(map(str, c)))
def test_rising_scores_raise_offsets(gpu, case):
    """Key rows scaled up along the sequence (x1 .. x24), so that the scores of
    later key tiles rise tens of log2 units above the first tile's: the P of
    such tiles overflow the offset taken so far (past the 16-bit range for
    fp16), and every such tile must raise the row's offset and rescale O and
    l before its P.V. The oracle computes the definition directly."""
    dt, sq, skv, d, causal = case
    announce(f"fwd rising scores {case}")
    q, k, v = W.dense_inputs(1, 2, sq, skv, d, dt, "bhsd", seed=401 + skv + d)
    ramp = 1.0 + 23.0 * torch.arange(skv, dtype=torch.float32) / max(skv - 1, 1)
    k = (k.float() * ramp[None, None, :, None]).to(k.dtype)
    scale = 1.0 / np.sqrt(d)
    o, lse = _run(q, k, v, scale, causal, gpu)
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), scale, causal)
    check_o(f64(o), o_ref, dt)
    check_lse(f64(lse), lse_ref)


@pytest.mark.parametrize("parity", [0, 1])
@pytest.mark.parametrize("dt,causal", [("bf16", True), ("fp16", False)])
def test_rises_on_alternate_key_tiles(gpu, parity, dt, causal):
    """Scores that jump up only on every other 64-key tile (the rest scaled
    down), so that the offset has to be raised on tiles of one parity of the
    key loop only: after the first tile of a pair of steps, or after the
    second, in turn for the two parities."""
    announce(f"fwd alternating rises parity={parity} {dt} causal={causal}")
    s, d = 460, 64
    q, k, v = W.dense_inputs(1, 2, s, s, d, dt, "bhsd", seed=433 + parity)
    tile = torch.arange(s) // 64
    f = torch.where(tile % 2 == parity, 1.0 + 5.0 * tile.float(), torch.full((s,), 0.5))
    k = (k.float() * f[None, None, :, None]).to(k.dtype)
    scale = 1.0 / np.sqrt(d)
    o, lse = _run(q, k, v, scale, causal, gpu)
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), scale, causal)
    check_o(f64(o), o_ref, dt)
    check_lse(f64(lse), lse_ref)


def test_no_keys_gives_dead_rows(gpu):
    import scaled_dot_product_07_amd as sdpa
    announce("fwd s_kv=0")
    q = torch.randn(1, 2, 70, 64, dtype=torch.bfloat16, device=gpu)
    k = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=gpu)
    o = torch.full_like(q, 7.0)
    o, lse = sdpa.fwd(q, k, k, causal=False, out=o)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_output_strides_and_lse_optional(gpu):
    """O written through a non-contiguous (BSHD) view; lse=None path."""
    import scaled_dot_product_07_amd as sdpa
    announce("fwd strided out")
    q, k, v = W.dense_inputs(2, 4, 140, 140, 64, "bf16", "bhsd", seed=41)
    qd, kd, vd = (x.to(gpu) for x in (q, k, v))
    out = torch.empty(2, 140, 4, 64, dtype=torch.bfloat16, device=gpu).transpose(1, 2)
    o, lse = sdpa.fwd(qd, kd, vd, causal=True, out=out, return_lse=False)
    torch.cuda.synchronize()
    assert lse is None and o.data_ptr() == out.data_ptr()
    o_ref, _ = oracle.fwd(f64(q), f64(k), f64(v), 1 / 8, True)
    check_o(f64(o), o_ref, "bf16")


def test_guard_band_untouched(gpu):
    """Nothing is written outside O and LSE: canaries around both survive."""
    import scaled_dot_product_07_amd as sdpa
    announce("fwd guard band")
    b, h, s, d = 1, 2, 200, 64
    q, k, v = (x.to(gpu) for x in W.dense_inputs(b, h, s, s, d, "bf16", "bhsd", seed=51))
    n = b * h * s * d
    obuf = torch.full((n + 4096,), 123.0, dtype=torch.bfloat16, device=gpu)
    lbuf = torch.full((b * h * s + 1024,), 321.0, dtype=torch.float32, device=gpu)
    o = obuf[:n].view(b, h, s, d)
    lse = lbuf[:b * h * s].view(b, h, s)
    sdpa.fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[n:] == 123.0) and torch.all(lbuf[b * h * s:] == 321.0)


def test_deterministic(gpu):
    import scaled_dot_product_07_amd as sdpa
    announce("fwd determinism")
    q, k, v = (x.to(gpu) for x in W.dense_inputs(2, 4, 513, 513, 128, "bf16", "bhsd", seed=61))
    o1, l1 = sdpa.fwd(q, k, v, causal=True)
    o2, l2 = sdpa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---- the workloads at full size ---------------------------------------------

def test_workload_fp32_b1h2s128d64(gpu):
    c = W.FWD_FP32_B1H2S128D64
    announce(c.name)
    q, k, v = W.case_inputs(c)
    o, lse = _run(q, k, v, c.scale, c.causal, gpu)
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), c.scale, c.causal)
    check_o(f64(o), o_ref, "fp32")
    check_lse(f64(lse), lse_ref)


def test_workload_bf16_b4h16s1024d64_full(gpu):
    """The headline workload: the whole output against the oracle."""
    c = W.FWD_BF16_B4H16S1024D64
    announce(c.name)
    q, k, v = W.case_inputs(c)
    o, lse = _run(q, k, v, c.scale, c.causal, gpu)
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), c.scale, c.causal)
    check_o(f64(o), o_ref, "bf16")
    check_lse(f64(lse), lse_ref)


@pytest.mark.parametrize("case", [W.FWD_BF16_B2H16S4096D128, W.FWD_FP16_B2H16S4096D128],
                         ids=["bf16", "fp16"])
def test_workload_b2h16s4096d128_bshd_full(gpu, case):
    """The non-causal BSHD workload at full size, in the benchmark's launch
    configuration: every output element and every statistic against the oracle."""
    announce(case.name)
    q, k, v = W.case_inputs(case)
    assert q.stride() == (4096 * 16 * 128, 128, 16 * 128, 1)  # BSHD viewed as BHSD
    o, lse = _run(q, k, v, case.scale, case.causal, gpu)
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), case.scale, case.causal)
    check_o(f64(o), o_ref, case.dtype)
    check_lse(f64(lse), lse_ref)
