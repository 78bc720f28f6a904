"""GPU check of sdpa_bwd_ex_noalloc, the dense backward that allocates nothing
(its workspace is the library's fixed per-device array), against sdpa_bwd_ex
with a workspace of the caller's: two calls in a row on the same array, the
second on a smaller problem, each bit-identical to sdpa_bwd_ex (same kernels,
same launch shapes; every workspace value read is written by the same call, so
what the first call left in the array cannot show in the second). Neither call
may allocate: torch's allocator statistics and the device's free memory are
unchanged across the two calls.
"""

import pytest
import torch

import workloads as W
from tests.parity import announce

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, b, h, h_kv, s_q, s_kv, d, causal, bottom_right, window_left, layout
    ("bf16", 2, 8, 2, 700, 700, 64, True, False, -1, "bhsd"),
    ("fp16", 1, 2, 1, 300, 420, 128, True, True, 100, "bshd"),
]


def _inputs(case, dev):
    dt, b, h, h_kv, sq, skv, d, causal, br, window, layout = case
    q, k, v, do = W.dense_inputs(b, h, sq, skv, d, dt, layout, seed=901 + sq + d,
                                 with_dout=True)
    k, v = k[:, :h_kv], v[:, :h_kv]
    return [x.to(dev) for x in (q, k, v, do)]


def _prepared(case, dev):
    import scaled_dot_product_07_amd as sdpa
    dt, b, h, h_kv, sq, skv, d, causal, br, window, layout = case
    q, k, v, do = _inputs(case, dev)
    opts = dict(scale=0.11, causal=causal, bottom_right=br, window_left=window)
    o, lse = sdpa.fwd(q, k, v, **opts)
    want = sdpa.bwd(q, k, v, o, do, lse, **opts)
    got = tuple(torch.full_like(x, 1234.0) for x in (q, k, v))
    return (q, k, v, o, do, lse), opts, want, got


def test_noalloc_matches_bwd_ex_on_two_calls(gpu):
    import scaled_dot_product_07_amd as sdpa
    prepared = []
    for case in CASES:
        announce(f"bwd noalloc prepare {case}")
        prepared.append(_prepared(case, gpu))
    torch.cuda.synchronize()
    alloc0 = torch.cuda.memory_allocated(gpu)
    reserved0 = torch.cuda.memory_reserved(gpu)
    free0 = torch.cuda.mem_get_info(gpu)[0]
    for case, (args, opts, want, got) in zip(CASES, prepared):
        announce(f"bwd noalloc {case}")
        sdpa.bwd_noalloc(*args, *got, **opts)
        torch.cuda.synchronize()
    # before the comparisons, which allocate their own small results
    assert torch.cuda.memory_allocated(gpu) == alloc0
    assert torch.cuda.memory_reserved(gpu) == reserved0
    assert torch.cuda.mem_get_info(gpu)[0] == free0
    for case, (args, opts, want, got) in zip(CASES, prepared):
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(g, w), f"{name} differs from sdpa_bwd_ex for {case}"


def test_noalloc_rejects_problems_beyond_the_fixed_workspace(gpu):
    """2^21 + 64 query rows: refused before anything is launched, outputs untouched."""
    import scaled_dot_product_07_amd as sdpa
    announce("bwd noalloc oversize")
    b, h, sq, skv, d = 1, 32, (1 << 16) + 2, 64, 64
    q = torch.zeros(b, h, sq, d, dtype=torch.bfloat16, device=gpu)
    k = torch.zeros(b, h, skv, d, dtype=torch.bfloat16, device=gpu)
    lse = torch.zeros(b, h, sq, dtype=torch.float32, device=gpu)
    dq = torch.full_like(q, 3.0)
    dk = torch.full_like(k, 3.0)
    with pytest.raises(NotImplementedError, match="fixed workspace"):
        sdpa.bwd_noalloc(q, k, k, q, q, lse, dq, dk, dk.clone())
    torch.cuda.synchronize()
    assert torch.all(dq == 3.0) and torch.all(dk == 3.0)
