"""GPU parity of the packed THD forward (sdpa_fwd_varlen) against the fp64 oracle.

Every packed buffer is allocated with a NaN-poisoned capacity tail (rows past
the packed total), and O / LSE tails are pre-filled with a sentinel: the
kernels must neither read the poison (O stays finite and matches) nor write
past the total (the sentinels survive).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import announce, check_lse, check_o, f64

pytestmark = pytest.mark.gpu


def _run(inp, h, d, scale, causal, dev, max_q=None, max_kv=None):
    import scaled_dot_product_07_amd as sdpa
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    cu_q, cu_kv = inp.cu_q.to(dev), inp.cu_kv.to(dev)
    o = torch.full_like(q, 77.0)
    lse = torch.full((q.shape[0], h), 55.0, dtype=torch.float32, device=dev)
    max_q = int(inp.lens_q.max()) if max_q is None else max_q
    max_kv = max(int(inp.lens_kv.max()), 1) if max_kv is None else max_kv
    sdpa.fwd_varlen(q, k, v, cu_q, cu_kv, max_q, max_kv, total_q=inp.total_q,
                    total_kv=inp.total_kv, scale=scale, causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def _check_all(inp, o, lse, scale, causal, dt):
    tq = inp.total_q
    o_ref, lse_ref = oracle.fwd_varlen(f64(inp.q[:tq]), f64(inp.k[:inp.total_kv]),
                                       f64(inp.v[:inp.total_kv]), inp.cu_q.numpy(),
                                       inp.cu_kv.numpy(), scale, causal)
    check_o(f64(o[:tq]), o_ref, dt)
    check_lse(f64(lse[:tq]), lse_ref)
    assert torch.all(o[tq:] == 77.0), "O written past the packed total"
    assert torch.all(lse[tq:] == 55.0), "LSE written past the packed total"


SMALL = [
    ("bf16", 64, True), ("bf16", 64, False), ("bf16", 128, True), ("fp16", 128, False),
    ("fp32", 64, True), ("fp32", 128, False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_small_vs_oracle(gpu, case):
    dt, d, causal = case
    lens = [5, 1, 130, 257, 0, 64, 200]
    announce(f"varlen small {case} lens={lens}")
    inp = W.varlen_inputs(lens, lens, 3, d, dt, seed=300 + d)
    o, lse = _run(inp, 3, d, 1 / np.sqrt(d), causal, gpu)
    _check_all(inp, o, lse, 1 / np.sqrt(d), causal, dt)


@pytest.mark.parametrize("case", [("bf16", 64), ("fp16", 128)], ids=lambda c: "-".join(map(str, c)))
def test_causal_pairs_within_each_sequence(gpu, case):
    """Causal units pair the query tiles of each sequence among themselves
    (tile n_s-1-i with tile i of the sequence's own n_s tiles), and the
    workgroups take the live pairs of all sequences heaviest first: every
    tile count from 0 to 9, odd and even, in one pack, so that pairs, lone
    middle tiles and sequences without tiles all occur."""
    dt, d = case
    lens = [1100, 0, 129, 700, 385, 1, 900, 256, 1024, 640, 513, 128, 64, 300, 830]
    announce(f"varlen causal tile pairs {case} lens={lens}")
    inp = W.varlen_inputs(lens, lens, 2, d, dt, seed=410 + d)
    o, lse = _run(inp, 2, d, 1 / np.sqrt(d), True, gpu)
    _check_all(inp, o, lse, 1 / np.sqrt(d), True, dt)


def test_unequal_q_kv_lengths_and_dead_rows(gpu):
    """Query and key lengths differ per sequence; a sequence with no keys gives dead rows."""
    lens_q = [40, 3, 129, 0, 70]
    lens_kv = [90, 0, 64, 10, 300]
    announce(f"varlen unequal q={lens_q} kv={lens_kv}")
    inp = W.varlen_inputs(lens_q, lens_kv, 2, 64, "bf16", seed=401)
    for causal in (False, True):
        o, lse = _run(inp, 2, 64, 0.125, causal, gpu)
        _check_all(inp, o, lse, 0.125, causal, "bf16")


LIVE_UNITS = [
    # dtype, d, causal, window_left
    ("bf16", 64, True, -1), ("bf16", 64, False, -1), ("fp16", 128, True, -1),
    ("bf16", 64, True, 100), ("fp32", 64, True, -1), ("fp32", 128, False, -1),
]


@pytest.mark.parametrize("case", LIVE_UNITS, ids=lambda c: "-".join(map(str, c)))
def test_many_sequences_live_units(gpu, case):
    """150 sequences (more than one wave's 64 lanes, so the unit search reads
    cu_seqlens in several chunks), a fifth of them empty, lengths 0 .. 400:
    the grid holds total_q / 256 (or / 128) + num_seqs units per head and
    each workgroup finds its unit on the device. Every row of every
    sequence must be written (O and LSE start as sentinels) and match the
    oracle; rows past the total stay untouched."""
    import scaled_dot_product_07_amd as sdpa
    dt, d, causal, window = case
    g = np.random.default_rng(77 + d)
    lens = g.integers(0, 401, size=150)
    lens[g.random(150) < 0.2] = 0
    lens = lens.tolist()
    announce(f"varlen live units {case} n=150 T={sum(lens)}")
    h = 2
    inp = W.varlen_inputs(lens, lens, h, d, dt, seed=500 + d)
    q, k, v = (x.to(gpu) for x in (inp.q, inp.k, inp.v))
    o = torch.full_like(q, 77.0)
    lse = torch.full((q.shape[0], h), 55.0, dtype=torch.float32, device=gpu)
    sdpa.fwd_varlen(q, k, v, inp.cu_q.to(gpu), inp.cu_kv.to(gpu), max(lens), max(lens),
                    total_q=inp.total_q, total_kv=inp.total_kv, scale=1 / np.sqrt(d),
                    causal=causal, window_left=window, out=o, lse=lse)
    torch.cuda.synchronize()
    tq = inp.total_q
    o_ref, lse_ref = oracle.fwd_varlen(f64(inp.q[:tq]), f64(inp.k[:tq]), f64(inp.v[:tq]),
                                       inp.cu_q.numpy(), inp.cu_kv.numpy(), 1 / np.sqrt(d),
                                       causal, window_left=window)
    check_o(f64(o[:tq]), o_ref, dt)
    check_lse(f64(lse[:tq]), lse_ref)
    assert torch.all(o[tq:] == 77.0) and torch.all(lse[tq:] == 55.0)


def test_one_live_sequence_among_many_empty(gpu):
    """200 sequences of which only the 137th has rows: almost every workgroup
    of the grid (total_q / 256 + 200 per head) finds no unit and exits."""
    lens = [0] * 200
    lens[137] = 700
    announce("varlen one live sequence of 200")
    inp = W.varlen_inputs(lens, lens, 3, 64, "bf16", seed=503)
    o, lse = _run(inp, 3, 64, 0.125, True, gpu)
    _check_all(inp, o, lse, 0.125, True, "bf16")


def test_loose_max_seqlen_bound(gpu):
    """max_seqlen_q larger than the longest sequence only adds empty tiles."""
    lens = [33, 250, 17]
    announce("varlen loose bound")
    inp = W.varlen_inputs(lens, lens, 2, 128, "bf16", seed=402)
    o, lse = _run(inp, 2, 128, 0.1, True, gpu, max_q=inp.total_q, max_kv=4096)
    _check_all(inp, o, lse, 0.1, True, "bf16")


def test_workload_varlen_32seq_full(gpu):
    """The packed workload at full size (32 sequences, h16 d128, causal bf16) in
    the benchmark's launch configuration: every row of every sequence and head
    against the oracle, and the NaN-poisoned capacity tail never reaches O."""
    c = W.VARLEN_BF16_32SEQ_H16D128
    inp = W.varlen_case_inputs(c)
    announce(f"{c.name} T={inp.total_q}")
    o, lse = _run(inp, c.h, c.d, c.scale, c.causal, gpu)
    tq = inp.total_q
    o64, l64 = f64(o[:tq]), f64(lse[:tq])
    assert np.all(np.isfinite(o64)), "NaN from the poisoned capacity tail reached O"
    assert torch.all(o[tq:] == 77.0) and torch.all(lse[tq:] == 55.0)
    o_ref, l_ref = oracle.fwd_varlen(f64(inp.q[:tq]), f64(inp.k[:tq]), f64(inp.v[:tq]),
                                     inp.cu_q.numpy(), inp.cu_kv.numpy(), c.scale, True)
    check_o(o64, o_ref, "bf16")
    check_lse(l64, l_ref)
