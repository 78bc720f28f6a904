"""Launch discipline of every entry point: the calls only enqueue work on the
caller's stream, never synchronise with the host and never allocate.

cudnn-frontend PR #554 asks for exactly this (its host-sync commit: prove
that the sdpa path makes no host synchronisation and keep the check as a
test). Two checks per entry point:
  * torch's sync debug mode set to "error" around the calls: any host sync
    that torch performs in the binding raises;
  * the calls are issued on a side stream kept busy by a spin kernel queued
    just before them: if any call synchronised the host with the device
    (inside the library as well), the stream would be idle when the calls
    return. Afterwards the side stream's results must equal the default
    stream's bit for bit.
A third check captures every entry point in one HIP graph and replays it:
each replay must equal the eager results bit for bit.
"""

import pytest
import torch

import workloads as W
from tests.parity import announce

pytestmark = pytest.mark.gpu


def _inputs(dev):
    q, k, v, do = (x.to(dev) for x in W.dense_inputs(2, 2, 200, 200, 64, "bf16", "bhsd", seed=91,
                                                     with_dout=True))
    lens = [70, 0, 130]
    vi = W.varlen_inputs(lens, lens, 2, 64, "bf16", seed=92, poison_tail=False, with_dout=True)
    tq, tk, tv, tdo = (x.to(dev) for x in (vi.q, vi.k, vi.v, vi.dout))
    cu = vi.cu_q.to(dev)
    q8, k8, v8 = (x.to(torch.float8_e4m3fn) for x in (q, k, v))
    t8q, t8k, t8v = (x.to(torch.float8_e4m3fn) for x in (tq, tk, tv))
    return dict(q=q, k=k, v=v, do=do, tq=tq, tk=tk, tv=tv, tdo=tdo, cu=cu, mx=130, q8=q8, k8=k8,
                v8=v8, t8q=t8q, t8k=t8k, t8v=t8v)


def _outputs(x):
    """Every output buffer, allocated up front."""
    e = torch.empty_like
    f32 = dict(dtype=torch.float32, device=x["q"].device)
    bf = dict(dtype=torch.bfloat16, device=x["q"].device)
    import scaled_dot_product_07_amd as sdpa
    ws = torch.empty(sdpa.bwd_workspace_size(2, 2, 200, 64, torch.bfloat16), dtype=torch.uint8,
                     device=x["q"].device)
    wsv = torch.empty(sdpa.bwd_workspace_size(1, 2, x["tq"].shape[0], 64, torch.bfloat16),
                      dtype=torch.uint8, device=x["q"].device)
    return dict(o=e(x["q"]), lse=torch.empty(2, 2, 200, **f32), to=e(x["tq"]),
                tlse=torch.empty(x["tq"].shape[0], 2, **f32), dq=e(x["q"]), dk=e(x["k"]),
                dv=e(x["v"]), tdq=e(x["tq"]), tdk=e(x["tk"]), tdv=e(x["tv"]), ws=ws, wsv=wsv,
                o8=torch.empty(x["q"].shape, **bf), to8=torch.empty(x["tq"].shape, **bf),
                amax=torch.empty(1, **f32))


def _run_all(sdpa, x, y, stream):
    """Every entry point, in dependency order, on `stream`."""
    sdpa.fwd(x["q"], x["k"], x["v"], causal=True, out=y["o"], lse=y["lse"], stream=stream)
    sdpa.fwd_varlen(x["tq"], x["tk"], x["tv"], x["cu"], x["cu"], x["mx"], x["mx"], causal=True,
                    out=y["to"], lse=y["tlse"], stream=stream)
    sdpa.bwd(x["q"], x["k"], x["v"], y["o"], x["do"], y["lse"], causal=True, dq=y["dq"],
             dk=y["dk"], dv=y["dv"], workspace=y["ws"], stream=stream)
    sdpa.bwd_varlen(x["tq"], x["tk"], x["tv"], y["to"], x["tdo"], y["tlse"], x["cu"], x["cu"],
                    x["mx"], x["mx"], causal=True, dq=y["tdq"], dk=y["tdk"], dv=y["tdv"],
                    workspace=y["wsv"], stream=stream)
    sdpa.fwd_fp8(x["q8"], x["k8"], x["v8"], causal=True, out=y["o8"], return_lse=False,
                 amax_o=y["amax"], stream=stream)
    sdpa.fwd_fp8_varlen(x["t8q"], x["t8k"], x["t8v"], x["cu"], x["cu"], x["mx"], x["mx"],
                        causal=True, out=y["to8"], return_lse=False, stream=stream)


def test_no_host_sync_and_caller_stream(gpu):
    import scaled_dot_product_07_amd as sdpa
    announce("launch discipline: sync debug mode, busy side stream")
    x = _inputs(gpu)
    ref = _outputs(x)
    _run_all(sdpa, x, ref, torch.cuda.current_stream())
    torch.cuda.synchronize()

    got = _outputs(x)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    torch.cuda.set_sync_debug_mode("error")
    try:
        with torch.cuda.stream(side):
            torch.cuda._sleep(200_000_000)  # a bounded spin that keeps `side` busy
            _run_all(sdpa, x, got, side)
    finally:
        torch.cuda.set_sync_debug_mode(0)
    still_busy = not side.query()
    side.synchronize()
    assert still_busy, "the side stream drained while the calls ran: some call synchronised"
    for key in ref:
        if key in ("ws", "wsv"):
            continue
        assert torch.equal(got[key], ref[key]), f"{key} differs between the two streams"


def test_graph_replay_matches_eager(gpu):
    """Every entry point captured in one HIP graph (as a caller that replays a
    step does) gives the eager results on every replay. Between replays the
    outputs and workspaces are refilled with junk by ordinary eager work, so
    a replay that skipped a write, or read what an earlier one left, shows."""
    import scaled_dot_product_07_amd as sdpa
    announce("launch discipline: graph capture, three replays against eager")
    x = _inputs(gpu)
    ref = _outputs(x)
    _run_all(sdpa, x, ref, torch.cuda.current_stream())
    torch.cuda.synchronize()

    got = _outputs(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run_all(sdpa, x, got, side)  # one eager pass on the capture stream first
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run_all(sdpa, x, got, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        for key, t in got.items():
            if t.dtype == torch.uint8:
                t.fill_(255)
            else:
                t.fill_(float("nan") if rep % 2 == 0 else -3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in ref:
            if key in ("ws", "wsv"):
                continue
            assert torch.equal(got[key], ref[key]), f"replay {rep}: {key} differs from eager"
