"""Stream and graph semantics of the entry points: every launch goes to the caller's stream
(torch's current stream in the binding), so the work can run on a side stream or be captured
into a HIP graph and replayed.

- A side stream (default priority) gives the default stream's results bit for bit.
- A captured fwd + bwd, replayed several times with the inputs rewritten eagerly between
  replays (the graph reads whatever the buffers hold), matches an eager call on the same
  contents every time, and the first replay also matches the oracle.
"""
import pytest

import oracle
import workloads
from parity_helpers import assert_close, say, to_np64

pytestmark = pytest.mark.gpu

W = workloads.Workload("graph", "bf16", 1, 4, 2, 333, 333, 128, True, seed=6100)


def eager(fab, q, k, v, do, window=0):
    o, lse = fab.fwd(q, k, v, causal=W.causal, scale=W.scale, window_size=window)
    dq, dk, dv = fab.bwd(do, q, k, v, o, lse, causal=W.causal, scale=W.scale, window_size=window)
    return o, lse, dq, dk, dv


def test_side_stream_matches_default_stream(fab):
    import torch
    say("[case] side stream, bf16 D=128")
    dev = torch.device("cuda:0")
    q, k, v, do = (x.to(dev) for x in workloads.make_inputs(W))
    ref = eager(fab, q, k, v, do)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)  # default priority
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        got = eager(fab, q, k, v, do)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("window", [0, 70])
def test_graph_replays_match_eager_calls(fab, window):
    import torch
    say(f"[case] graph capture and replay, bf16 D=128 window={window}")
    dev = torch.device("cuda:0")
    q0, k0, v0, do0 = workloads.make_inputs(W)
    q, k, v, do = (x.to(dev) for x in (q0, k0, v0, do0))
    # warm up on a side stream before capture (library load, allocator pools)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        eager(fab, q, k, v, do, window)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = eager(fab, q, k, v, do, window)
    torch.cuda.synchronize()

    gen = torch.Generator(device=dev)
    gen.manual_seed(6101)
    for rep in range(3):
        if rep > 0:  # new contents in the same buffers, written eagerly between replays
            for t in (q, k, v, do):
                t.copy_(torch.randn(t.shape, generator=gen, device=dev, dtype=torch.float32).to(t.dtype))
        g.replay()
        torch.cuda.synchronize()
        ref = eager(fab, q, k, v, do, window)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), outs, ref):
            assert torch.equal(a, b), (rep, name)
        if rep == 0:
            r = oracle.attention_grads(q0, k0, v0, do0, W.causal, W.scale, window=window)
            for name, a in zip(("o", "lse", "dq", "dk", "dv"), outs):
                assert_close(name, to_np64(a), r[name], "fp32" if name == "lse" else "bf16")
