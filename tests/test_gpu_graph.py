"""GPU: the entry points under HIP graph capture.  The library allocates
nothing and issues no memset, so its calls can be captured with
torch.cuda.graph; each graph is replayed several times, with eager work and
synchronizations between the replays, and every replay must equal the
eager result bit for bit (the kernels are deterministic)."""
import pytest
import torch

import x3_conv2d_epilogue_amd as x3
from x3_conv2d_epilogue_amd.synthetic import WORKLOADS, make_inputs, random_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def _check_replays(make_call, n_replays=3):
    """make_call(out) enqueues one call writing `out`; returns out's eager
    value and checks every graph replay against it."""
    out_eager = make_call(None)
    torch.cuda.synchronize()
    ref = out_eager.clone()
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # (warm-up on the capture stream, as torch advises)
        make_call(out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        make_call(out)
    for r in range(n_replays):
        out.fill_(float("nan"))
        # eager work between the replays
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs from the eager result"
        assert torch.isfinite(junk)


def test_graph_tiny_min_tanh2():
    d = _dev(make_inputs(WORKLOADS["tiny_min_tanh2"]))

    def call(out):
        return x3.conv3x3_min_tanh2(d["x"], d["weight"], d["bias"], out=out)
    _check_replays(call)


def test_graph_gn_with_workspace_and_noalloc():
    d = _dev(random_case("gn_scale_pool_clamp", 4, 8, 34, 70, 64, seed=700))
    ws = torch.empty(x3.gn_workspace_bytes(4, 8, 34, 70, 64, 16, 4), dtype=torch.uint8,
                     device=DEV)

    def call_ws(out):
        return x3.conv3x3_gn_scale_pool_clamp(d["x"], d["weight"], d["bias"], d["gamma"],
                                              d["beta"], d["scale"], 16, 1e-5, 4, -1e3, 1e3,
                                              out=out, workspace=ws)

    def call_na(out):
        return x3.conv3x3_gn_scale_pool_clamp_noalloc(d["x"], d["weight"], d["bias"], d["gamma"],
                                                      d["beta"], d["scale"], 16, 1e-5, 4, -1e3,
                                                      1e3, out=out)
    _check_replays(call_ws)
    _check_replays(call_na)


def test_graph_many_calls_in_one_graph():
    """Twenty tiny calls captured back to back, each into its own output."""
    d = _dev(make_inputs(WORKLOADS["tiny_min_tanh2"]))
    ref = x3.conv3x3_min_tanh2(d["x"], d["weight"], d["bias"])
    torch.cuda.synchronize()
    outs = [torch.empty_like(ref) for _ in range(20)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for o in outs:
            x3.conv3x3_min_tanh2(d["x"], d["weight"], d["bias"], out=o)
    for _ in range(2):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o in outs:
            assert torch.equal(o, ref)
