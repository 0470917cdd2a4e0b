"""Every entry point's kernels captured in a HIP graph (torch.cuda.graph) and replayed: each
replay, with the program's own eager work and synchronisations in between, gives the eager result
bit for bit. The library queues only kernels on the caller's stream (no memset, no allocation, no
host synchronisation), so a whole call can be captured."""
import numpy as np
import pytest
import torch

from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.inputs import make_inputs, ncssd_inputs, random_orders
from gpu_helpers import IO_NAMES, PARAM_NAMES, to_device

pytestmark = pytest.mark.gpu


def _replays_match(make_call, replays=3):
    """make_call(stream) -> a callable queuing the work on that stream and returning its output."""
    eager_call = make_call(torch.cuda.current_stream().cuda_stream)
    eager = eager_call().clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        captured = make_call(side.cuda_stream)
        captured()                              # one warm-up call on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        captured_call = make_call(torch.cuda.current_stream().cuda_stream)
        out = captured_call()
    for r in range(replays):
        out.fill_(float("nan"))                 # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"
        eager_call()                            # and an eager call of the library itself
        torch.cuda.synchronize()


@pytest.mark.parametrize("io,chunk", [("bf16", 0), ("f32", 48)])
def test_bidirectional_scan_in_a_graph(io, chunk):
    inp = make_inputs(2, 197, 128, 16, io, seed=1)
    dev = to_device(inp, io)
    args = [dev[k] for k in IO_NAMES + PARAM_NAMES]
    _replays_match(lambda s: binding.PreparedCall(*args, chunk_len=chunk, stream=s))


def test_ordered_scan_in_a_graph():
    inp = make_inputs(2, 100, 64, 16, "bf16", seed=2)
    dev = to_device(inp, "bf16")
    args = [dev[k] for k in IO_NAMES + PARAM_NAMES]
    order = torch.from_numpy(random_orders(2, 100, seed=3)).to("cuda:0")
    _replays_match(lambda s: binding.PreparedCall(*args, chunk_len=32, order=order, stream=s))


@pytest.mark.parametrize("chunk", [0, 32])
def test_ncssd_in_a_graph(chunk):
    inp = ncssd_inputs(3, 130, 64, 16, "bf16", seed=4)
    d = {k: torch.from_numpy(inp[k]).to("cuda:0") for k in ("x", "B", "C", "m")}
    for k in ("x", "B", "C"):
        d[k] = d[k].to(torch.bfloat16)
    _replays_match(lambda s: binding.PreparedNcssd(d["x"], d["B"], d["C"], d["m"], chunk_len=chunk, stream=s))
