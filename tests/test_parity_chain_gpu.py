"""The one-pass chunked scan (bidirectional plans of 2..16 chunks, one kernel per call), on the GPU
through the C ABI: chunks hand their aggregates to the later chunks of their sequence through the
workspace within one kernel, marked by a tag unique to the kernel dispatch.

What these tests pin down beyond the plain parity tests:
* the workspace's previous contents never matter: random bytes, all-ones bytes, or the aggregates
  and tags a previous call left there with other inputs -- the output equals the float64 oracle
  and, bit for bit, the output of the same call on a fresh workspace;
* a queue of calls on one workspace, each with its own inputs and no synchronisation in between,
  gives every call its own result bit for bit (no call reads another call's aggregates);
* two streams, each with its own workspace, interleaved, likewise;
* the plan: one kernel per call, a tag word per (direction, sequence, chunk, channel block) in the
  workspace after the other regions;
* the same for the forward-only scan (vimscan_fwd), whose chunked plans of up to 16 chunks are one
  kernel as well;
* no wait of any of these calls (or of any earlier test in the process) gave up after its bound
  (vimscan_wait_timeouts stays 0).
Shapes: ragged last chunks, a ragged last channel block and an odd channel-block count (a spare
wave that neither publishes nor waits), 2 to 16 chunks, fp32 and bf16 io."""
import numpy as np
import pytest
import torch

import oracle
from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.inputs import make_inputs
from gpu_helpers import IO_NAMES, PARAM_NAMES, assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu

CASES = [  # (batch, tokens, d_inner, io, chunk_len)
    (3, 300, 200, "f32", 20),    # 15 chunks, ragged channel block, 2 spare waves per pair of blocks
    (2, 197, 192, "bf16", 50),   # 4 chunks, 3 channel blocks (odd: a spare wave pair)
    (2, 65, 32, "f32", 8),       # 9 chunks of a tiny case
    (2, 1025, 128, "bf16", 65),  # 16 chunks of a long sequence
    (1, 130, 64, "f32", 65),     # 2 chunks, one channel block
]


def _args(dev):
    return [dev[k] for k in IO_NAMES + PARAM_NAMES]


def _plan(B, L, Di, io, chunk):
    return binding.launch_info(B, L, Di, 16, 0, io, chunk_len=chunk)


@pytest.mark.parametrize("B,L,Di,io,chunk", CASES)
def test_plan_is_one_kernel(B, L, Di, io, chunk):
    p = _plan(B, L, Di, io, chunk)
    assert 2 <= p["chunks"] <= 16 and p["kernels"] == 1
    ncb = -(-Di // 64)
    carry = 2 * B * p["chunks"] * 16 * Di * 4
    dsum = 2 * B * p["chunks"] * Di * 4
    park = p["workgroups"] * (2 if ncb >= 2 else 1) * p["chunk_len"] * 64 * 4 if p["park_in_workspace"] else 0
    up = lambda v: -(-v // 256) * 256
    assert p["workspace_bytes"] == up(up(up(carry) + dsum) + park) + 2 * B * p["chunks"] * ncb * 8


@pytest.mark.parametrize("fill", ["random", "ones", "stale"])
@pytest.mark.parametrize("B,L,Di,io,chunk", CASES)
def test_workspace_contents_do_not_matter(B, L, Di, io, chunk, fill):
    inp = make_inputs(B, L, Di, 16, io, seed=B * L + Di)
    dev = to_device(inp, io)
    need = binding.workspace_bytes(B, L, Di, 16, 0, io, chunk_len=chunk)
    fresh = binding.bidir_fwd(*_args(dev), chunk_len=chunk, workspace=torch.zeros(need, dtype=torch.uint8,
                                                                                 device="cuda:0"))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    if fill == "random":
        g = torch.Generator(device="cuda:0")
        g.manual_seed(11)
        ws.copy_(torch.randint(0, 256, (need,), generator=g, device="cuda:0", dtype=torch.int32).to(torch.uint8))
    elif fill == "ones":
        ws.fill_(255)
    else:  # a previous call with other inputs leaves its aggregates and its tags
        other = to_device(make_inputs(B, L, Di, 16, io, seed=B * L + Di + 1), io)
        binding.bidir_fwd(*_args(other), chunk_len=chunk, workspace=ws)
    y = binding.bidir_fwd(*_args(dev), chunk_len=chunk, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, fresh), f"{fill} workspace changes the output"
    assert_close(to_f64(y), oracle.bidir_fwd(inp), io, f"chain B={B} L={L} Di={Di} {io} chunk={chunk} {fill}")


@pytest.mark.parametrize("B,L,Di,io,chunk", CASES[:2])
def test_a_queue_of_calls_on_one_workspace(B, L, Di, io, chunk):
    """Twelve calls, four input sets in turn, one workspace, no synchronisation in between: each
    output equals the result of its own inputs computed alone."""
    sets = [to_device(make_inputs(B, L, Di, 16, io, seed=100 + s), io) for s in range(4)]
    alone = []
    for d in sets:
        alone.append(binding.bidir_fwd(*_args(d), chunk_len=chunk).clone())
        torch.cuda.synchronize()
    ws = torch.empty(binding.workspace_bytes(B, L, Di, 16, 0, io, chunk_len=chunk), dtype=torch.uint8,
                     device="cuda:0")
    outs = [binding.bidir_fwd(*_args(sets[i % 4]), chunk_len=chunk, workspace=ws) for i in range(12)]
    torch.cuda.synchronize()
    for i, y in enumerate(outs):
        assert torch.equal(y, alone[i % 4]), f"call {i} differs from its inputs' own result"


def test_two_streams_each_with_its_workspace():
    B, L, Di, io, chunk = 2, 197, 192, "bf16", 25
    sets = [to_device(make_inputs(B, L, Di, 16, io, seed=200 + s), io) for s in range(2)]
    alone = [binding.bidir_fwd(*_args(d), chunk_len=chunk).clone() for d in sets]
    torch.cuda.synchronize()
    need = binding.workspace_bytes(B, L, Di, 16, 0, io, chunk_len=chunk)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.empty(need, dtype=torch.uint8, device="cuda:0") for _ in streams]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [[], []]
    for i in range(6):
        for j, s in enumerate(streams):
            with torch.cuda.stream(s):
                outs[j].append(binding.bidir_fwd(*_args(sets[j]), chunk_len=chunk, workspace=wss[j]))
    torch.cuda.synchronize()
    for j in range(2):
        for i, y in enumerate(outs[j]):
            assert torch.equal(y, alone[j]), f"stream {j} call {i} differs"


FWD_KEYS = {"x": "x", "dt": "dt", "z": "z", "B": "B_f", "C": "C_f", "A": "A_f", "D": "D_f", "dt_bias": "dt_bias_f"}


@pytest.mark.parametrize("fill", ["random", "stale"])
@pytest.mark.parametrize("B,L,Di,io,chunk", [(3, 300, 200, "f32", 20), (2, 197, 320, "bf16", 50), (2, 65, 32, "f32", 8)])
def test_forward_only_workspace_contents_do_not_matter(B, L, Di, io, chunk, fill):
    p = binding.launch_info(B, L, Di, 16, 0, io, chunk_len=chunk, forward_only=True)
    assert 2 <= p["chunks"] <= 16 and p["kernels"] == 1
    inp = make_inputs(B, L, Di, 16, io, seed=B * L + Di + 7)
    dev = to_device(inp, io)
    fargs = [dev[FWD_KEYS[k]] for k in FWD_KEYS]
    need = binding.workspace_bytes(B, L, Di, 16, 0, io, chunk_len=chunk, forward_only=True)
    fresh = binding.fwd(*fargs, chunk_len=chunk, workspace=torch.zeros(need, dtype=torch.uint8, device="cuda:0"))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    if fill == "random":
        g = torch.Generator(device="cuda:0")
        g.manual_seed(12)
        ws.copy_(torch.randint(0, 256, (need,), generator=g, device="cuda:0", dtype=torch.int32).to(torch.uint8))
    else:
        other = to_device(make_inputs(B, L, Di, 16, io, seed=B * L + Di + 8), io)
        binding.fwd(*[other[FWD_KEYS[k]] for k in FWD_KEYS], chunk_len=chunk, workspace=ws)
    y = binding.fwd(*fargs, chunk_len=chunk, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, fresh), f"{fill} workspace changes the forward-only output"
    ref = oracle.fwd({k: inp[v] for k, v in FWD_KEYS.items()})
    assert_close(to_f64(y), ref, io, f"fwd chain B={B} L={L} Di={Di} {io} chunk={chunk} {fill}")


def test_no_wait_gave_up():
    """Runs after the calls above in this file (and whatever ran before in the process)."""
    dev = to_device(make_inputs(3, 300, 200, 16, "f32", seed=5), "f32")
    binding.bidir_fwd(*_args(dev), chunk_len=20)
    torch.cuda.synchronize()
    assert binding.wait_timeouts() == 0
