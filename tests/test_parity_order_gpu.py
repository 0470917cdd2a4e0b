"""Parity of the scan in a given token order (vimscan_bidir_order_fwd) with the float64 oracle, on
the GPU, through the C ABI. Tolerances as for the raster scan. Orders: raster, Hilbert curve,
local windows and re-ranked (DefMamba page, sections 1 and 2.1), and random permutations."""
import numpy as np
import pytest
import torch

import oracle
from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.inputs import (deformable_order, grid_order, make_inputs, random_orders,
                                                     random_params)
from gpu_helpers import IO_NAMES, PARAM_NAMES, assert_close, run_gpu, to_device, to_f64

pytestmark = pytest.mark.gpu


def _case(B, L, Di, io, seed, params=True):
    inp = make_inputs(B, L, Di, 16, io, seed)
    if params:
        inp.update(random_params(Di, 16, seed + 5))
    return inp


def _run(inp, io, order, seg_len=0, **kw):
    dev = to_device(inp, io)
    o = torch.from_numpy(np.ascontiguousarray(order, dtype=np.int32)).to("cuda:0")
    y = run_gpu(dev, seg_len, order=o, **kw)
    torch.cuda.synchronize()
    return y


def _orders(kind, nseq, T, seed):
    if kind == "random":
        return random_orders(nseq, T, seed)
    if kind == "deformable":
        return np.stack([deformable_order(T, seed + i) for i in range(nseq)])
    side = int(np.sqrt(T))
    if kind == "hilbert":
        side = 1 << (side.bit_length() - 1)
    return np.tile(grid_order(kind, side, T, window=max(2, side // 2)), (nseq, 1))


CASES = [
    # (batch, L, Di, io, seg_len, chunk_len, order)
    (2, 65, 32, "f32", 0, 0, "random"),         # the tiny configuration's shape
    (2, 65, 32, "f32", 0, 0, "local"),
    (2, 65, 96, "bf16", 0, 0, "hilbert"),        # 8 x 8 grid + 1 token
    (1, 197, 128, "bf16", 0, 0, "local"),        # long chunk: the park in the workspace
    (1, 197, 64, "f32", 0, 0, "deformable"),
    (1, 257, 64, "bf16", 0, 64, "hilbert"),      # chunked: aggregates + carries in the order
    (2, 300, 40 * 2, "f32", 0, 48, "random"),    # ragged channel block, chunked
    (1, 6 * 51, 96, "bf16", 51, 0, "random"),    # folded: an order per segment
    (3, 4 * 20, 64, "f32", 20, 16, "deformable"),
    (1, 1, 64, "f32", 0, 0, "random"),
    (1, 256, 64, "bf16", 0, 256, "random"),     # one 256-token chunk: rows and order in LDS (66.5 KB)
    (1, 512, 64, "f32", 0, 256, "hilbert"),     # two of them, with a carry
]


@pytest.mark.parametrize("B,L,Di,io,seg,chunk,kind", CASES)
def test_matches_oracle(B, L, Di, io, seg, chunk, kind):
    inp = _case(B, L, Di, io, seed=L + Di)
    T = seg or L
    order = _orders(kind, B * L // T, T, seed=T)
    y = _run(inp, io, order, seg, chunk_len=chunk)
    ref = oracle.bidir_order_fwd(inp, order, seg)
    assert_close(to_f64(y), ref, io, f"order {kind} B={B} L={L} Di={Di} {io} seg={seg} chunk={chunk}")


@pytest.mark.parametrize("kind,B,L,Di,io,seg,side", [
    ("local", 128, 197, 768, "bf16", 0, 14),      # Vim-S, 7 x 7 windows
    ("deformable", 128, 197, 768, "bf16", 0, 14),
    ("hilbert", 8, 1025, 768, "bf16", 0, 32),     # high resolution, 32 x 32 Hilbert curve
    ("random", 1, 256 * 51, 1536, "bf16", 51, 7),  # folded, an order per segment
])
def test_full_size_matches_oracle(kind, B, L, Di, io, seg, side):
    """Full workload shapes in the launch configuration the benchmark would use; every output
    against the oracle."""
    inp = make_inputs(B, L, Di, 16, io, seed=0)
    T = seg or L
    nseq = B * L // T
    if kind in ("local", "hilbert"):
        order = np.tile(grid_order(kind, side, T), (nseq, 1))
    else:
        order = _orders(kind, nseq, T, seed=11)
    y = _run(inp, io, order, seg)
    assert_close(to_f64(y), oracle.bidir_order_fwd(inp, order, seg, nthreads=16), io, f"{kind} full")


@pytest.mark.parametrize("io,chunk", [("f32", 0), ("bf16", 0), ("f32", 32)])
def test_raster_order_equals_plain_scan_bit_for_bit(io, chunk):
    inp = _case(2, 120, 128, io, seed=3)
    dev = to_device(inp, io)
    plain = run_gpu(dev, 0, chunk_len=chunk)
    o = torch.arange(120, dtype=torch.int32, device="cuda:0").repeat(2, 1).contiguous()
    ordered = run_gpu(dev, 0, chunk_len=chunk, order=o)
    torch.cuda.synchronize()
    assert torch.equal(plain, ordered)


def test_reverse_order_exchanges_the_branches():
    inp = _case(2, 97, 64, "f32", seed=4)
    sw = dict(inp)
    for a, b in (("B_f", "B_b"), ("C_f", "C_b"), ("A_f", "A_b"), ("D_f", "D_b"), ("dt_bias_f", "dt_bias_b")):
        sw[a], sw[b] = inp[b], inp[a]
    rev = np.tile(np.arange(96, -1, -1, dtype=np.int32), (2, 1))
    y_rev = to_f64(_run(inp, "f32", rev))
    y_sw = to_f64(run_gpu(to_device(sw, "f32"), 0))
    np.testing.assert_allclose(y_rev, y_sw, rtol=1e-5, atol=1e-5)


def test_segments_use_their_own_orders_and_do_not_leak():
    k, T = 4, 30
    inp = _case(1, k * T, 64, "f32", seed=5)
    order = random_orders(k, T, seed=6)
    base = _run(inp, "f32", order, T)
    bad = {n: a.copy() for n, a in inp.items()}
    bad["x"][0, 2 * T + 7, 3] = np.nan
    y = _run(bad, "f32", order, T)
    for s in range(k):
        seg = slice(s * T, (s + 1) * T)
        if s == 2:
            assert torch.isnan(y[0, seg]).any()
        else:
            assert torch.equal(y[0, seg], base[0, seg])
