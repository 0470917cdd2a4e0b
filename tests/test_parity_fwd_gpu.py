"""Parity of the forward-only scan (vimscan_fwd) and of the auxiliary swap (VIMSCAN_FLAG_AUX_SWAP,
both entry points) with the float64 oracle, on the GPU, through the C ABI. Same tolerances as the
bidirectional scan."""
import numpy as np
import pytest
import torch

import oracle
from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.configs import WORKLOADS
from bidirectional_selective_scan_amd.inputs import (make_inputs, make_workload_inputs, progression_params,
                                                     random_params)
from gpu_helpers import IO_NAMES, PARAM_NAMES, assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu
FWD_KEYS = {"x": "x", "dt": "dt", "z": "z", "B": "B_f", "C": "C_f", "A": "A_f", "D": "D_f", "dt_bias": "dt_bias_f"}


def _fwd_inputs(inp):
    return {k: inp[v] for k, v in FWD_KEYS.items()}


def _case(B, L, Di, io, seed, params="s4d"):
    inp = make_inputs(B, L, Di, 16, io, seed)
    if params == "random":
        inp.update(random_params(Di, 16, seed + 7))
    elif params == "progression":
        inp.update(progression_params(Di, 16, seed + 7))
    return inp


def _run_fwd(inp, io, seg_len=0, **kw):
    dev = to_device(inp, io)
    return binding.fwd(*[dev[FWD_KEYS[k]] for k in FWD_KEYS], seg_len=seg_len, **kw)


def _swap_rows(y, seg_len):
    L = y.shape[1]
    T = seg_len or L
    out = y.copy()
    first = np.arange(0, L, T)
    out[:, first], out[:, first + T - 1] = y[:, first + T - 1], y[:, first]
    return out


@pytest.mark.parametrize("swap", [False, True], ids=["plain", "swap"])
@pytest.mark.parametrize("general", [False, True], ids=["auto", "general_decay"])
@pytest.mark.parametrize("wi", [1, 2, 3, 4], ids=lambda i: WORKLOADS[i].name)
def test_fwd_workload_full_size(wi, general, swap):
    w = WORKLOADS[wi]
    inp = make_workload_inputs(w)
    y = to_f64(_run_fwd(inp, w.io_dtype, w.seg_len, general_decay=general, aux_swap=swap))
    assert np.isfinite(y).all()
    assert_close(y, oracle.fwd(_fwd_inputs(inp), seg_len=w.seg_len, swap=swap), w.io_dtype, w.name + " fwd")


FWD_SHAPES = [
    # B, L, Di, seg_len, chunk_len, swap
    (1, 1, 1, 0, 0, True),
    (2, 2, 3, 0, 0, True),
    (3, 63, 65, 0, 0, False),
    (2, 65, 130, 0, 0, True),    # three channel blocks: the last workgroup has spare waves
    (1, 200, 300, 0, 0, True),   # five channel blocks
    (2, 257, 64, 0, 0, True),    # chunked, ragged last chunk: the swap crosses chunks
    (2, 197, 64, 0, 16, False),
    (2, 197, 64, 0, 1, True),
    (1, 120, 64, 12, 0, True),   # folded: one swap per segment
    (1, 120, 64, 12, 5, True),
    (1, 60, 64, 1, 0, True),     # segments of one token: the swap is the identity
    (1, 1025, 64, 0, 0, False),
]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("params", ["s4d", "random", "progression"], ids=lambda p: p + "_A")
@pytest.mark.parametrize("shape", FWD_SHAPES, ids=lambda s: "B%d_L%d_D%d_seg%d_chunk%d_swap%d" % s)
def test_fwd_shapes(shape, params, io):
    B, L, Di, seg, chunk, swap = shape
    inp = _case(B, L, Di, io, seed=L * 13 + Di, params=params)
    y = to_f64(_run_fwd(inp, io, seg, chunk_len=chunk, aux_swap=swap))
    assert_close(y, oracle.fwd(_fwd_inputs(inp), seg_len=seg, swap=swap), io, f"{shape} params={params}")


@pytest.mark.parametrize("seg,chunk", [(0, 0), (0, 40), (51, 0)])
def test_bidir_with_swap(seg, chunk):
    inp = _case(4, 102, 192, "bf16", 77)
    dev = to_device(inp, "bf16")
    y = to_f64(binding.bidir_fwd(*[dev[k] for k in IO_NAMES + PARAM_NAMES], seg_len=seg, chunk_len=chunk,
                                 aux_swap=True))
    assert_close(y, _swap_rows(oracle.bidir_fwd(inp, seg_len=seg), seg), "bf16", f"bidir swap seg={seg}")


def test_fwd_folded_equals_unfolded_bitwise():
    k, T, Di = 24, 51, 192
    unf = _case(k, T, Di, "bf16", 23)
    y_u = _run_fwd(unf, "bf16", aux_swap=True)
    fold = dict(unf)
    for n in ("x", "dt", "z", "B_f", "C_f", "B_b", "C_b"):
        fold[n] = np.asarray(unf[n]).reshape((1, k * T) + np.asarray(unf[n]).shape[2:])
    y_f = _run_fwd(fold, "bf16", seg_len=T, aux_swap=True)
    assert torch.equal(y_f.reshape(k, T, Di).view(torch.int16), y_u.view(torch.int16))


def test_fwd_equals_bidir_with_backward_branch_off():
    """The forward-only kernels against the bidirectional ones with B_b = 0 and D_b = 0 (the
    backward branch then contributes exactly 0)."""
    inp = _case(4, 197, 256, "f32", 31, params="random")
    off = dict(inp)
    off["B_b"] = np.zeros_like(np.asarray(inp["B_b"]))
    off["D_b"] = np.zeros_like(np.asarray(inp["D_b"]))
    dev = to_device(off, "f32")
    yb = to_f64(binding.bidir_fwd(*[dev[k] for k in IO_NAMES + PARAM_NAMES]))
    yf = to_f64(_run_fwd(inp, "f32"))
    assert np.abs(yf - yb).max() <= 1e-5 * (1 + np.abs(yb).max())
