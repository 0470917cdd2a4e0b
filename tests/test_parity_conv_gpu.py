"""Parity of the scan with the directional convolution in front (vimscan_bidir_conv_fwd, through
the C ABI) with the float64 oracle, on the GPU. Same tolerances as the plain scan."""
import numpy as np
import pytest
import torch

import oracle
from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.configs import WORKLOADS
from bidirectional_selective_scan_amd.inputs import (conv_params, make_inputs, make_workload_inputs,
                                                     progression_params, random_params)
from gpu_helpers import IO_NAMES, PARAM_NAMES, assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu
CONV_NAMES = ("conv_w_f", "conv_b_f", "conv_w_b", "conv_b_b")


def _case(B, L, Di, io, seed, K=4, params="s4d"):
    inp = make_inputs(B, L, Di, 16, io, seed)
    if params == "random":
        inp.update(random_params(Di, 16, seed + 7))
    elif params == "progression":
        inp.update(progression_params(Di, 16, seed + 7))
    inp.update(conv_params(Di, K, seed + 13))
    return inp


def _run(inp, io, seg_len=0, **kw):
    dev = to_device(inp, io)
    conv = tuple(torch.from_numpy(np.array(inp[k], dtype=np.float32)).to("cuda:0") for k in CONV_NAMES)
    return binding.bidir_fwd(*[dev[k] for k in IO_NAMES + PARAM_NAMES], seg_len=seg_len, conv=conv, **kw)


@pytest.mark.parametrize("general", [False, True], ids=["auto", "general_decay"])
@pytest.mark.parametrize("wi", [1, 2, 3, 4], ids=lambda i: WORKLOADS[i].name)
def test_conv_workload_full_size(wi, general):
    w = WORKLOADS[wi]
    inp = make_workload_inputs(w)
    inp.update(conv_params(w.d_inner, 4, w.seed + 101))
    y = to_f64(_run(inp, w.io_dtype, w.seg_len, general_decay=general))
    assert np.isfinite(y).all()
    assert_close(y, oracle.bidir_conv_fwd(inp, seg_len=w.seg_len), w.io_dtype, w.name + " conv")


CONV_SHAPES = [
    # B, L, Di, seg_len, chunk_len, K
    (1, 1, 1, 0, 0, 4),
    (2, 3, 65, 0, 0, 4),       # shorter than the taps
    (2, 65, 130, 0, 0, 3),     # odd number of 64-channel blocks
    (1, 200, 70, 0, 0, 2),
    (2, 257, 64, 0, 0, 4),     # chunked: the window crosses chunk boundaries
    (2, 197, 64, 0, 16, 4),    # forced chunks, ragged tail
    (2, 197, 64, 0, 1, 4),     # one token per chunk: the whole window comes from neighbours
    (2, 197, 100, 0, 2, 3),
    (1, 120, 64, 12, 0, 4),    # folded: zero padding at every segment boundary
    (1, 120, 64, 12, 5, 4),    # folded, chunks that do not divide the segment
    (2, 102, 33, 51, 0, 1),
    (1, 60, 64, 2, 0, 4),      # segments shorter than the taps
    (1, 1025, 64, 0, 0, 4),
]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("params", ["s4d", "random", "progression"], ids=lambda p: p + "_A")
@pytest.mark.parametrize("shape", CONV_SHAPES, ids=lambda s: "B%d_L%d_D%d_seg%d_chunk%d_K%d" % s)
def test_conv_shapes(shape, params, io):
    B, L, Di, seg, chunk, K = shape
    inp = _case(B, L, Di, io, seed=L * 17 + Di + K, K=K, params=params)
    y = to_f64(_run(inp, io, seg, chunk_len=chunk))
    assert_close(y, oracle.bidir_conv_fwd(inp, seg_len=seg), io, f"{shape} params={params}")


def test_conv_folded_equals_unfolded_bitwise():
    k, T, Di = 24, 51, 192
    unf = _case(k, T, Di, "bf16", 21)
    y_u = _run(unf, "bf16")
    fold = dict(unf)
    for n in ("x", "dt", "z", "B_f", "C_f", "B_b", "C_b"):
        fold[n] = np.asarray(unf[n]).reshape((1, k * T) + np.asarray(unf[n]).shape[2:])
    y_f = _run(fold, "bf16", seg_len=T)
    assert torch.equal(y_f.reshape(k, T, Di).view(torch.int16), y_u.view(torch.int16))


def test_conv_deterministic_and_differs_from_plain():
    inp = _case(8, 197, 256, "bf16", 5)
    a = _run(inp, "bf16").clone()
    b = _run(inp, "bf16").clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    dev = to_device(inp, "bf16")
    plain = binding.bidir_fwd(*[dev[k] for k in IO_NAMES + PARAM_NAMES])
    assert (plain.float() - a.float()).abs().max().item() > 1e-2


def test_conv_errors_are_reported():
    inp = _case(1, 12, 64, "f32", 1, K=4)
    dev = to_device(inp, "f32")
    conv = [torch.from_numpy(np.array(inp[k], dtype=np.float32)).to("cuda:0") for k in CONV_NAMES]
    wide = [torch.zeros(64, 5, device="cuda:0"), conv[1], torch.zeros(64, 5, device="cuda:0"), conv[3]]
    with pytest.raises(binding.VimscanError):
        binding.bidir_fwd(*[dev[k] for k in IO_NAMES + PARAM_NAMES], conv=tuple(wide))   # 5 taps
    with pytest.raises(ValueError):
        binding.bidir_fwd(*[dev[k] for k in IO_NAMES + PARAM_NAMES], conv=(conv[0], conv[1], conv[2][:, :3].contiguous(),
                                                                             conv[3]))
