"""The allocation-free entry point (vimscan_bidir_fwd_noalloc, for callers that cannot allocate)
against vimscan_bidir_fwd, on the GPU through the C ABI: the same kernels with the scratch taken
from the library's static per-GPU array instead of a caller's workspace give the same bits. Two
calls in a row, the second with a smaller input (the array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import oracle
from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.inputs import device_inputs, make_inputs
from gpu_helpers import IO_NAMES, PARAM_NAMES, assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu


def _args(dev):
    return [dev[k] for k in IO_NAMES + PARAM_NAMES]


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_equals_bidir_fwd_two_calls(io):
    # 1: Vim-S (its 77.5 MB park in the scratch, bf16) or Vim-Ti (4 chunks: carries, fp32);
    # 2: a smaller, chunked call (carries and delta sums, then no park) on the same array
    first = (128, 197, 768) if io == "bf16" else (64, 197, 384)
    for B, L, Di in (first, (2, 300, 96)):
        info = binding.launch_info(B, L, Di, 16, 0, io)
        assert 0 < info["workspace_bytes"] <= binding.NOALLOC_SCRATCH_BYTES
        dev = device_inputs(B, L, Di, 16, io, seed=B + L)
        ref = binding.bidir_fwd(*_args(dev))
        out = torch.empty_like(dev["x"])
        y = binding.bidir_fwd_noalloc(*_args(dev), out=out)
        torch.cuda.synchronize()
        assert y.data_ptr() == out.data_ptr()
        assert torch.equal(y.view(torch.int16 if io == "bf16" else torch.int32),
                           ref.view(torch.int16 if io == "bf16" else torch.int32)), (B, L, Di, info)


def test_noalloc_against_the_oracle_and_folded():
    """Folded (reset every 51 tokens) and forced into chunks, after a larger call: every output
    against the float64 oracle."""
    inp = make_inputs(1, 51 * 12, 130, 16, "bf16", seed=21)
    dev = to_device(inp, "bf16")
    big = device_inputs(8, 1025, 768, 16, "bf16", seed=3)   # high-res: 16 chunks of carries first
    binding.bidir_fwd_noalloc(*_args(big))
    y = to_f64(binding.bidir_fwd_noalloc(*_args(dev), seg_len=51, chunk_len=17))
    assert_close(y, oracle.bidir_fwd(inp, seg_len=51), "bf16", "noalloc folded chunked")


def test_noalloc_rejects_a_call_larger_than_its_array():
    dev = device_inputs(256, 197, 768, 16, "bf16", seed=5)   # a 155 MB park
    with pytest.raises(binding.VimscanError) as e:
        binding.bidir_fwd_noalloc(*_args(dev))
    assert e.value.status == -12
