"""The scan and NC-SSD at the largest size the C ABI accepts: batch * seqlen * d_inner just under
2^31 elements (one sequence of 2,097,151 tokens, 1024 channels, bf16), so every offset of the
kernels and the host plan runs at its widest (about ten thousand chunks and carries, a park of
several GB).
Inputs are drawn on the device; the oracle checks every token of sampled channels (channels are
independent, so the oracle runs the full definition on the sliced channels)."""
import numpy as np
import pytest
import torch

import oracle
from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.inputs import device_inputs, device_ncssd_inputs
from gpu_helpers import IO_NAMES, PARAM_NAMES, assert_close

pytestmark = pytest.mark.gpu
B, DI = 1, 1024
L = (1 << 31) // DI - 1          # B * L * DI = 2^31 - 1024
CHANNELS = [0, 63, 64, 511, 1023]  # block edges and the last channel


def _host(t):
    return t.float().cpu().numpy()


def test_scan_at_the_element_limit():
    assert B * L * DI < 2 ** 31
    dev = device_inputs(B, L, DI, 16, "bf16", seed=5)
    plan = binding.launch_info(B, L, DI, 16, 0, "bf16")
    assert plan["chunks"] >= -(-L // 256) and plan["kernels"] == 3
    y = binding.bidir_fwd(*[dev[k] for k in IO_NAMES + PARAM_NAMES])
    torch.cuda.synchronize()
    got = _host(y[:, :, CHANNELS]).astype(np.float64)
    sub = {k: _host(dev[k][:, :, CHANNELS]) for k in ("x", "dt", "z")}
    sub.update({k: _host(dev[k]) for k in ("B_f", "C_f", "B_b", "C_b")})
    sub.update({k: dev[k][CHANNELS].cpu().numpy() for k in PARAM_NAMES})
    del dev, y
    torch.cuda.empty_cache()
    ref = oracle.bidir_fwd(sub, nthreads=len(CHANNELS))
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", "scan at 2^31 - 1024 elements")


def test_ncssd_at_the_element_limit():
    dev = device_ncssd_inputs(B, L, DI, 16, "bf16", seed=6)
    y = binding.ncssd_fwd(dev["x"], dev["B"], dev["C"], dev["m"])
    torch.cuda.synchronize()
    got = _host(y[:, :, CHANNELS]).astype(np.float64)
    x = _host(dev["x"][:, :, CHANNELS])
    Bh, Ch, m = _host(dev["B"]), _host(dev["C"]), dev["m"].cpu().numpy()
    del dev, y
    torch.cuda.empty_cache()
    ref = oracle.ncssd(x, Bh, Ch, m, nthreads=len(CHANNELS))
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", "NC-SSD at 2^31 - 1024 elements")
