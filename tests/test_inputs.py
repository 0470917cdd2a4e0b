"""The seeded input generator: determinism, the stated distributions, bf16 rounding."""
import numpy as np
import pytest
import torch

from bidirectional_selective_scan_amd.configs import WORKLOADS
from bidirectional_selective_scan_amd.inputs import (bf16_bits_to_f32, f32_to_bf16_bits, make_inputs,
                                                     progression_params, round_to_io)


def test_deterministic_and_seed_dependent():
    a = make_inputs(2, 65, 32, 16, "f32", 0)
    b = make_inputs(2, 65, 32, 16, "f32", 0)
    c = make_inputs(2, 65, 32, 16, "f32", 1)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert not np.array_equal(a["x"], c["x"])


def test_distributions():
    inp = make_inputs(4, 197, 384, 16, "f32", 0)
    assert abs(inp["x"].std() - 1) < 0.01 and abs(inp["x"].mean()) < 0.01
    assert abs(inp["dt"].std() - 0.5) < 0.005
    assert abs(inp["B_b"].std() - 1) < 0.02
    dt0 = np.log1p(np.exp(inp["dt_bias_f"].astype(np.float64)))   # softplus recovers dt0
    assert dt0.min() >= 1e-3 * (1 - 1e-5) and dt0.max() <= 1e-1 * (1 + 1e-5)
    np.testing.assert_array_equal(inp["A_f"][5], -np.arange(1, 17, dtype=np.float32))
    np.testing.assert_array_equal(inp["D_b"], np.ones(384, np.float32))
    assert not np.array_equal(inp["dt_bias_f"], inp["dt_bias_b"])


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -1e-40, np.inf, -np.inf],
                                 np.float32)])
    ours = bf16_bits_to_f32(f32_to_bf16_bits(v))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)
    nan = bf16_bits_to_f32(f32_to_bf16_bits(np.array([np.nan], np.float32)))
    assert np.isnan(nan).all()


@pytest.mark.parametrize("w", WORKLOADS[:3], ids=lambda w: w.name)
def test_io_values_representable(w):
    inp = make_inputs(2, 9, w.d_inner, 16, w.io_dtype, 0)
    for k in ("x", "z", "dt", "B_f", "C_b"):
        np.testing.assert_array_equal(round_to_io(inp[k], w.io_dtype), inp[k])


def test_workload_table():
    names = [w.name for w in WORKLOADS]
    assert len(set(names)) == 5
    vim_s = WORKLOADS[2]
    assert (vim_s.batch, vim_s.seqlen, vim_s.d_inner, vim_s.io_dtype) == (128, 197, 768, "bf16")
    assert vim_s.algorithmic_bytes() == 158_265_344
    folded = WORKLOADS[4]
    assert folded.seqlen == 256 * 51 and folded.seg_len == 51


def test_progression_params_are_exact_progressions():
    p = progression_params(200, 16, 5)
    n = np.arange(16, dtype=np.float32)
    for sfx in ("f", "b"):
        A = p["A_" + sfx]
        s = (A[:, 1] - A[:, 0]).astype(np.float32)
        assert np.array_equal(A, (A[:, :1] + n[None, :] * s[:, None]).astype(np.float32))
        assert (A < 0).all()
        geometric = A[:, 1] == 2 * A[:, 0]
        assert geometric[64:128].all() and geometric[192:].all()
        assert not geometric[:64].all()


def test_ncssd_inputs_recipe():
    from bidirectional_selective_scan_amd.inputs import ncssd_inputs
    a = ncssd_inputs(3, 11, 32, 16, "bf16", 4)
    b = ncssd_inputs(3, 11, 32, 16, "bf16", 4)
    for k in ("x", "B", "C", "m"):
        assert np.array_equal(a[k], b[k]) and a[k].dtype == np.float32
    assert a["x"].shape == (3, 11, 32) and a["B"].shape == (3, 11, 16) and a["m"].shape == (3, 11)
    for k in ("x", "B", "C"):
        np.testing.assert_array_equal(round_to_io(a[k], "bf16"), a[k])
    assert (a["m"] > 1.0).all() and (a["m"] <= np.float32(np.e)).all()


def test_device_generators_follow_the_recipe():
    """device_inputs / device_ncssd_inputs (used where the host cannot draw the inputs): seeded,
    the stated distributions, the io dtype, and make_inputs' parameters."""
    from bidirectional_selective_scan_amd.inputs import device_inputs, device_ncssd_inputs
    a = device_inputs(2, 3000, 64, 16, "bf16", seed=3, device="cpu")
    b = device_inputs(2, 3000, 64, 16, "bf16", seed=3, device="cpu")
    for k in a:
        assert torch.equal(a[k], b[k])
    assert a["x"].dtype == torch.bfloat16 and a["B_f"].shape == (2, 3000, 16)
    assert abs(a["x"].float().std().item() - 1) < 0.02 and abs(a["dt"].float().std().item() - 0.5) < 0.01
    ref = make_inputs(1, 1, 64, 16, "f32", 3)
    for k in ("A_f", "A_b", "D_f", "D_b", "dt_bias_f", "dt_bias_b"):
        np.testing.assert_array_equal(a[k].numpy(), ref[k])
    n = device_ncssd_inputs(1, 5000, 32, 16, "f32", seed=4, device="cpu")
    m = n["m"].numpy()
    assert n["x"].dtype == torch.float32 and m.min() > 1.0 and m.max() <= np.e * (1 + 1e-6)
