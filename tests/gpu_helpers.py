"""Helpers shared by the GPU tests: move seeded numpy inputs to the device, run the HIP path
through the C ABI binding, compare with the float64 oracle at the stated tolerances."""
import numpy as np
import torch

from bidirectional_selective_scan_amd import binding

IO_NAMES = ("x", "dt", "z", "B_f", "C_f", "B_b", "C_b")
PARAM_NAMES = ("A_f", "A_b", "D_f", "D_b", "dt_bias_f", "dt_bias_b")

# Tolerances (elementwise):
#   fp32 io:  |y - y_ref| <= 1e-4 * (1 + |y_ref|)
#   bf16 io:  |y - y_ref| <= 2e-2 * max(|y_ref|, 0.1 * rms(y_ref))   (2e-2 relative; below a tenth of
#             the output's rms the bound stays at 2e-3 rms, so zero crossings of the SiLU gate are
#             not judged by pure relative error)
F32_TOL = 1e-4
BF16_TOL = 2e-2
BF16_FLOOR = 0.1


def bf16_bound(ref: np.ndarray) -> np.ndarray:
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    return BF16_TOL * np.maximum(np.abs(ref), BF16_FLOOR * rms)


def to_device(inp: dict, io_dtype: str, device="cuda:0") -> dict:
    tdt = torch.float32 if io_dtype == "f32" else torch.bfloat16
    out = {}
    for k in IO_NAMES:
        out[k] = torch.from_numpy(np.array(inp[k], dtype=np.float32)).to(device).to(tdt)
    for k in PARAM_NAMES:
        out[k] = torch.from_numpy(np.array(inp[k], dtype=np.float32)).to(device)
    return out


def run_gpu(dev_inp: dict, seg_len=0, **kw):
    return binding.bidir_fwd(*[dev_inp[k] for k in IO_NAMES + PARAM_NAMES], seg_len=seg_len, **kw)


def to_f64(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def violations(got: np.ndarray, ref: np.ndarray, io_dtype: str) -> np.ndarray:
    err = np.abs(got - ref)
    if io_dtype == "f32":
        bound = F32_TOL * (1.0 + np.abs(ref))
    else:
        bound = bf16_bound(ref)
    bad = ~(err <= bound)   # NaN counts as a violation
    return bad


def assert_close(got: np.ndarray, ref: np.ndarray, io_dtype: str, what: str = ""):
    assert got.shape == ref.shape
    bad = violations(got, ref, io_dtype)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        err = np.abs(got - ref)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; max abs err "
                             f"{np.nanmax(err):.3e}; first at {idx.tolist()}: got {got[tuple(idx[0])]!r} "
                             f"ref {ref[tuple(idx[0])]!r}")
