"""Exact zeros of x at single tokens, on the GPU, through the C ABI.

A zero x makes the token's input delta * x * B vanish: the state only decays there. These tests
put such zeros at positions spread over the steps of a walk's unrolled loop, its tail and its first
step, in some 64-channel blocks only (others keep none), in the bidirectional scan (one pass,
chunked, chunks parked in the workspace, the long sequence) and the forward-only scan, and compare
every output with the float64 oracle; with x = 0 everywhere every output is exactly 0. Same
tolerances as the other parity tests."""
import numpy as np
import pytest

import oracle
from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.inputs import make_inputs, progression_params
from gpu_helpers import assert_close, run_gpu, to_device, to_f64

pytestmark = pytest.mark.gpu

FWD_KEYS = {"x": "x", "dt": "dt", "z": "z", "B": "B_f", "C": "C_f", "A": "A_f", "D": "D_f", "dt_bias": "dt_bias_f"}


def _zeros(inp, seed, every=0):
    """Per (sequence, 64-channel block): the first zero of x at its own position (0 .. L-1 spread
    by a stride of 7), a second one 9 tokens later; every third block has none. every > 0 also
    zeroes x at every `every`-th token of the first block of each sequence."""
    x = inp["x"]
    B, L, Di = x.shape
    rng = np.random.Generator(np.random.PCG64(seed))
    i = 0
    for b in range(B):
        for cb in range(0, Di, 64):
            if (cb // 64) % 3 == 2:
                continue
            p = (7 * i + int(rng.integers(0, 3))) % L
            x[b, p, cb:cb + 64] = 0.0
            if p + 9 < L:
                x[b, p + 9, cb:cb + 32] = 0.0
            i += 1
        if every:
            x[b, ::every, 0:64] = 0.0
    return inp


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("params", ["s4d", "progression"])
@pytest.mark.parametrize("B,L,Di,chunk", [(3, 197, 512, 0), (2, 197, 256, 13), (2, 400, 256, 150), (4, 65, 256, 0),
                                          (2, 1025, 128, 0)])
def test_bidir_zero_x_tokens(B, L, Di, chunk, params, io):
    inp = make_inputs(B, L, Di, 16, io, seed=L + chunk)
    if params == "progression":
        inp.update(progression_params(Di, 16, seed=5))
    _zeros(inp, seed=L, every=23)
    y = to_f64(run_gpu(to_device(inp, io), chunk_len=chunk))
    assert np.isfinite(y).all()
    assert_close(y, oracle.bidir_fwd(inp), io, f"zero x B={B} L={L} Di={Di} chunk={chunk} {params}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("B,L,Di,chunk", [(3, 197, 512, 0), (2, 197, 256, 13), (2, 300, 128, 64)])
def test_fwd_zero_x_tokens(B, L, Di, chunk, io):
    inp = make_inputs(B, L, Di, 16, io, seed=L + chunk + 1)
    _zeros(inp, seed=L + 1, every=17)
    dev = to_device(inp, io)
    y = to_f64(binding.fwd(*[dev[FWD_KEYS[k]] for k in FWD_KEYS], chunk_len=chunk))
    assert np.isfinite(y).all()
    ref = oracle.fwd({k: inp[v] for k, v in FWD_KEYS.items()})
    assert_close(y, ref, io, f"fwd zero x B={B} L={L} Di={Di} chunk={chunk}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_all_zero_x(io):
    """x = 0 everywhere: the state stays 0 and y = silu(z) * 0 = 0 exactly."""
    inp = make_inputs(2, 197, 128, 16, io, seed=3)
    inp["x"][:] = 0.0
    y = to_f64(run_gpu(to_device(inp, io)))
    assert np.array_equal(y, np.zeros_like(y))
