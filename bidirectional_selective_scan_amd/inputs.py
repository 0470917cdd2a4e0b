"""Seeded synthetic inputs for the bidirectional selective scan.

This module draws random numbers and rounds them to the I/O dtype; it performs none of the
scan's own arithmetic. Both the HIP path's tests/bench and the float64 oracle take their inputs
from here, so it imports nothing else from this package or from the oracle.

Recipe (one numpy ``Generator(PCG64(seed))``, draws in this fixed order, all float32):

1. x ~ N(0, 1), shape (B, L, Di)
2. z ~ N(0, 1), shape (B, L, Di)
3. dt ~ N(0, 0.5^2), shape (B, L, Di)   (the pre-bias step; the scan adds dt_bias)
4. B_f, 5. C_f, 6. B_b, 7. C_b ~ N(0, 1), each shape (B, L, N)
8. u_f, 9. u_b ~ U(ln 1e-3, ln 1e-1), each shape (Di,): dt0 = exp(u) is log-uniform in
   [1e-3, 1e-1] and dt_bias = dt0 + log(-expm1(-dt0)), the value whose softplus is dt0.

A_f = A_b = -(n+1) for n = 0..N-1, the same for every channel; D_f = D_b = 1.
For bf16 workloads, x, z, dt, B_*, C_* are rounded float32 -> bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the uint16 bits.
    NaN stays NaN (quiet)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)
    nan = np.isnan(a)
    if nan.any():
        rounded = np.where(nan, ((u >> 16) | 0x40).astype(np.uint32), rounded)
    return (rounded & 0xFFFF).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_io(a: np.ndarray, io_dtype: str) -> np.ndarray:
    """float32 values exactly representable in io_dtype (bf16 rounding is RNE)."""
    if io_dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if io_dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a))
    raise ValueError(f"unsupported io dtype {io_dtype!r}")


TENSOR_NAMES = ("x", "z", "dt", "B_f", "C_f", "B_b", "C_b")
PARAM_NAMES = ("A_f", "A_b", "D_f", "D_b", "dt_bias_f", "dt_bias_b")


def make_inputs(batch: int, seqlen: int, d_inner: int, d_state: int = 16, io_dtype: str = "f32",
                seed: int = 0) -> dict:
    """Draw one seeded input set. Returns float32 numpy arrays; the I/O tensors already hold
    values exactly representable in ``io_dtype``. Keys: TENSOR_NAMES + PARAM_NAMES."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, L, Di, N = batch, seqlen, d_inner, d_state
    out = {}
    out["x"] = rng.standard_normal((B, L, Di), dtype=np.float32)
    out["z"] = rng.standard_normal((B, L, Di), dtype=np.float32)
    out["dt"] = (np.float32(0.5) * rng.standard_normal((B, L, Di), dtype=np.float32)).astype(np.float32)
    for name in ("B_f", "C_f", "B_b", "C_b"):
        out[name] = rng.standard_normal((B, L, N), dtype=np.float32)
    for name in ("dt_bias_f", "dt_bias_b"):
        u = rng.uniform(np.log(1e-3), np.log(1e-1), size=Di)
        dt0 = np.exp(u)
        out[name] = (dt0 + np.log(-np.expm1(-dt0))).astype(np.float32)
    a_row = -np.arange(1, N + 1, dtype=np.float32)
    out["A_f"] = np.ascontiguousarray(np.broadcast_to(a_row, (Di, N)))
    out["A_b"] = out["A_f"].copy()
    out["D_f"] = np.ones(Di, dtype=np.float32)
    out["D_b"] = np.ones(Di, dtype=np.float32)
    for name in TENSOR_NAMES:
        out[name] = round_to_io(out[name], io_dtype)
    return out


def _device_normal(shape, std, dtype, g, device, slab=1 << 26):
    """A tensor of N(0, std^2) draws made on the device in slabs along dim 1 (bounded temporaries),
    rounded to ``dtype``."""
    import torch
    out = torch.empty(shape, dtype=dtype, device=device)
    per = max(1, slab // max(1, shape[0] * int(np.prod(shape[2:]))))
    for t0 in range(0, shape[1], per):
        t1 = min(shape[1], t0 + per)
        part = torch.randn((shape[0], t1 - t0) + tuple(shape[2:]), generator=g, device=device)
        out[:, t0:t1] = (part * std).to(dtype)
    return out


def device_inputs(batch: int, seqlen: int, d_inner: int, d_state: int = 16, io_dtype: str = "bf16",
                  seed: int = 0, device: str = "cuda:0") -> dict:
    """The scan's input recipe drawn on a device, for sizes too large to draw on the host: x, z ~
    N(0, 1), dt ~ N(0, 0.5^2) (batch, seqlen, d_inner) and B_f, C_f, B_b, C_b ~ N(0, 1) (batch,
    seqlen, d_state) from one seeded torch generator on the device (a different stream of numbers
    than make_inputs at the same seed), rounded to the io dtype; the parameters are make_inputs'
    (they do not depend on the length). Returns torch tensors on the device."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tdt = torch.bfloat16 if io_dtype == "bf16" else torch.float32
    out = {}
    for name, std in (("x", 1.0), ("z", 1.0), ("dt", 0.5)):
        out[name] = _device_normal((batch, seqlen, d_inner), std, tdt, g, device)
    for name in ("B_f", "C_f", "B_b", "C_b"):
        out[name] = _device_normal((batch, seqlen, d_state), 1.0, tdt, g, device)
    params = make_inputs(1, 1, d_inner, d_state, "f32", seed)
    for name in PARAM_NAMES:
        out[name] = torch.from_numpy(params[name]).to(device)
    return out


def device_ncssd_inputs(batch: int, seqlen: int, d_inner: int, d_state: int = 16, io_dtype: str = "bf16",
                        seed: int = 0, device: str = "cuda:0") -> dict:
    """ncssd_inputs' recipe drawn on a device (x, B, C ~ N(0, 1) rounded to the io dtype;
    m = exp(exp(u)), u ~ U(ln 1e-3, 0), float32), for sizes too large to draw on the host."""
    import math
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tdt = torch.bfloat16 if io_dtype == "bf16" else torch.float32
    out = {"x": _device_normal((batch, seqlen, d_inner), 1.0, tdt, g, device)}
    for name in ("B", "C"):
        out[name] = _device_normal((batch, seqlen, d_state), 1.0, tdt, g, device)
    u = torch.rand((batch, seqlen), generator=g, device=device) * (-math.log(1e-3)) + math.log(1e-3)
    out["m"] = torch.exp(torch.exp(u)).to(torch.float32)
    return out


def make_workload_inputs(w: Workload) -> dict:
    return make_inputs(w.batch, w.seqlen, w.d_inner, w.d_state, w.io_dtype, w.seed)


def random_params(d_inner: int, d_state: int, seed: int) -> dict:
    """Per-direction parameters that differ between directions and across channels and states
    (A in [-4, -0.05), D in [0.5, 1.5), dt_bias in [-5, 0.5)). Used by tests that must tell the
    forward parameters from the backward ones, which the default recipe (A_f = A_b, D_f = D_b)
    cannot."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for sfx in ("f", "b"):
        out["A_" + sfx] = (-rng.uniform(0.05, 4.0, size=(d_inner, d_state))).astype(np.float32)
        out["D_" + sfx] = rng.uniform(0.5, 1.5, size=d_inner).astype(np.float32)
        out["dt_bias_" + sfx] = rng.uniform(-5.0, 0.5, size=d_inner).astype(np.float32)
    return out


def progression_params(d_inner: int, d_state: int, seed: int) -> dict:
    """Per-direction parameters whose A rows are exact arithmetic progressions in n,
    A[d, n] = a0[d] + n * s[d], with a0 and s multiples of 1/16 in [-2, -1/16] so that every
    sum is exact in float32 (a row spans [-32, -1/16]). Channels in odd blocks of 64 have
    a0 == s (the rows are then (n + 1) * a0, like the S4D-real initialisation); in the others
    a0 and s are drawn independently. D and dt_bias as in random_params."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    n = np.arange(d_state, dtype=np.float32)
    for sfx in ("f", "b"):
        a0 = -rng.integers(1, 33, size=d_inner).astype(np.float32) / np.float32(16)
        s = -rng.integers(1, 33, size=d_inner).astype(np.float32) / np.float32(16)
        same = (np.arange(d_inner) // 64) % 2 == 1
        s = np.where(same, a0, s).astype(np.float32)
        out["A_" + sfx] = (a0[:, None] + n[None, :] * s[:, None]).astype(np.float32)
        out["D_" + sfx] = rng.uniform(0.5, 1.5, size=d_inner).astype(np.float32)
        out["dt_bias_" + sfx] = rng.uniform(-5.0, 0.5, size=d_inner).astype(np.float32)
    return out


def conv_params(d_inner: int, k: int, seed: int) -> dict:
    """Depthwise convolution weights and biases for both directions, drawn like PyTorch's
    default conv1d initialisation for a depthwise layer (fan-in k): U(-1/sqrt(k), 1/sqrt(k)).
    Keys conv_w_f, conv_w_b (d_inner, k) and conv_b_f, conv_b_b (d_inner,), float32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bound = 1.0 / np.sqrt(k)
    out = {}
    for sfx in ("f", "b"):
        out["conv_w_" + sfx] = rng.uniform(-bound, bound, size=(d_inner, k)).astype(np.float32)
        out["conv_b_" + sfx] = rng.uniform(-bound, bound, size=d_inner).astype(np.float32)
    return out


NCSSD_NAMES = ("x", "B", "C", "m")


def ncssd_inputs(batch: int, seqlen: int, d_inner: int, d_state: int = 16, io_dtype: str = "f32",
                 seed: int = 0) -> dict:
    """Inputs of the NC-SSD global-state form. One ``Generator(PCG64(seed))``, draws in this
    order, all float32: x ~ N(0, 1) (B, L, Di); B, C ~ N(0, 1) (B, L, N) each; u ~ U(ln 1e-3, 0)
    (B, L) and m = exp(exp(u)), the token weights: m is the reciprocal of a per-token decay
    exp(-v) with v log-uniform in [1e-3, 1], so m lies in (1, e]. x, B and C are rounded to
    ``io_dtype``; m stays float32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {"x": rng.standard_normal((batch, seqlen, d_inner), dtype=np.float32)}
    for name in ("B", "C"):
        out[name] = rng.standard_normal((batch, seqlen, d_state), dtype=np.float32)
    u = rng.uniform(np.log(1e-3), 0.0, size=(batch, seqlen))
    out["m"] = np.exp(np.exp(u)).astype(np.float32)
    for name in ("x", "B", "C"):
        out[name] = round_to_io(out[name], io_dtype)
    return out


# ---------------------------------------------------------------------------------------------
# Token orders for the scan in a given order (DefMamba page, section 1: raster, Hilbert curve and
# local-window scans; section 2.1: deformable re-ranking by per-token index offsets). An order is
# data: row s lists the token positions 0..T-1 of sequence s in the order the forward scan visits
# them. Tokens that are not patches of the grid (a class token, auxiliary tokens) keep their
# place in the order.


def _hilbert_xy(n: int, d: int):
    """Cell (x, y) of step d on the Hilbert curve through an n x n grid, n a power of two: the
    curve is built quadrant by quadrant, each sub-curve rotated or reflected so its ends meet."""
    x = y = 0
    s = 1
    t = d
    while s < n:
        rx = 1 & (t // 2)
        ry = 1 & (t ^ rx)
        if ry == 0:
            if rx == 1:
                x, y = s - 1 - x, s - 1 - y
            x, y = y, x
        x += s * rx
        y += s * ry
        t //= 4
        s *= 2
    return x, y


def grid_order(kind: str, side: int, T: int, window: int = 7) -> np.ndarray:
    """One sequence's order for a side x side patch grid plus T - side^2 other tokens placed in
    the middle of the sequence (as Vision Mamba places its class token): 'raster', 'hilbert'
    (side a power of two), 'local' (window x window blocks in raster order, raster inside each
    block). Returns int32 (T,)."""
    P = side * side
    extra = T - P
    if extra < 0:
        raise ValueError("T must hold the grid")
    mid = P // 2                       # patches before the extra tokens
    def token_of_patch(p):             # token position of raster patch p
        return p if p < mid else p + extra
    if kind == "raster":
        cells = [(r, c) for r in range(side) for c in range(side)]
    elif kind == "hilbert":
        if side & (side - 1):
            raise ValueError("the Hilbert order needs a power-of-two side")
        cells = [_hilbert_xy(side, d)[::-1] for d in range(P)]
    elif kind == "local":
        cells = [(br + r, bc + c) for br in range(0, side, window) for bc in range(0, side, window)
                 for r in range(min(window, side - br)) for c in range(min(window, side - bc))]
    else:
        raise ValueError(f"unknown order {kind!r}")
    patches = [token_of_patch(r * side + c) for r, c in cells]
    order = patches[:mid] + list(range(mid, mid + extra)) + patches[mid:]
    return np.asarray(order, dtype=np.int32)


def deformable_order(T: int, seed: int, scale: float = 8.0) -> np.ndarray:
    """A re-ranked order: position k gets the key k + scale * tanh(g_k), g_k ~ N(0, 1), and the
    tokens are visited by increasing key (ties by position) -- the shape of DefMamba's
    scan-order offsets, drawn at random instead of predicted by a network."""
    rng = np.random.Generator(np.random.PCG64(seed))
    key = np.arange(T) + scale * np.tanh(rng.standard_normal(T))
    return np.argsort(key, kind="stable").astype(np.int32)


def random_orders(nseq: int, T: int, seed: int) -> np.ndarray:
    """nseq independent uniformly random permutations of 0..T-1, int32 (nseq, T)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.stack([rng.permutation(T) for _ in range(nseq)]).astype(np.int32).reshape(nseq, T)
