"""A seeded random sweep of every scan entry point against the float64 oracle, on the GPU.

Each case draws its shape (batch, length, d_inner with ragged channel blocks, reset period),
chunking (the library's plan or a forced chunk length), io dtype, parameter family (S4D-real,
random per-state, arithmetic progressions), transition flag and variant (plain, with the
directional convolution, forward only with or without the auxiliary swap, in a given order) from
one generator, so the sweep covers combinations the hand-written cases do not. Sizes are kept
small enough for the oracle to finish each case in well under a second."""
import numpy as np
import pytest
import torch

import oracle
from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.inputs import (conv_params, deformable_order, make_inputs, progression_params,
                                                     random_orders, random_params)
from gpu_helpers import IO_NAMES, PARAM_NAMES, assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu

VARIANTS = ("plain", "conv", "fwd", "fwd_swap", "ordered")
N_CASES = 60


def _draw(i):
    rng = np.random.Generator(np.random.PCG64(1000 + i))
    variant = VARIANTS[i % len(VARIANTS)]
    io = ("f32", "bf16")[rng.integers(2)]
    params = ("s4d", "random", "progression")[rng.integers(3)]
    B = int(rng.integers(1, 4))
    if rng.random() < 0.35:                       # folded: m segments of T tokens per row
        T = int(rng.integers(1, 80))
        L, seg = T * int(rng.integers(1, 7)), T
    else:
        L, seg = int(rng.integers(1, 600)), 0
    Di = int(rng.integers(1, 200))
    seq_len = seg or L
    chunk = int(rng.integers(1, min(seq_len, 256) + 1)) if rng.random() < 0.4 else 0
    general = bool(rng.random() < 0.3)
    taps = int(rng.integers(1, 5))
    return dict(variant=variant, io=io, params=params, B=B, L=L, seg=seg, Di=Di, chunk=chunk, general=general,
                taps=taps, seed=int(rng.integers(1 << 30)))


CASES = [_draw(i) for i in range(N_CASES)]


def _id(c):
    return "{variant}-{io}-{params}-B{B}-L{L}-seg{seg}-D{Di}-chunk{chunk}{g}".format(
        g="-general" if c["general"] else "", **c)


@pytest.mark.parametrize("c", CASES, ids=[_id(c) for c in CASES])
def test_random_case_matches_oracle(c):
    B, L, Di, io, seg, seed = c["B"], c["L"], c["Di"], c["io"], c["seg"], c["seed"]
    inp = make_inputs(B, L, Di, 16, io, seed)
    if c["params"] == "random":
        inp.update(random_params(Di, 16, seed + 7))
    elif c["params"] == "progression":
        inp.update(progression_params(Di, 16, seed + 7))
    dev = to_device(inp, io)
    kw = dict(seg_len=seg, chunk_len=c["chunk"], general_decay=c["general"])
    what = _id(c)
    if c["variant"] in ("fwd", "fwd_swap"):
        swap = c["variant"] == "fwd_swap"
        keys = ("x", "dt", "z", "B_f", "C_f", "A_f", "D_f", "dt_bias_f")
        y = binding.fwd(*[dev[k] for k in keys], aux_swap=swap, **kw)
        ref = oracle.fwd({"x": inp["x"], "dt": inp["dt"], "z": inp["z"], "B": inp["B_f"], "C": inp["C_f"],
                          "A": inp["A_f"], "D": inp["D_f"], "dt_bias": inp["dt_bias_f"]}, seg_len=seg, swap=swap)
    elif c["variant"] == "conv":
        inp.update(conv_params(Di, c["taps"], seed + 13))
        conv = tuple(torch.from_numpy(np.array(inp[k], dtype=np.float32)).to("cuda:0")
                     for k in ("conv_w_f", "conv_b_f", "conv_w_b", "conv_b_b"))
        y = binding.bidir_fwd(*[dev[k] for k in IO_NAMES + PARAM_NAMES], conv=conv, **kw)
        ref = oracle.bidir_conv_fwd(inp, seg_len=seg)
    elif c["variant"] == "ordered":
        T = seg or L
        nseq = B * L // T
        if seed % 2:
            order = random_orders(nseq, T, seed + 3)
        else:
            order = np.stack([deformable_order(T, seed + 3 + s) for s in range(nseq)]).astype(np.int32)
        o = torch.from_numpy(np.ascontiguousarray(order, dtype=np.int32)).to("cuda:0")
        y = binding.bidir_fwd(*[dev[k] for k in IO_NAMES + PARAM_NAMES], order=o, **kw)
        ref = oracle.bidir_order_fwd(inp, order, seg_len=seg)
    else:
        y = binding.bidir_fwd(*[dev[k] for k in IO_NAMES + PARAM_NAMES], **kw)
        ref = oracle.bidir_fwd(inp, seg_len=seg)
    assert_close(to_f64(y), ref, io, what)


def test_sweep_covers_every_variant_and_path():
    """The draw reaches every variant, both io types, every parameter family, folding, forced
    chunking and the general-transition flag."""
    seen = {k: {c[k] for c in CASES} for k in ("variant", "io", "params", "general")}
    assert seen["variant"] == set(VARIANTS)
    assert seen["io"] == {"f32", "bf16"} and seen["params"] == {"s4d", "random", "progression"}
    assert seen["general"] == {False, True}
    assert any(c["seg"] for c in CASES) and any(c["chunk"] for c in CASES)
    assert any(c["chunk"] == 0 and (c["seg"] or c["L"]) > 256 for c in CASES)   # the plan chunks by itself


# Plans of up to this many chunks per sequence fold the chunk aggregates in the scan workgroups.
FOLD_MAX_CHUNKS = 16


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("K", [2, 3, 4, 5, 6, 9, 13, FOLD_MAX_CHUNKS, FOLD_MAX_CHUNKS + 1, 32])
def test_chunk_counts_around_the_in_scan_fold(K, variant, io):
    """A sequence of up to FOLD_MAX_CHUNKS chunks runs without the carry-combine kernel: each scan
    workgroup folds the aggregates of the chunks before its own, four chunks per round of loads (one
    round up to 5 chunks, several from 6), the aggregates computed and handed over inside the same
    kernel (one kernel per call); past that the aggregate pass and the combine supply the entering
    states.
    Every variant against the oracle at each count, with a ragged last chunk and a ragged channel
    block, general transitions with fp32 io and geometric ones with bf16."""
    T, Di = 7, 96
    c = dict(variant=variant, io=io, params="random" if io == "f32" else "s4d", B=2, L=T * (K - 1) + 4, seg=0,
             Di=Di, chunk=T, general=False, taps=3, seed=7000 + 10 * K + VARIANTS.index(variant))
    info = binding.launch_info(c["B"], c["L"], Di, 16, 0, io, chunk_len=T,
                               forward_only=variant in ("fwd", "fwd_swap"), aux_swap=variant == "fwd_swap")
    assert info["chunks"] == K
    assert info["kernels"] == (1 if K <= FOLD_MAX_CHUNKS else 3) + (1 if variant == "fwd_swap" else 0)
    test_random_case_matches_oracle(c)
