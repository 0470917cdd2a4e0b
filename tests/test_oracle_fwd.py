"""Pins of the oracle's unidirectional scan with the auxiliary-token swap (SF-Mamba page,
"auxiliary patch swapping"), and a check that they catch plausible mistakes in it.

Expectations: the forward SSD matrix form of the pins module (brute force), the rows of that
result exchanged by numpy indexing for the swap, and the bidirectional oracle with its backward
branch switched off (B_b = 0, D_b = 0). CPU only."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from test_oracle_pins import random_case, silu_lib, softplus_lib, ssd_matrix_direction

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "vimscan_oracle.c")).read()


def fwd_inputs(inp):
    return {"x": inp["x"], "dt": inp["dt"], "z": inp["z"], "B": inp["B_f"], "C": inp["C_f"], "A": inp["A_f"],
            "D": inp["D_f"], "dt_bias": inp["dt_bias_f"]}


def brute_fwd(f, seg_len=0, swap=False):
    x, dt, z = f["x"], f["dt"], f["z"]
    Bsz, L, Di = x.shape
    y = np.zeros_like(x)
    for b in range(Bsz):
        for d in range(Di):
            delta = softplus_lib(dt[b, :, d] + f["dt_bias"][d])
            y[b, :, d] = silu_lib(z[b, :, d]) * ssd_matrix_direction(delta, x[b, :, d], f["B"][b], f["C"][b],
                                                                     f["A"][d], f["D"][d], True, seg_len)
    if swap:
        T = seg_len or L
        first = np.arange(0, L, T)
        last = first + T - 1
        perm = np.arange(L)
        perm[first], perm[last] = last, first
        out = np.empty_like(y)
        out[:, perm] = y            # the output of token t goes to position perm[t]
        y = out
    return y


@pytest.mark.parametrize("B,L,Di,N,seg,swap", [(2, 9, 3, 4, 0, False), (2, 9, 3, 4, 0, True), (1, 12, 2, 16, 4, True),
                                               (1, 12, 2, 16, 3, False), (2, 1, 2, 3, 0, True), (1, 6, 2, 5, 1, True)])
def test_fwd_matches_brute_force(B, L, Di, N, seg, swap):
    f = fwd_inputs(random_case(B, L, Di, N, 50 + L))
    np.testing.assert_allclose(oracle.fwd(f, seg_len=seg, swap=swap), brute_fwd(f, seg, swap), rtol=1e-10, atol=1e-12)


def test_fwd_is_the_bidirectional_scan_without_its_backward_branch():
    inp = random_case(3, 14, 5, 16, 61)
    off = dict(inp)
    off["B_b"] = np.zeros_like(inp["B_b"])
    off["D_b"] = np.zeros_like(inp["D_b"])
    np.testing.assert_allclose(oracle.fwd(fwd_inputs(inp)), oracle.bidir_fwd(off), rtol=1e-13, atol=1e-14)


def test_swap_exchanges_only_the_end_rows():
    f = fwd_inputs(random_case(2, 10, 4, 8, 62))
    a, b = oracle.fwd(f, seg_len=5), oracle.fwd(f, seg_len=5, swap=True)
    for s0 in (0, 5):
        assert np.array_equal(b[:, s0], a[:, s0 + 4]) and np.array_equal(b[:, s0 + 4], a[:, s0])
        assert np.array_equal(b[:, s0 + 1:s0 + 4], a[:, s0 + 1:s0 + 4])


FWD_MUTATIONS = {
    "swap_ignores_segments": ("const int64_t first = (t / T) * T, last = first + T - 1;",
                              "const int64_t first = 0, last = L - 1;"),
    "swap_to_neighbour": ("if (swap && t == first) dst = last;", "if (swap && t == first) dst = first + 1;"),
    "swap_one_way": ("else if (swap && t == last) dst = first;", ""),
    "fwd_ungated": ("y[(b * L + dst) * Di + d] = vimscan_oracle_silu(z[i]) * of[t];", "y[(b * L + dst) * Di + d] = of[t];"),
    "fwd_scans_backward": ("seg_len, +1,\n                                   h, of);", "seg_len, -1,\n                                   h, of);"),
}


def _build_variant(tmp_path, name, src):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(so), str(c), "-lm"],
                   check=True)
    return oracle.load_variant(str(so))


def _fwd_battery(lib):
    failed = []
    for name, (B, L, Di, N, seg, swap) in {"p_plain": (2, 9, 3, 4, 0, False), "p_swap": (2, 9, 3, 4, 0, True),
                                            "p_seg_swap": (1, 12, 2, 16, 4, True)}.items():
        try:
            f = fwd_inputs(random_case(B, L, Di, N, 50 + L))
            ok = np.allclose(oracle.fwd(f, seg_len=seg, swap=swap, lib=lib), brute_fwd(f, seg, swap), rtol=1e-10,
                             atol=1e-12)
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    return failed


def test_unmodified_source_passes_fwd_battery(tmp_path):
    assert _fwd_battery(_build_variant(tmp_path, "orig", SRC)) == []


@pytest.mark.parametrize("name", sorted(FWD_MUTATIONS))
def test_each_fwd_mutation_is_caught(tmp_path, name):
    old, new = FWD_MUTATIONS[name]
    assert SRC.count(old) == 1, f"pattern for {name} must occur once in the oracle source"
    assert _fwd_battery(_build_variant(tmp_path, name, SRC.replace(old, new))), f"no pin caught {name}"
