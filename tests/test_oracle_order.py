"""Pins of the oracle's scan in a given token order (DefMamba page, section 1: raster, Hilbert and
local-window orders; section 2.1: re-ranking by per-token index offsets), and a check that they
catch plausible mistakes in it; plus the order generators of the input module.

Expectations: the pinned plain bidirectional oracle run on inputs gathered into the order with
numpy indexing and its output scattered back to the token positions; the raster order, which is
the plain scan; and the reversed order, which is the plain scan with the two branches' parameters
exchanged. CPU only."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from bidirectional_selective_scan_amd.inputs import (_hilbert_xy, deformable_order, grid_order, random_orders)
from test_oracle_pins import random_case

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "vimscan_oracle.c")).read()
TOKEN_TENSORS = ("x", "dt", "z", "B_f", "C_f", "B_b", "C_b")


def gather_scatter(inp, order, seg_len=0, lib=None):
    """Plain oracle on the gathered sequences: sequence s of the gathered input holds token
    order[s][k] at position k; its output at k belongs to token order[s][k]."""
    Bsz, L, Di = inp["x"].shape
    T = seg_len or L
    S = Bsz * L // T
    g = dict(inp)
    for k in TOKEN_TENSORS:
        a = inp[k].reshape((S, T) + inp[k].shape[2:])
        g[k] = np.take_along_axis(a, order.reshape((S, T) + (1,) * (a.ndim - 2)).astype(np.int64), axis=1)
    yg = oracle.bidir_fwd({k: (v.reshape((S, T) + v.shape[2:]) if k in TOKEN_TENSORS else v) for k, v in g.items()},
                          lib=lib)
    y = np.empty_like(yg)
    np.put_along_axis(y, order.reshape(S, T, 1).astype(np.int64), yg, axis=1)
    return y.reshape(Bsz, L, Di)


@pytest.mark.parametrize("B,L,Di,N,seg", [(2, 9, 3, 4, 0), (1, 12, 2, 16, 4), (3, 1, 2, 5, 0), (2, 10, 4, 8, 5)])
def test_order_matches_gathered_plain_scan(B, L, Di, N, seg):
    inp = random_case(B, L, Di, N, 70 + L)
    T = seg or L
    order = random_orders(B * L // T, T, seed=L)
    np.testing.assert_allclose(oracle.bidir_order_fwd(inp, order, seg), gather_scatter(inp, order, seg),
                               rtol=1e-13, atol=1e-14)


def test_raster_order_is_the_plain_scan():
    inp = random_case(2, 13, 3, 16, 71)
    order = np.tile(np.arange(13, dtype=np.int32), (2, 1))
    np.testing.assert_array_equal(oracle.bidir_order_fwd(inp, order), oracle.bidir_fwd(inp))


def test_reverse_order_exchanges_the_branches():
    """Visiting the tokens from the last to the first makes the forward branch the plain scan's
    backward walk and vice versa: the result is the plain scan with the forward and backward
    parameters exchanged."""
    inp = random_case(2, 11, 3, 16, 72)
    order = np.tile(np.arange(10, -1, -1, dtype=np.int32), (2, 1))
    sw = dict(inp)
    for a, b in (("B_f", "B_b"), ("C_f", "C_b"), ("A_f", "A_b"), ("D_f", "D_b"), ("dt_bias_f", "dt_bias_b")):
        sw[a], sw[b] = inp[b], inp[a]
    np.testing.assert_allclose(oracle.bidir_order_fwd(inp, order), oracle.bidir_fwd(sw), rtol=1e-13, atol=1e-14)


def test_rejects_bad_orders():
    inp = random_case(1, 6, 2, 4, 73)
    with pytest.raises(ValueError):
        oracle.bidir_order_fwd(inp, np.array([[0, 1, 2, 3, 4, 6]], dtype=np.int32))
    with pytest.raises(ValueError):
        oracle.bidir_order_fwd(inp, np.zeros((2, 6), dtype=np.int32))


ORDER_MUTATIONS = {
    "forward_ignores_order": ("const int64_t t = ord[dir == 0 ? k : T - 1 - k];",
                              "const int64_t t = dir == 0 ? k : ord[T - 1 - k];"),
    "backward_not_reversed": ("const int64_t t = ord[dir == 0 ? k : T - 1 - k];", "const int64_t t = ord[k];"),
    "output_at_step": ("                        out[t] = acc + Dd * xt;", "                        out[k] = acc + Dd * xt;"),
    "readout_of_step_row": ("acc += Cm[row * N + n] * h[n];", "acc += Cm[(s * T + k) * N + n] * h[n];"),
    "gate_of_step": ("const int64_t i = (s * T + t) * Di + d;\n                    y[i] = vimscan_oracle_silu(z[i])",
                     "const int64_t i = (s * T + t) * Di + d;\n                    y[i] = vimscan_oracle_silu(z[(s * T + ord[t]) * Di + d])"),
}


def _build_variant(tmp_path, name, src):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(so), str(c), "-lm"],
                   check=True)
    return oracle.load_variant(str(so))


def _battery(lib):
    failed = []
    for name, (B, L, Di, N, seg) in {"plain": (2, 9, 3, 4, 0), "segments": (1, 12, 2, 16, 4)}.items():
        inp = random_case(B, L, Di, N, 70 + L)
        T = seg or L
        order = random_orders(B * L // T, T, seed=L)
        try:
            ok = np.allclose(oracle.bidir_order_fwd(inp, order, seg, lib=lib), gather_scatter(inp, order, seg),
                             rtol=1e-10, atol=1e-12)
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    return failed


def test_unmodified_source_passes_battery(tmp_path):
    assert _battery(_build_variant(tmp_path, "orig", SRC)) == []


@pytest.mark.parametrize("name", sorted(ORDER_MUTATIONS))
def test_each_mutation_is_caught(tmp_path, name):
    old, new = ORDER_MUTATIONS[name]
    assert SRC.count(old) == 1, f"pattern for {name} must occur once in the oracle source"
    assert _battery(_build_variant(tmp_path, name, SRC.replace(old, new))), f"no pin caught {name}"


# ---------------------------------------------------------------------------------------------
# The order generators


@pytest.mark.parametrize("kind,side,T", [("raster", 14, 197), ("local", 14, 197), ("hilbert", 16, 257),
                                         ("hilbert", 32, 1025), ("local", 7, 51)])
def test_grid_orders_are_permutations_keeping_extra_tokens(kind, side, T):
    o = grid_order(kind, side, T)
    assert o.dtype == np.int32 and sorted(o.tolist()) == list(range(T))
    mid = side * side // 2
    assert list(o[mid:mid + T - side * side]) == list(range(mid, mid + T - side * side))


def test_hilbert_steps_are_grid_neighbours():
    for n in (2, 4, 8, 32):
        cells = [_hilbert_xy(n, d) for d in range(n * n)]
        assert len(set(cells)) == n * n
        for a, b in zip(cells, cells[1:]):
            assert abs(a[0] - b[0]) + abs(a[1] - b[1]) == 1


def test_local_order_visits_each_window_whole():
    o = grid_order("local", 14, 196, window=7)
    for w in range(4):
        cells = {(int(t) // 14 // 7, int(t) % 14 // 7) for t in o[49 * w:49 * (w + 1)]}
        assert len(cells) == 1


def test_deformable_order_is_a_bounded_reranking():
    o = deformable_order(300, seed=3, scale=8.0)
    assert sorted(o.tolist()) == list(range(300))
    # a token moves by less than twice the offset bound
    assert np.abs(np.argsort(o) - np.arange(300)).max() < 16
