"""The pins catch plausible mistakes in the oracle.

Each case compiles a copy of the oracle's C source with one deliberate mistake (a dropped
term, a wrong sign, index or operand, a swapped direction parameter) on the CPU, and checks that
at least one pin from test_oracle_pins fails against it. The unmodified source must pass them
all. Nothing here touches a GPU.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from test_oracle_pins import (random_case, ssd_matrix_bidir, softplus_lib, silu_lib, GOLDEN)

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "vimscan_oracle.c")).read()

MUTATIONS = {
    "bwd_uses_fwd_bias": ("D_b[d], dt_bias_b[d]", "D_b[d], dt_bias_f[d]"),
    "bwd_uses_fwd_B": ("scan_one_direction(x, dt, B_b, C_b, A_b", "scan_one_direction(x, dt, B_f, C_b, A_b"),
    "bwd_uses_fwd_A": ("C_b, A_b,", "C_b, A_f,"),
    "bwd_uses_fwd_D": ("D_b[d], dt_bias_b", "D_f[d], dt_bias_b"),
    "bwd_reset_at_t": ("(step > 0) ? t : (t + 1)", "t"),
    "fwd_reset_off_by_one": ("(step > 0) ? t : (t + 1)", "(t + 1)"),
    "skip_term_dropped": ("out[t] = y + Dd * xt;", "out[t] = y;"),
    "decay_without_delta": ("exp(delta * A[d * N + n])", "exp(A[d * N + n])"),
    "decay_sign": ("exp(delta * A[d * N + n])", "exp(-delta * A[d * N + n])"),
    "input_without_delta": ("delta * Bt[n] * xt", "Bt[n] * xt"),
    "input_uses_C": ("delta * Bt[n] * xt", "delta * Ct[n] * xt"),
    "readout_uses_B": ("y += Ct[n] * h[n];", "y += Bt[n] * h[n];"),
    "readout_before_update": ("h[n] = abar * h[n] + delta * Bt[n] * xt;\n            y += Ct[n] * h[n];",
                              "y += Ct[n] * h[n];\n            h[n] = abar * h[n] + delta * Bt[n] * xt;"),
    "A_transposed": ("A[d * N + n]", "A[n * Di + d]"),
    "gate_is_sigmoid": ("return v / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(-v));"),
    "silu_sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "softplus_branch": ("return v + log1p(exp(-v));", "return log1p(exp(-v));"),
    "branches_subtracted": ("(of[t] + ob[t])", "(of[t] - ob[t])"),
    "gate_on_x": ("vimscan_oracle_silu(z[i])", "vimscan_oracle_silu(x[i])"),
    "bwd_not_reversed": ("(step > 0) ? k : (L - 1 - k)", "k"),
    "dt_channel_dropped": ("dt[(b * L + t) * Di + d]", "dt[(b * L + t) * Di]"),
    "B_batch_dropped": ("Bm + (b * L + t) * N", "Bm + t * N"),
    "state_not_reset_between_dirs": ("    for (int64_t n = 0; n < N; ++n) h[n] = 0.0;\n    for (int64_t k = 0;",
                                     "    for (int64_t k = 0;"),
}


def _build_variant(tmp_path, name, src):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(so), str(c), "-lm"],
                   check=True)
    return oracle.load_variant(str(so))


def _battery(lib):
    """Run the pins against ``lib``; return the names of those that fail."""
    failed = []

    def check(name, fn):
        try:
            ok = fn()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)

    def p1():
        inp = random_case(2, 7, 3, 4, 1)
        y, yf, yb = oracle.bidir_fwd(inp, return_parts=True, lib=lib)
        ey, eyf, eyb = ssd_matrix_bidir(inp)
        return np.allclose(y, ey, rtol=1e-10, atol=1e-12) and np.allclose(yf, eyf, rtol=1e-10, atol=1e-12)

    def p1_reset():
        inp = random_case(2, 12, 3, 5, 11)
        y = oracle.bidir_fwd(inp, seg_len=3, lib=lib)
        return np.allclose(y, ssd_matrix_bidir(inp, 3)[0], rtol=1e-10, atol=1e-12)

    def p3():
        inp = random_case(2, 9, 4, 16, 7)
        inp["B_f"][:] = 0.0
        inp["B_b"][:] = 0.0
        y = oracle.bidir_fwd(inp, lib=lib)
        return np.allclose(y, silu_lib(inp["z"]) * (inp["D_f"] + inp["D_b"]) * inp["x"], rtol=1e-13)

    def p6():
        unf = random_case(5, 7, 6, 16, 10)
        fold = dict(unf)
        for k in ("x", "dt", "z", "B_f", "C_f", "B_b", "C_b"):
            fold[k] = unf[k].reshape((1, 35) + unf[k].shape[2:])
        return np.array_equal(oracle.bidir_fwd(fold, seg_len=7, lib=lib).reshape(5, 7, 6),
                              oracle.bidir_fwd(unf, lib=lib))

    def nonlin():
        vs = [-30.0, -2.0, 0.3, 4.0, 40.0]
        return all(np.isclose(lib.vimscan_oracle_softplus(v), softplus_lib(v), rtol=1e-14) and
                   np.isclose(lib.vimscan_oracle_silu(v), silu_lib(v), rtol=1e-14) for v in vs)

    check("p1", p1)
    check("p1_reset", p1_reset)
    check("p3", p3)
    check("p6", p6)
    check("nonlin", nonlin)
    return failed


def test_unmodified_source_passes_battery(tmp_path):
    lib = _build_variant(tmp_path, "orig", SRC)
    assert _battery(lib) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_each_mutation_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) >= 1, f"pattern for {name} not found in the oracle source"
    lib = _build_variant(tmp_path, name, SRC.replace(old, new, 1))
    assert _battery(lib), f"no pin caught the mutation {name}"
