"""Float64 CPU oracle for the bidirectional selective scan.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg are
the only code that may import, build or call this package. The product path
(``bidirectional_selective_scan_amd``) never imports it, and this package imports nothing from
the product path: the two share no code. Inputs reach both from the seeded generator module.

The arithmetic lives in ``vimscan_oracle.c`` (plain C, double precision, OpenMP over
(batch, channel) pairs, a sequential loop over tokens inside each pair); its header states the
definition it follows and the passages of the source pages each step comes from. This module
builds it with gcc and calls it through ctypes.

Every part of the oracle is pinned by the ``not gpu`` tests against results fixed outside it:
the SSD quadratic (matrix) form by brute force, the convolution form and the geometric-series
closed form for a time-invariant system, the B = 0 skip path, the reversed-scan symmetry, the
bidirectional-sum identity at A = 0, folding with a periodic reset, the worked one-step and
decay examples, and a first-order IIR filter from scipy. The directional convolution is pinned
against torch's conv1d on zero-padded segments and the composed path against the plain scan run
on the convolved inputs. The NC-SSD global-state form is pinned against the running sums of its
simplified recurrence in both directions (the bidirectional-sum identity), against the pinned scan
at A = 0, and by the invariance of its state under a joint reordering of the tokens. The scan in
a given token order is pinned against the plain scan run on inputs gathered into that order
(numpy indexing) and scattered back, and against the reverse order, which swaps the two branches.
No function here is parity unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vimscan_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libvimscan_oracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc -O2 -fopenmp into oracle/_build/. Returns the .so path."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _declare(lib):
    lib.vimscan_oracle_bidir_f64.restype = ctypes.c_int
    lib.vimscan_oracle_bidir_f64.argtypes = [_D] * 13 + [ctypes.c_int64] * 5 + [_D] * 3 + [ctypes.c_int]
    lib.vimscan_oracle_softplus.restype = ctypes.c_double
    lib.vimscan_oracle_softplus.argtypes = [ctypes.c_double]
    lib.vimscan_oracle_silu.restype = ctypes.c_double
    lib.vimscan_oracle_silu.argtypes = [ctypes.c_double]
    lib.vimscan_oracle_max_threads.restype = ctypes.c_int
    lib.vimscan_oracle_max_threads.argtypes = []
    lib.vimscan_oracle_dirconv_f64.restype = ctypes.c_int
    lib.vimscan_oracle_dirconv_f64.argtypes = ([_D] * 3 + [ctypes.c_int64, ctypes.c_int] + [ctypes.c_int64] * 4
                                               + [_D])
    lib.vimscan_oracle_bidir_conv_f64.restype = ctypes.c_int
    lib.vimscan_oracle_bidir_conv_f64.argtypes = ([_D] * 5 + [ctypes.c_int64] + [_D] * 12 + [ctypes.c_int64] * 5
                                                  + [_D] * 3 + [ctypes.c_int])
    lib.vimscan_oracle_fwd_f64.restype = ctypes.c_int
    lib.vimscan_oracle_fwd_f64.argtypes = [_D] * 8 + [ctypes.c_int64] * 5 + [ctypes.c_int, _D, ctypes.c_int]
    lib.vimscan_oracle_bidir_order_f64.restype = ctypes.c_int
    lib.vimscan_oracle_bidir_order_f64.argtypes = ([_D] * 13 + [ctypes.POINTER(ctypes.c_int32)] + [ctypes.c_int64] * 5
                                                   + [_D, ctypes.c_int])
    lib.vimscan_oracle_ncssd_f64.restype = ctypes.c_int
    lib.vimscan_oracle_ncssd_f64.argtypes = [_D] * 4 + [ctypes.c_int64] * 5 + [_D, _D, ctypes.c_int]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def load_variant(so_path: str):
    """Open another build of the oracle's C source (the tests compile deliberately broken
    copies to show that the pins catch each mistake)."""
    return _declare(ctypes.CDLL(so_path))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_D)


ARG_ORDER = ("x", "dt", "z", "B_f", "C_f", "B_b", "C_b", "A_f", "A_b", "D_f", "D_b",
             "dt_bias_f", "dt_bias_b")


def bidir_fwd(inputs: dict, seg_len: int = 0, return_parts: bool = False, nthreads: int = 0,
              lib=None):
    """y = silu(z) * (y_fwd + y_bwd) in float64 for the arrays in ``inputs`` (keys as
    ``ARG_ORDER``; any float dtype, widened exactly to float64).

    Shapes: x, dt, z (B, L, Di); B_*, C_* (B, L, N); A_* (Di, N); D_*, dt_bias_* (Di,).
    Returns y, or (y, y_fwd, y_bwd) with ``return_parts``. ``lib`` selects another build
    (see ``load_variant``)."""
    lib = lib if lib is not None else _load()
    arrs = [_f64(inputs[k]) for k in ARG_ORDER]
    x = arrs[0]
    if x.ndim != 3:
        raise ValueError("x must be (batch, seqlen, d_inner)")
    Bsz, L, Di = x.shape
    N = arrs[3].shape[-1]
    expect = {"x": (Bsz, L, Di), "dt": (Bsz, L, Di), "z": (Bsz, L, Di), "B_f": (Bsz, L, N),
              "C_f": (Bsz, L, N), "B_b": (Bsz, L, N), "C_b": (Bsz, L, N), "A_f": (Di, N),
              "A_b": (Di, N), "D_f": (Di,), "D_b": (Di,), "dt_bias_f": (Di,), "dt_bias_b": (Di,)}
    for k, a in zip(ARG_ORDER, arrs):
        if a.shape != expect[k]:
            raise ValueError(f"{k}: shape {a.shape}, expected {expect[k]}")
    y = np.empty((Bsz, L, Di), dtype=np.float64)
    yf = np.empty_like(y) if return_parts else None
    yb = np.empty_like(y) if return_parts else None
    null = ctypes.cast(None, _D)
    rc = lib.vimscan_oracle_bidir_f64(*[_ptr(a) for a in arrs], Bsz, L, Di, N, int(seg_len),
                                      _ptr(y), _ptr(yf) if yf is not None else null,
                                      _ptr(yb) if yb is not None else null, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return (y, yf, yb) if return_parts else y


CONV_KEYS = ("conv_w_f", "conv_b_f", "conv_w_b", "conv_b_b")


def dirconv(x, w, cb, step: int, seg_len: int = 0, lib=None) -> np.ndarray:
    """One direction's convolution + SiLU in float64: x (B, L, Di), w (Di, K), cb (Di,);
    step +1 is the causal forward one, -1 the anti-causal backward one."""
    lib = lib if lib is not None else _load()
    x, w, cb = _f64(x), _f64(w), _f64(cb)
    Bsz, L, Di = x.shape
    if w.ndim != 2 or w.shape[0] != Di or cb.shape != (Di,):
        raise ValueError("w must be (Di, K) and cb (Di,)")
    u = np.empty_like(x)
    rc = lib.vimscan_oracle_dirconv_f64(_ptr(x), _ptr(w), _ptr(cb), w.shape[1], int(step), Bsz, L, Di,
                                        int(seg_len), _ptr(u))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return u


def bidir_conv_fwd(inputs: dict, seg_len: int = 0, return_parts: bool = False, nthreads: int = 0, lib=None):
    """The bidirectional scan with each direction's depthwise convolution + SiLU in front of it,
    in float64. ``inputs`` holds the ``ARG_ORDER`` arrays plus conv_w_f, conv_w_b (Di, K) and
    conv_b_f, conv_b_b (Di,). Returns y, or (y, y_fwd, y_bwd) with ``return_parts``."""
    lib = lib if lib is not None else _load()
    arrs = [_f64(inputs[k]) for k in ARG_ORDER]
    cw_f, cb_f, cw_b, cb_b = (_f64(inputs[k]) for k in CONV_KEYS)
    x = arrs[0]
    if x.ndim != 3:
        raise ValueError("x must be (batch, seqlen, d_inner)")
    Bsz, L, Di = x.shape
    N = arrs[3].shape[-1]
    K = cw_f.shape[-1]
    if cw_f.shape != (Di, K) or cw_b.shape != (Di, K) or cb_f.shape != (Di,) or cb_b.shape != (Di,):
        raise ValueError("conv weights must be (Di, K) and biases (Di,)")
    y = np.empty((Bsz, L, Di), dtype=np.float64)
    yf = np.empty_like(y) if return_parts else None
    yb = np.empty_like(y) if return_parts else None
    null = ctypes.cast(None, _D)
    rc = lib.vimscan_oracle_bidir_conv_f64(_ptr(x), _ptr(cw_f), _ptr(cb_f), _ptr(cw_b), _ptr(cb_b), K,
                                           *[_ptr(a) for a in arrs[1:]], Bsz, L, Di, N, int(seg_len),
                                           _ptr(y), _ptr(yf) if yf is not None else null,
                                           _ptr(yb) if yb is not None else null, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return (y, yf, yb) if return_parts else y


FWD_ORDER = ("x", "dt", "z", "B", "C", "A", "D", "dt_bias")


def fwd(inputs: dict, seg_len: int = 0, swap: bool = False, nthreads: int = 0, lib=None):
    """The unidirectional (forward) scan, gated: y = silu(z) * (C.h + D x), in float64, with the
    optional auxiliary swap of each sequence's (segment's) first and last output. ``inputs``
    holds x, dt, z (B, L, Di), B, C (B, L, N), A (Di, N), D, dt_bias (Di,)."""
    lib = lib if lib is not None else _load()
    arrs = [_f64(inputs[k]) for k in FWD_ORDER]
    x = arrs[0]
    if x.ndim != 3:
        raise ValueError("x must be (batch, seqlen, d_inner)")
    Bsz, L, Di = x.shape
    N = arrs[3].shape[-1]
    expect = {"x": (Bsz, L, Di), "dt": (Bsz, L, Di), "z": (Bsz, L, Di), "B": (Bsz, L, N), "C": (Bsz, L, N),
              "A": (Di, N), "D": (Di,), "dt_bias": (Di,)}
    for k, a in zip(FWD_ORDER, arrs):
        if a.shape != expect[k]:
            raise ValueError(f"{k}: shape {a.shape}, expected {expect[k]}")
    y = np.empty((Bsz, L, Di), dtype=np.float64)
    rc = lib.vimscan_oracle_fwd_f64(*[_ptr(a) for a in arrs], Bsz, L, Di, N, int(seg_len), int(bool(swap)), _ptr(y),
                                    int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return y


def bidir_order_fwd(inputs: dict, order, seg_len: int = 0, nthreads: int = 0, lib=None):
    """The bidirectional scan in a given token order (DefMamba page, sections 1 and 2.1), in
    float64: the forward path visits order[s][0..T-1] of every sequence (segment) s, the backward
    path the same tokens from the end of the list; outputs land at the tokens' own positions.
    ``inputs`` as ``bidir_fwd``; order (batch * L / T, T) integer, rows permutations of 0..T-1."""
    lib = lib if lib is not None else _load()
    arrs = [_f64(inputs[k]) for k in ARG_ORDER]
    x = arrs[0]
    Bsz, L, Di = x.shape
    N = arrs[3].shape[-1]
    T = seg_len if seg_len > 0 else L
    ordr = np.ascontiguousarray(np.asarray(order), dtype=np.int32)
    if ordr.shape != (Bsz * L // max(T, 1), T):
        raise ValueError(f"order must be (batch * seqlen / T, T) = ({Bsz * L // max(T, 1)}, {T})")
    y = np.empty((Bsz, L, Di), dtype=np.float64)
    rc = lib.vimscan_oracle_bidir_order_f64(*[_ptr(a) for a in arrs], ordr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                            Bsz, L, Di, N, int(seg_len), _ptr(y), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return y


def ncssd(x, B, C, m, seg_len: int = 0, return_state: bool = False, nthreads: int = 0, lib=None):
    """NC-SSD, the non-causal global-state form (VSSD page, sections 4.2.3 to 4.2.5), in float64:
    per sequence (segment when seg_len > 0) H = B^T (X . m) and y = C H. x (Bsz, L, Di);
    B, C (Bsz, L, N); m (Bsz, L), the weight 1/A_j of every token. Returns y, or (y, H) with
    ``return_state``, H of shape (Bsz * L / T, N, Di)."""
    lib = lib if lib is not None else _load()
    x, B, C, m = _f64(x), _f64(B), _f64(C), _f64(m)
    if x.ndim != 3:
        raise ValueError("x must be (batch, seqlen, d_inner)")
    Bsz, L, Di = x.shape
    N = B.shape[-1]
    if B.shape != (Bsz, L, N) or C.shape != (Bsz, L, N) or m.shape != (Bsz, L):
        raise ValueError("B, C must be (batch, seqlen, d_state) and m (batch, seqlen)")
    T = seg_len if seg_len > 0 else L
    y = np.empty((Bsz, L, Di), dtype=np.float64)
    H = np.empty((Bsz * L // max(T, 1), N, Di), dtype=np.float64) if return_state else None
    rc = lib.vimscan_oracle_ncssd_f64(_ptr(x), _ptr(B), _ptr(C), _ptr(m), Bsz, L, Di, N, int(seg_len), _ptr(y),
                                      _ptr(H) if H is not None else ctypes.cast(None, _D), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return (y, H) if return_state else y


def softplus(v: float) -> float:
    return _load().vimscan_oracle_softplus(float(v))


def silu(v: float) -> float:
    return _load().vimscan_oracle_silu(float(v))


def max_threads() -> int:
    return _load().vimscan_oracle_max_threads()


def sample_channels(inputs: dict, seg_len: int, b_idx, d_idx, nthreads: int = 0):
    """Oracle outputs for selected (b, d) channels only, every token: returns y[len(b_idx),
    L, len(d_idx)]. Channels are independent, so this slices the inputs to the chosen batch
    rows and channels and runs the full definition on that slice."""
    b_idx = np.asarray(b_idx)
    d_idx = np.asarray(d_idx)
    sub = {}
    for k in ("x", "dt", "z"):
        sub[k] = np.asarray(inputs[k])[b_idx][:, :, d_idx]
    for k in ("B_f", "C_f", "B_b", "C_b"):
        sub[k] = np.asarray(inputs[k])[b_idx]
    for k in ("A_f", "A_b"):
        sub[k] = np.asarray(inputs[k])[d_idx]
    for k in ("D_f", "D_b", "dt_bias_f", "dt_bias_b"):
        sub[k] = np.asarray(inputs[k])[d_idx]
    return bidir_fwd(sub, seg_len=seg_len, nthreads=nthreads)
