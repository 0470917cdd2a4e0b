"""Parity of the NC-SSD global-state form (vimscan_ncssd_fwd) with the float64 oracle, on the GPU,
through the C ABI. Tolerances as for the scan: fp32 |y - y_ref| <= 1e-4 (1 + |y_ref|); bf16
|y - y_ref| <= 2e-2 max(|y_ref|, 0.1 rms(y_ref)). Inputs from the seeded NC-SSD recipe: x, B, C ~ N(0, 1),
token weights m in (1, e]."""
import numpy as np
import pytest
import torch

import oracle
from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.inputs import ncssd_inputs
from gpu_helpers import assert_close, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(inp, io):
    tdt = torch.float32 if io == "f32" else torch.bfloat16
    out = {k: torch.from_numpy(np.array(inp[k])).to(DEV).to(tdt) for k in ("x", "B", "C")}
    out["m"] = torch.from_numpy(np.array(inp["m"], dtype=np.float32)).to(DEV)
    return out


def _run(inp, io, seg_len=0, **kw):
    d = _dev(inp, io)
    y = binding.ncssd_fwd(d["x"], d["B"], d["C"], d["m"], seg_len=seg_len, **kw)
    torch.cuda.synchronize()
    return y


def _ref(inp, seg_len=0):
    return oracle.ncssd(inp["x"], inp["B"], inp["C"], inp["m"], seg_len=seg_len)


CASES = [
    # (batch, L, Di, N, io, seg_len, chunk_len)
    (2, 65, 32, 16, "f32", 0, 0),      # the tiny configuration's shape
    (2, 65, 32, 16, "bf16", 0, 0),
    (1, 1, 16, 16, "f32", 0, 0),       # a single token
    (3, 15, 48, 16, "bf16", 0, 0),     # one partial tile; a partial channel block
    (2, 16, 80, 16, "f32", 0, 0),      # exactly one tile
    (2, 17, 80, 32, "bf16", 0, 0),
    (1, 200, 144, 64, "f32", 0, 0),    # several tiles per wave, ragged tail
    (1, 200, 144, 64, "bf16", 0, 0),
    (2, 130, 96, 32, "f32", 0, 0),
    (1, 5 * 51, 64, 16, "bf16", 51, 0),   # folded sequences
    (2, 4 * 13, 32, 16, "f32", 13, 0),
    (2, 65, 32, 16, "f32", 0, 16),     # split into 5 ranges of 16 tokens
    (2, 65, 32, 16, "bf16", 0, 48),
    (1, 300, 208, 64, "bf16", 0, 64),
    (1, 300, 208, 32, "f32", 0, 100),  # 112-token ranges
    (3, 4 * 20, 64, 16, "bf16", 20, 16),  # folded and split
]


@pytest.mark.parametrize("B,L,Di,N,io,seg,chunk", CASES)
def test_matches_oracle(B, L, Di, N, io, seg, chunk):
    inp = ncssd_inputs(B, L, Di, N, io, seed=L + Di + N)
    y = _run(inp, io, seg, chunk_len=chunk)
    assert_close(to_f64(y), _ref(inp, seg), io, f"ncssd B={B} L={L} Di={Di} N={N} {io} seg={seg} chunk={chunk}")


FULL = [
    ("vim_ti_b64_l197_d384_f32", 64, 197, 384, "f32", 0),
    ("vim_s_b128_l197_d768_bf16", 128, 197, 768, "bf16", 0),
    ("highres_b8_l1025_d768_bf16", 8, 1025, 768, "bf16", 0),
    ("folded_256x51_d1536_bf16", 1, 256 * 51, 1536, "bf16", 51),
]


@pytest.mark.parametrize("name,B,L,Di,io,seg", FULL, ids=[f[0] for f in FULL])
def test_full_size_matches_oracle(name, B, L, Di, io, seg):
    """The workloads at full size, in the launch configuration the benchmark times, every output
    against the oracle."""
    inp = ncssd_inputs(B, L, Di, 16, io, seed=0)
    y = _run(inp, io, seg)
    assert_close(to_f64(y), _ref(inp, seg), io, name)


def test_split_and_whole_sequence_agree():
    inp = ncssd_inputs(2, 257, 64, 16, "f32", seed=3)
    whole = to_f64(_run(inp, "f32"))
    for chunk in (16, 64, 128):
        np.testing.assert_allclose(to_f64(_run(inp, "f32", chunk_len=chunk)), whole, rtol=2e-5, atol=2e-4)


def test_repeatable_bit_for_bit():
    inp = ncssd_inputs(4, 300, 128, 32, "bf16", seed=4)
    for chunk in (0, 64):
        a = _run(inp, "bf16", chunk_len=chunk)
        b = _run(inp, "bf16", chunk_len=chunk)
        assert torch.equal(a, b)


def test_folded_equals_unfolded_bit_for_bit():
    k, T = 6, 51
    unf = ncssd_inputs(k, T, 96, 16, "bf16", seed=5)
    fold = {n: a.reshape((1, k * T) + a.shape[2:]) for n, a in unf.items()}
    y_unf = _run(unf, "bf16")
    y_fold = _run(fold, "bf16", seg_len=T)
    assert torch.equal(y_fold.reshape(y_unf.shape), y_unf)


def test_segments_do_not_leak():
    """A NaN planted in one segment's x leaves every other segment's output unchanged."""
    k, T = 4, 20
    inp = ncssd_inputs(1, k * T, 64, 16, "f32", seed=6)
    base = _run(inp, "f32", seg_len=T)
    bad = {n: a.copy() for n, a in inp.items()}
    bad["x"][0, 2 * T + 3, 5] = np.nan
    y = _run(bad, "f32", seg_len=T)
    for s in range(k):
        seg = slice(s * T, (s + 1) * T)
        if s == 2:
            assert torch.isnan(y[0, seg]).any()
        else:
            assert torch.equal(y[0, seg], base[0, seg])


def test_empty_and_out_argument():
    x = torch.empty(0, 7, 32, device=DEV)
    B = torch.empty(0, 7, 16, device=DEV)
    m = torch.empty(0, 7, device=DEV)
    assert binding.ncssd_fwd(x, B, B, m).shape == (0, 7, 32)
    inp = ncssd_inputs(1, 9, 32, 16, "f32", seed=8)
    d = _dev(inp, "f32")
    out = torch.full_like(d["x"], 7.0)
    y = binding.ncssd_fwd(d["x"], d["B"], d["C"], d["m"], out=out)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    assert_close(to_f64(out), _ref(inp), "f32", "out=")


@pytest.mark.parametrize("chunk", [0, 64])
def test_timing_events_bracket_the_kernels(chunk):
    """The optional event pair is recorded around the call's kernels: its interval is positive
    and inside the interval of the whole call; the result is unchanged."""
    inp = ncssd_inputs(4, 197, 128, 16, "bf16", seed=9)
    d = _dev(inp, "bf16")
    call = binding.PreparedNcssd(d["x"], d["B"], d["C"], d["m"], chunk_len=chunk)
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:   # torch creates the HIP event at its first record
        e.record(s)
    torch.cuda.synchronize()
    call.set_scan_events(ev[1].cuda_event, ev[2].cuda_event)
    ev[0].record(s)
    call()
    ev[3].record(s)
    torch.cuda.synchronize()
    assert 0.0 < ev[1].elapsed_time(ev[2]) <= ev[0].elapsed_time(ev[3])
    assert_close(to_f64(call.out), _ref(inp), "bf16", "timed call")
