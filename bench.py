"""Throughput of the bidirectional selective scan on one MI355X.

One step = one call of the whole path (forward scan, backward scan, gate) over one batch of the
Vim-S workload (batch 128, 197 tokens, d_inner 768, N 16, bf16 I/O, fp32 state). Prints one JSON
line. ``value`` is GB/s of algorithmic traffic (read x, dt, z, B_f, C_f, B_b, C_b and the fp32
parameters once, write y once) over the K timed steps. The steps rotate over several copies of the
inputs (more than the 256 MB Infinity Cache holds), so every step reads its inputs from HBM.

Also reported: the dominant kernel's ALU roofline (the scan's exponentials and fp32 arithmetic
bind before HBM does), the same path with the per-state exponential forced (general_decay), and
the float64 CPU oracle timed on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, published
FP32_VECTOR_TFLOPS = 157.3    # MI355X fp32 vector peak, published: 256 CU x 128 lanes x 2 flops x 2.4 GHz
CACHE_BYTES = 256 * 2 ** 20   # Infinity Cache
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_vim_s.json")
KERNEL_SOURCE = os.path.join(ROOT, "bidirectional_selective_scan_amd", "csrc", "vimscan.hip")

# ALU work of the scan per (batch, token, channel), in fp32 VALU issue slots: an FMA, multiply,
# add, compare or select is one slot per lane; a transcendental (exp2, log2, rcp) is four, since
# CDNA issues them at a quarter of the FMA rate and they do not overlap with it. Per direction:
#   softplus: v*log2e, exp2, +1, log2, *ln2, compare, select       5 ops + 2 transcendentals
#   u = delta*x, D*x                                                2 ops
#   transitions exp(delta*A[n]), 16 states:
#     general: 16 x (delta*A, exp2)                                16 ops + 16 transcendentals
#     arithmetic progression: delta*a0, delta*da, 2 exp2,
#                             q^2, q^4, 15 products                19 ops + 2 transcendentals
#   delta*x*B[n]: 16 multiplies; state h = h*e + ub: 16 FMAs; readout 16 FMAs + 3 adds
# Combine: yf + yb, silu (-z*log2e, exp2, +1, rcp, *z), product    5 ops + 2 transcendentals
TRANS_SLOTS = 4


def alu_slots_per_element(progression: bool) -> float:
    per_dir_ops = 5 + 2 + (19 if progression else 16) + 16 + 16 + 19
    per_dir_trans = 2 + (2 if progression else 16)
    ops = 2 * per_dir_ops + 5
    trans = 2 * per_dir_trans + 2
    return ops + TRANS_SLOTS * trans


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def load_traffic(workload: str):
    """Per-launch HBM traffic of the main scan kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    try:
        rec = json.load(open(PROFILE_TRAFFIC))
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp: dict, w) -> dict:
    import oracle
    oracle.build(force=False)
    x64 = {k: np.asarray(v, dtype=np.float64) for k, v in inp.items()}
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.bidir_fwd(x64, seg_len=w.seg_len)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": round(w.algorithmic_bytes() / t / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle", "seconds": round(t, 4),
            "sample": f"the full {w.name} batch in float64, median of 3 runs"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="workload name (default: Vim-S)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-general", action="store_true", help="skip the forced general-decay measurement")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-mebibyte buffer 5 times (a known-size kernel for HBM counter scaling)")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build runs the scan on a single MI355X and has no "
              "multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy * 2 ** 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return 0
    from bidirectional_selective_scan_amd import binding
    from bidirectional_selective_scan_amd.configs import HEADLINE, WORKLOADS
    from bidirectional_selective_scan_amd.inputs import make_workload_inputs

    w = WORKLOADS[HEADLINE] if args.workload is None else next(x for x in WORKLOADS if x.name == args.workload)
    dev = torch.device("cuda:0")
    inp = make_workload_inputs(w)
    tdt = torch.float32 if w.io_dtype == "f32" else torch.bfloat16
    io_names = ("x", "dt", "z", "B_f", "C_f", "B_b", "C_b")
    par_names = ("A_f", "A_b", "D_f", "D_b", "dt_bias_f", "dt_bias_b")
    base = {k: torch.from_numpy(np.array(inp[k])).to(dev).to(tdt) for k in io_names}
    params = [torch.from_numpy(np.array(inp[k])).to(dev) for k in par_names]
    nbytes = w.algorithmic_bytes()
    ncopy = max(2, -(-2 * CACHE_BYTES // nbytes) + 1)
    copies = [[base[k].clone() for k in io_names] for _ in range(ncopy)]
    outs = [torch.empty_like(base["x"]) for _ in range(ncopy)]
    plan = binding.launch_info(w.batch, w.seqlen, w.d_inner, 16, w.seg_len, w.io_dtype)
    ws = None
    if plan["workspace_bytes"]:
        ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=dev)

    calls = {g: [binding.PreparedCall(*copies[i], *params, seg_len=w.seg_len, out=outs[i], workspace=ws,
                                      general_decay=g) for i in range(ncopy)] for g in (False, True)}

    def step(i, general=False):
        calls[general][i % ncopy]()

    def timed(general):
        for i in range(args.warmup):
            step(i, general)
        torch.cuda.synchronize(dev)
        stream = torch.cuda.current_stream(dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step(i, general)
            ev[i][1].record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t0
        per = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3  # seconds per call, GPU timeline
        return wall, per

    wall, per = timed(False)
    ms_per_step = wall / args.steps * 1e3
    value = nbytes * args.steps / wall / 1e9
    kernel_s = float(np.mean(per))

    progression = True   # the workloads use A[d, n] = -(n+1), an arithmetic progression in n
    slots = alu_slots_per_element(progression) * w.tokens_channels
    alu_tflops = 2 * slots / kernel_s / 1e12
    traffic = load_traffic(w.name)
    out = {
        "metric": "bidirectional selective-scan GB/s & % HBM peak at Vim-S shape (B128,L197,Di768)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {**w.describe(), "chunks": plan["chunks"], "kernels_per_step": plan["kernels"],
                   "input_copies": ncopy},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernel_us": round(kernel_s * 1e6, 3),
        "kernel_gbs": round(nbytes / kernel_s / 1e9, 2),
        "tokens_channels_per_s": round(w.tokens_channels / kernel_s, 1),
        "roofline": {"bound": "alu", "achieved": round(alu_tflops, 3), "peak": FP32_VECTOR_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(alu_tflops / FP32_VECTOR_TFLOPS, 4),
                     "traffic": traffic,
                     "hbm": {"achieved": round(nbytes / kernel_s / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(nbytes / kernel_s / 1e9 / HBM_PEAK_GBS, 4)}},
    }
    if not args.no_general:
        wall_g, per_g = timed(True)
        kg = float(np.mean(per_g))
        slots_g = alu_slots_per_element(False) * w.tokens_channels
        out["general_decay"] = {"value": round(nbytes * args.steps / wall_g / 1e9, 2), "unit": "GB/s",
                                "kernel_us": round(kg * 1e6, 3),
                                "alu_frac": round(2 * slots_g / kg / 1e12 / FP32_VECTOR_TFLOPS, 4)}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
