"""Throughput of the bidirectional selective scan on one MI355X.

One step = one call of the whole path (forward scan, backward scan, gate) over one batch of the
Vim-S workload (batch 128, 197 tokens, d_inner 768, N 16, bf16 I/O, fp32 state). Prints one JSON
line. ``value`` is GB/s of algorithmic traffic (read x, dt, z, B_f, C_f, B_b, C_b and the fp32
parameters once, write y once) over the K timed steps. The timed steps are replays of HIP graphs
holding one whole library call (the scan kernel, with the chunk passes when the plan has them) per input copy, so host
launch work is off the critical path (``--no-graph`` times eager calls instead); the per-kernel times
come from an eager pass in which the library records its events around the scan kernel. The steps rotate over several copies of the
inputs (more than the 256 MB Infinity Cache holds), so every step reads its inputs from HBM.

Also reported: the dominant kernel's ALU roofline (the scan's exponentials and fp32 arithmetic
bind before HBM does; that kernel is timed alone with HIP events the library records around it),
the same path with the per-state exponential forced (general_decay), the directional convolution
fused in front (conv_fused), the forward-only scan with and without the auxiliary-token swap, the
scan in a given token order (ordered: local windows of the patch grid), the NC-SSD global-state form on the same shape (ncssd: an HBM roofline, on the matrix cores), and the
float64 CPU oracle timed on this host's cores.

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
FP32_VECTOR_TFLOPS = 157.3    # MI355X fp32 vector peak, published: packed FMA, 256 CU x 128 lanes x 2 x 2.4 GHz
# Issue peak of the fp32 VALU without packed instructions (the library is compiled without them): each of
# the 4 SIMDs of a CU issues one wave64 instruction per 4 cycles, 16 lanes a cycle, so
# 256 CU x 64 lanes x 2.4 GHz lane-operations per second.
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
CACHE_BYTES = 256 * 2 ** 20   # Infinity Cache
SETTLE_S = 0.15               # untimed device work before every leg's warm-up (clock ramp)
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_vim_s.json")
KERNEL_SOURCE = os.path.join(ROOT, "bidirectional_selective_scan_amd", "csrc", "vimscan.hip")
NCSSD_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_ncssd_vim_s.json")
NCSSD_SOURCE = os.path.join(ROOT, "bidirectional_selective_scan_amd", "csrc", "ncssd.hip")
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense matrix peaks, published

# ALU work of the scan per (batch, token, channel), in fp32 VALU lane-operations: an FMA,
# multiply, add, compare or select is one; a transcendental (exp2, log2, rcp) counts two: on the
# scan kernel the SQ counters give 4.19 cycles per VALU instruction with 4.7% transcendental and
# 4.76 with 19% (profiles/valu_*), i.e. 4 cycles per wave64 FMA and 8 per transcendental.
# Per direction:
#   softplus in log2 units: fma(dt, log2e, bias*log2e), exp2, +1, log2, compare, select
#                                                                   4 ops + 2 transcendentals
#   u = delta*x                                                     1 op
#   transitions exp(delta*A[n]), 16 states:
#     general: 16 x (delta*A, exp2)                                16 ops + 16 transcendentals
#     geometric row A[n] = (n+1)*A[0]: delta*A0, exp2, 15 products 16 ops + 1 transcendental
#   u*B[n]: 16 multiplies; state h = h*e + u*B: 16 FMAs; readout C.h: 16 FMAs + 1 add
# Combine: yf + yb, + (D_f + D_b)*x, silu (-z*log2e, exp2, +1, rcp, *z), product
#                                                                   6 ops + 2 transcendentals
# Forward scan alone: one direction, then + D*x, silu, product      5 ops + 2 transcendentals
TRANS_OPS = 2


def alu_ops_per_element(geometric: bool, directions: int = 2) -> float:
    """Lane-operations per (b, t, d) of the bidirectional path, or of the forward scan alone
    (directions=1: no yf + yb add, so the gate stage is 5 ops + 2 transcendentals)."""
    per_dir_ops = 4 + 1 + 16 + 16 + 16 + 17
    per_dir_trans = 2 + (1 if geometric else 16)
    ops = directions * per_dir_ops + (6 if directions == 2 else 5)
    trans = directions * per_dir_trans + 2
    return ops + TRANS_OPS * trans


def kernel_source_hash(path: str = KERNEL_SOURCE) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(workload: str, path: str = PROFILE_TRAFFIC, source: str = KERNEL_SOURCE):
    """Per-launch HBM traffic of a kernel from a committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("kernel_source_sha256_16") != kernel_source_hash(source):
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp: dict, w) -> dict:
    import oracle
    t = oracle_seconds(inp, w.seg_len)
    cores = oracle.max_threads()
    return {"value": round(w.algorithmic_bytes() / t / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "seconds": round(t, 4), "cpu": cpu_model(),
            "tokens_channels_per_s": round(w.tokens_channels / t, 1),
            "sample": f"the full {w.name} batch in float64 on {cores} OpenMP threads, median of 3 runs "
                      f"({round(3 * t * cores, 1)} core-seconds in all)"}


def ncssd_leg(w, timed, stats_us, plan, nbytes, ncopies, value_wall=None, launch="eager library calls") -> dict:
    """The NC-SSD global-state form y = C (B^T (x . m)) on the workload's shape: HBM roofline of
    the call (its kernels bracketed by the library's events) and the matrix-core rate."""
    wall, per_call, per_kern = timed("ncssd")
    k = float(np.mean(per_kern))
    flops = 2 * 2 * w.tokens_channels * 16   # state B^T (x . m) and readout C H, N = 16
    peak = MFMA_PEAK_TFLOPS[w.io_dtype]
    gbs = nbytes / k / 1e9
    kernel = "k_ncssd_fused" if plan["chunks"] == 1 else "k_ncssd_state + k_ncssd_reduce + k_ncssd_out"
    return {"what": "NC-SSD global-state form y = C (B^T (x . m)), N = 16 (vimscan_ncssd_fwd)",
            "value": round(nbytes * len(per_call) / (value_wall(wall) if value_wall else wall) / 1e9, 2),
            "unit": "GB/s", "launch": launch, "call_us": stats_us(per_call), "kernel_us": round(k * 1e6, 3), "kernels_per_step": plan["kernels"],
            "input_copies": ncopies, "algorithmic_bytes": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": kernel,
                         "traffic": load_traffic(w.name, NCSSD_TRAFFIC, NCSSD_SOURCE)},
            "mfma": {"achieved": round(flops / k / 1e12, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(flops / k / 1e12 / peak, 5),
                     "basis": "algorithmic flops 4 x tokens x channels x N; the bf16 path issues twice that "
                              "(high and low parts of B*m and H)"}}


def oracle_seconds(inp_np: dict, seg_len: int, runs: int = 3) -> float:
    """Median wall time of the float64 oracle on one input set (host cores)."""
    import oracle
    oracle.build(force=False)
    x64 = {k: np.asarray(v, dtype=np.float64) for k, v in inp_np.items()}
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.bidir_fwd(x64, seg_len=seg_len)
        times.append(time.perf_counter() - t0)
    return float(np.median(times))


def configs_leg(graph_wall, dev, steps, headline=None, with_cpu=True):
    """Every workload at its full size (tiny, Vim-Ti, Vim-S, high-res, folded), timed as HIP graph
    replays of the whole library call with the plan's own chunking, on inputs drawn on the device
    with the same distributions; rotating input copies past the Infinity Cache (at most 64), timed
    over whole graphs of back-to-back calls (at least two of them: max(steps, 2 x copies) calls,
    rounded up to whole graphs), so that a small workload's time is its calls' and not the launch
    of a one-call graph per step. The
    headline workload's entry is the headline measurement itself (headline = (name, seconds per
    step)), so the line holds one number for it. With with_cpu, the float64 oracle is timed on each
    workload's inputs (median of 3 runs on the host's cores)."""
    import torch
    from bidirectional_selective_scan_amd import binding
    from bidirectional_selective_scan_amd.configs import WORKLOADS
    from bidirectional_selective_scan_amd.inputs import device_inputs
    io_names = ("x", "dt", "z", "B_f", "C_f", "B_b", "C_b")
    par_names = ("A_f", "A_b", "D_f", "D_b", "dt_bias_f", "dt_bias_b")
    res = {}
    for w in WORKLOADS:
        inp = device_inputs(w.batch, w.seqlen, w.d_inner, 16, w.io_dtype, seed=0, device=str(dev))
        nbytes = w.algorithmic_bytes()
        plan = binding.launch_info(w.batch, w.seqlen, w.d_inner, 16, w.seg_len, w.io_dtype)
        if headline is not None and headline[0] == w.name:
            step = headline[1]
            source = "the headline measurement"
        else:
            n = min(64, max(2, -(-2 * CACHE_BYTES // nbytes) + 1))
            copies = [[inp[k].clone() for k in io_names] for _ in range(n)]
            outs = [torch.empty_like(inp["x"]) for _ in range(n)]
            params = [inp[k] for k in par_names]
            ws = torch.empty(max(plan["workspace_bytes"], 1), dtype=torch.uint8, device=dev)
            nsteps = -(-max(steps, 2 * n) // n) * n
            wall = graph_wall(lambda i, s: binding.PreparedCall(*copies[i], *params, seg_len=w.seg_len, out=outs[i],
                                                                workspace=ws, stream=s), ncopy=n, steps=nsteps)
            step = wall / nsteps
            source = f"HIP graph replays of the whole call, {n} rotating input copies, {nsteps} calls"
            del copies, outs, ws
        ops = alu_ops_per_element(True) * w.tokens_channels
        res[w.name] = {"us_per_call": round(step * 1e6, 3), "gbs": round(nbytes / step / 1e9, 2),
                       "pct_hbm_peak": round(100 * nbytes / step / 1e9 / HBM_PEAK_GBS, 2),
                       "tokens_channels_per_s": round(w.tokens_channels / step, 1),
                       "alu_frac": round(ops / step / 1e12 / VALU_PEAK_TOPS, 4),
                       "source": source,
                       "plan": {k: plan[k] for k in ("chunk_len", "chunks", "workgroups", "kernels")}}
        if with_cpu:
            host = {k: (v.float().cpu().numpy() if v.dtype != torch.float32 else v.cpu().numpy())
                    for k, v in inp.items()}
            import oracle
            t = oracle_seconds(host, w.seg_len)
            res[w.name]["cpu"] = {"seconds": round(t, 4), "cores": oracle.max_threads(),
                                  "gbs": round(nbytes / t / 1e9, 4),
                                  "tokens_channels_per_s": round(w.tokens_channels / t, 1),
                                  "kind": "oracle (float64, median of 3)"}
            del host
        del inp
    return res


# Shapes of the forced-chunk sweep (--chunk-sweep): the five workloads and five more of the same
# family, bidirectional, then three forward only (batch, tokens, d_inner, io dtype, seg_len,
# forward only).
SWEEP_SHAPES = [
    (2, 65, 32, "f32", 0, False), (64, 197, 384, "f32", 0, False), (128, 197, 768, "bf16", 0, False),
    (8, 1025, 768, "bf16", 0, False), (1, 13056, 1536, "bf16", 51, False), (1, 1025, 768, "bf16", 0, False),
    (2, 4097, 768, "bf16", 0, False), (16, 197, 768, "bf16", 0, False), (8, 577, 768, "bf16", 0, False),
    (32, 257, 192, "f32", 0, False),
    (128, 197, 768, "bf16", 0, True), (64, 197, 384, "f32", 0, True), (8, 1025, 768, "bf16", 0, True),
]
SWEEP_CHUNK_COUNTS = (1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16, 20, 24, 28, 32, 40, 48, 64, 80, 96, 128)


def chunk_sweep(dev, steps, warmup, settle_s):
    """Every shape of SWEEP_SHAPES with the plan's own chunking and with forced chunk lengths: the
    even split ceil(L / K) into K chunks for each K of SWEEP_CHUNK_COUNTS that gives 8 to 256
    tokens per chunk. HIP graph replays of the whole call on rotating input copies, microseconds
    per call. Prints one JSON line per shape and returns them."""
    import torch
    from bidirectional_selective_scan_amd import binding
    from bidirectional_selective_scan_amd.inputs import device_inputs
    io_names = ("x", "dt", "z", "B_f", "C_f", "B_b", "C_b")
    par_names = ("A_f", "A_b", "D_f", "D_b", "dt_bias_f", "dt_bias_b")
    out = []
    for B, L, Di, io, seg, fwd in SWEEP_SHAPES:
        Lp = seg or L
        inp = device_inputs(B, L, Di, 16, io, seed=0, device=str(dev))
        nbytes = sum(int(inp[k].numel() * inp[k].element_size()) for k in io_names) + B * L * Di * (2 if io == "bf16" else 4)
        n = min(64, max(2, -(-2 * CACHE_BYTES // nbytes) + 1))
        copies = [[inp[k].clone() for k in io_names] for _ in range(n)]
        outs = [torch.empty_like(inp["x"]) for _ in range(n)]
        params = [inp[k] for k in par_names]
        plan = binding.launch_info(B, L, Di, 16, seg, io, forward_only=fwd)

        def prep(i, T, ws):
            if fwd:
                return binding.prepare_fwd(*copies[i][:5], params[0], params[2], params[4], seg_len=seg, out=outs[i],
                                           chunk_len=T, workspace=ws, stream=torch.cuda.current_stream().cuda_stream)
            return binding.PreparedCall(*copies[i], *params, seg_len=seg, out=outs[i], workspace=ws, chunk_len=T,
                                        stream=torch.cuda.current_stream().cuda_stream)
        cands = [0] + sorted({-(-Lp // K) for K in SWEEP_CHUNK_COUNTS if 8 <= -(-Lp // K) <= 256})
        times = {}
        for T in cands:
            wsb = binding.workspace_bytes(B, L, Di, 16, seg, io, chunk_len=T, forward_only=fwd)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
            calls = [prep(i, T, ws) for i in range(n)]
            for c in calls:
                c()
            torch.cuda.synchronize(dev)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in [prep(i, T, ws) for i in range(n)]:
                    c()
            t_end = time.perf_counter() + settle_s
            while True:   # clock ramp, then warm-up replays
                g.replay()
                torch.cuda.synchronize(dev)
                if time.perf_counter() >= t_end:
                    break
            reps = max(1, warmup // n)
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize(dev)
            reps = max(1, -(-steps // n))
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize(dev)
            times[T] = (time.perf_counter() - t0) / (reps * n) * 1e6
            del g, calls, ws
        forced = {T: v for T, v in times.items() if T}
        best_T = min(forced, key=forced.get)
        rec = {"shape": {"batch": B, "seqlen": L, "d_inner": Di, "io": io, "seg_len": seg, "forward_only": fwd},
               "plan": {"chunk_len": plan["chunk_len"], "chunks": plan["chunks"], "kernels": plan["kernels"]},
               "plan_us": round(times[0], 2), "best_chunk_len": best_T, "best_us": round(forced[best_T], 2),
               "plan_over_best": round(times[0] / forced[best_T], 4),
               "us_by_chunk_len": {str(T): round(v, 2) for T, v in forced.items()}}
        print(json.dumps(rec), flush=True)
        out.append(rec)
        del copies, outs, inp
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # Untimed calls before every leg's timed steps. Each leg first runs the same call untimed for
    # SETTLE_S seconds (the GPU needs tens of milliseconds of continuous work to reach its steady
    # clocks: after 10 calls from idle the Vim-S step measured ~125 us, after 500 ~101 us), then
    # the W warm-up calls, then the K timed steps.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed calls before each leg's warm-up (clock ramp; 0 for counter runs)")
    ap.add_argument("--workload", default=None, help="workload name (default: Vim-S)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-general", action="store_true", help="skip the forced general-decay measurement")
    ap.add_argument("--no-conv", action="store_true",
                    help="skip the measurement with the directional convolution (4 taps) in front of the scan")
    ap.add_argument("--no-fwd", action="store_true",
                    help="skip the forward-only scan measurements (with and without the auxiliary swap)")
    ap.add_argument("--no-ncssd", action="store_true", help="skip the NC-SSD global-state form measurement")
    ap.add_argument("--no-order", action="store_true",
                    help="skip the scan in a given token order (7 x 7 local windows of the patch grid)")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the scan on one GPU's share of an 8-way batch split (batch / 8)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config timings (every workload, graph replays of the whole call)")
    ap.add_argument("--no-copy", action="store_true", help="skip the device-copy bandwidth ceiling")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the headline steps as eager library calls instead of HIP graph replays")
    ap.add_argument("--only-ncssd", action="store_true",
                    help="measure only the NC-SSD global-state form (for its counter runs)")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="only time every sweep shape with the plan's chunking and with forced chunk lengths")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-mebibyte buffer 5 times (a known-size kernel for HBM counter scaling)")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs the scan on a single MI355X and has no "
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
    if args.chunk_sweep:
        recs = chunk_sweep(torch.device("cuda:0"), args.steps, args.warmup, args.settle)
        worst = max(r["plan_over_best"] for r in recs)
        print(json.dumps({"chunk_sweep_shapes": len(recs), "worst_plan_over_best": worst,
                          "within_3pct": sum(r["plan_over_best"] <= 1.03 for r in recs)}), flush=True)
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

    # mk[leg](i, stream) prepares the leg's call on input copy i (queued on `stream`, or torch's
    # current stream): eager calls time each call, graph replays of the same calls give `value`
    mk = {}
    for g in (False, True):
        mk[g] = (lambda g: lambda i, st=None: binding.PreparedCall(
            *copies[i], *params, seg_len=w.seg_len, out=outs[i], workspace=ws, general_decay=g, stream=st))(g)
    calls = {g: [mk[g](i) for i in range(ncopy)] for g in (False, True)}
    from bidirectional_selective_scan_amd.inputs import conv_params
    cp = conv_params(w.d_inner, 4, w.seed + 101)
    conv = tuple(torch.from_numpy(cp[k]).to(dev) for k in ("conv_w_f", "conv_b_f", "conv_w_b", "conv_b_b"))
    mk["conv"] = lambda i, st=None: binding.PreparedCall(*copies[i], *params, seg_len=w.seg_len, out=outs[i],
                                                         workspace=ws, conv=conv, stream=st)
    calls["conv"] = [mk["conv"](i) for i in range(ncopy)]
    # forward only: x, dt, z, B_f, C_f and the forward parameters of the same inputs
    for name, swap in (("fwd", False), ("fwd_swap", True)):
        mk[name] = (lambda swap: lambda i, st=None: binding.prepare_fwd(
            copies[i][0], copies[i][1], copies[i][2], copies[i][3], copies[i][4], params[0], params[2], params[4],
            seg_len=w.seg_len, out=outs[i], aux_swap=swap, stream=st))(swap)
        calls[name] = [mk[name](i) for i in range(ncopy)]

    # the same scan in a given token order: local windows of the patch grid (the grid is the
    # largest square the sequence holds; the remaining tokens keep their place)
    from bidirectional_selective_scan_amd.inputs import grid_order
    T = w.seg_len or w.seqlen
    side = int(np.sqrt(T - 1)) if T > 1 else 1
    order_np = np.tile(grid_order("local", side, T, window=max(1, (side + 1) // 2)), (w.batch * w.seqlen // T, 1))
    order = torch.from_numpy(np.ascontiguousarray(order_np, dtype=np.int32)).to(dev)
    mk["order"] = lambda i, st=None: binding.PreparedCall(*copies[i], *params, seg_len=w.seg_len, out=outs[i],
                                                          workspace=ws, order=order, stream=st)
    calls["order"] = [mk["order"](i) for i in range(ncopy)]
    order_desc = f"{side} x {side} patch grid in {max(1, (side + 1) // 2)} x {max(1, (side + 1) // 2)} local windows"

    # NC-SSD on inputs of the same shape: x, B, C in the io dtype, m fp32
    from bidirectional_selective_scan_amd.inputs import ncssd_inputs
    nci = ncssd_inputs(w.batch, w.seqlen, w.d_inner, 16, w.io_dtype, w.seed)
    e_io = 2 if w.io_dtype == "bf16" else 4
    nc_bytes = 2 * w.tokens_channels * e_io + 2 * w.batch * w.seqlen * 16 * e_io + w.batch * w.seqlen * 4
    nc_copies = max(2, -(-2 * CACHE_BYTES // nc_bytes) + 1)
    nc_base = {k: torch.from_numpy(nci[k]).to(dev) for k in ("x", "B", "C", "m")}
    for k in ("x", "B", "C"):
        nc_base[k] = nc_base[k].to(tdt)
    nc_in = [{k: v.clone() for k, v in nc_base.items()} for _ in range(nc_copies)]
    nc_out = [torch.empty_like(t["x"]) for t in nc_in]
    mk["ncssd"] = lambda i, st=None: binding.PreparedNcssd(nc_in[i]["x"], nc_in[i]["B"], nc_in[i]["C"], nc_in[i]["m"],
                                                           seg_len=w.seg_len, out=nc_out[i], stream=st)
    calls["ncssd"] = [mk["ncssd"](i) for i in range(nc_copies)]

    stream = torch.cuda.current_stream(dev)

    def make_events(n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:   # a first record creates the HIP events
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize(dev)
        return evs

    def settle(run_one):
        """Untimed calls for args.settle seconds of wall time (at least 20 calls unless it is 0),
        then a synchronize."""
        if args.settle <= 0:
            return
        t_end = time.perf_counter() + args.settle
        i = 0
        while i < 20 or time.perf_counter() < t_end:
            run_one(i)
            i += 1
            if i % 20 == 0:
                torch.cuda.synchronize(dev)
        torch.cuda.synchronize(dev)

    def timed(which):   # False: automatic transitions, True: forced general, "conv": with the convolution
        cl = calls[which]
        ncopy = len(cl)
        settle(lambda i: cl[i % ncopy]())
        for i in range(args.warmup):
            cl[i % ncopy]()
        torch.cuda.synchronize(dev)
        call_ev = make_events(args.steps)   # around each whole call (every kernel of the path)
        scan_ev = make_events(args.steps)   # recorded by the library around the main scan kernel
        t0 = time.perf_counter()
        for i in range(args.steps):
            c = cl[i % ncopy]
            c.set_scan_events(scan_ev[i][0].cuda_event, scan_ev[i][1].cuda_event)
            call_ev[i][0].record(stream)
            c()
            call_ev[i][1].record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t0
        for c in cl:
            c.set_scan_events()
        per_call = np.array([a.elapsed_time(b) for a, b in call_ev]) * 1e-3   # seconds, GPU timeline
        per_scan = np.array([a.elapsed_time(b) for a, b in scan_ev]) * 1e-3
        return wall, per_call, per_scan

    def stats_us(v):
        return {"median": round(float(np.median(v)) * 1e6, 3), "min": round(float(np.min(v)) * 1e6, 3),
                "p90": round(float(np.percentile(v, 90)) * 1e6, 3), "mean": round(float(np.mean(v)) * 1e6, 3)}

    if args.only_ncssd:
        print(json.dumps({"ncssd": ncssd_leg(w, timed, stats_us, calls["ncssd"][0].plan, nc_bytes, nc_copies)}),
              flush=True)
        return 0
    wall, per_call, per_scan = timed(False)
    kernel_s = float(np.mean(per_scan))
    launch_mode = "eager library calls"
    def graph_wall(make, ncopy=ncopy, warmup=None, steps=None):
        """Wall time of `steps` (default args.steps) steps replayed from HIP graphs, each step the
        whole library call (every kernel of the path) on input copy i % ncopy; make(i, stream)
        prepares that call on the given stream. One graph holds ncopy consecutive steps,
        single-step graphs the rest."""
        warmup = args.warmup if warmup is None else warmup
        steps = args.steps if steps is None else steps
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(ncopy):
                make(i, side.cuda_stream)()
        stream.wait_stream(side)
        torch.cuda.synchronize(dev)
        def capture(idx):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in idx:
                    make(i, torch.cuda.current_stream().cuda_stream)()
            return g
        block = capture(range(ncopy))
        singles = [capture([i]) for i in range(ncopy)]
        settle(lambda i: singles[i % ncopy].replay())
        for i in range(warmup):
            singles[i % ncopy].replay()
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for _ in range(steps // ncopy):
            block.replay()
        for i in range(steps % ncopy):
            singles[i].replay()
        torch.cuda.synchronize(dev)
        return time.perf_counter() - t0

    def leg_wall(name, eager_wall, n=ncopy):
        """A leg's wall time for its `value`: its calls replayed from HIP graphs, like the headline
        steps (eager calls' wall time with --no-graph)."""
        return eager_wall if args.no_graph else graph_wall(mk[name], ncopy=n)
    leg_launch = "eager library calls" if args.no_graph else "HIP graph replays of the whole call"

    if not args.no_graph:
        # The headline steps: the whole call replayed from HIP graphs, so the host's per-call
        # launch work is not on the GPU's critical path.
        wall = graph_wall(lambda i, s: binding.PreparedCall(*copies[i], *params, seg_len=w.seg_len, out=outs[i],
                                                            workspace=ws, stream=s))
        launch_mode = (f"HIP graph replays ({ncopy} steps per graph, one per input copy, each step the whole "
                       f"library call)")
    ms_per_step = wall / args.steps * 1e3
    value = nbytes * args.steps / wall / 1e9

    geometric = True   # the workloads use A[d, n] = -(n+1): every row is (n+1) * A[d, 0]
    ops = alu_ops_per_element(geometric) * w.tokens_channels
    alu_tops = ops / kernel_s / 1e12
    traffic = load_traffic(w.name)
    hbm_gbs = nbytes / kernel_s / 1e9
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
        # x, dt, z, B, C and y are stored in the workload's io dtype; state, transitions and every
        # sum are fp32
        "dtype": w.io_dtype,
        "state_dtype": "f32",
        "data": "synthetic",
        "config": {**w.describe(), "chunks": plan["chunks"], "kernels_per_step": plan["kernels"],
                   "input_copies": ncopy, "launch": launch_mode,
                   "clock_policy": f"every leg runs its call untimed for {args.settle} s, then the {args.warmup} "
                                   f"warm-up calls, then the timed steps"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "call_us": stats_us(per_call),
        "kernel_us": round(kernel_s * 1e6, 3),
        "scan_kernel_us": stats_us(per_scan),
        "kernel_gbs": round(hbm_gbs, 2),
        "tokens_channels_per_s": round(w.tokens_channels / kernel_s, 1),
        # The metric's roofline: algorithmic bytes per launch of the dominant kernel (the scan) over
        # its mean duration between the HIP events the library records around it on its stream.
        "roofline": {"bound": "hbm", "achieved": round(hbm_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_bidir_scan", "algorithmic_bytes": nbytes,
                     # What binds the scan: the fp32 vector ALU (its lane-operation rate).
                     "binding": "alu",
                     "alu": {"achieved": round(alu_tops, 3), "peak": round(VALU_PEAK_TOPS, 3), "unit": "Top/s",
                             "frac": round(alu_tops / VALU_PEAK_TOPS, 4),
                             "ops_per_element": alu_ops_per_element(geometric),
                             "peak_basis": "fp32 VALU lane-operations per second without packed instructions "
                                           "(256 CU x 64 lanes x 2.4 GHz); a transcendental counts 2",
                             # against the packed-instruction issue rate behind the published 157.3 TFLOP/s
                             "frac_of_packed_peak": round(alu_tops / (2 * VALU_PEAK_TOPS), 4)}},
    }
    if not args.no_general:
        wall_g, per_call_g, per_scan_g = timed(True)
        kg = float(np.mean(per_scan_g))
        ops_g = alu_ops_per_element(False) * w.tokens_channels
        out["general_decay"] = {"value": round(nbytes * args.steps / leg_wall(True, wall_g) / 1e9, 2), "unit": "GB/s",
                                "launch": leg_launch,
                                "call_us": stats_us(per_call_g), "kernel_us": round(kg * 1e6, 3),
                                "alu_achieved_tops": round(ops_g / kg / 1e12, 3),
                                "alu_frac": round(ops_g / kg / 1e12 / VALU_PEAK_TOPS, 4),
                                "ops_per_element": alu_ops_per_element(False)}
    if not args.no_conv:
        wall_c, per_call_c, per_scan_c = timed("conv")
        kc = float(np.mean(per_scan_c))
        cbytes = nbytes + 2 * w.d_inner * 5 * 4    # plus the taps and biases of both directions
        # the convolution adds, per direction: 4 taps (FMAs), SiLU (3 ops + 2 transcendentals), and a
        # second skip-term FMA instead of the shared one
        ops_c = (alu_ops_per_element(geometric) + 2 * (4 + 3 + TRANS_OPS * 2) + 1) * w.tokens_channels
        out["conv_fused"] = {"what": "directional depthwise conv1d (4 taps) + SiLU fused in front of both scans",
                             "value": round(cbytes * args.steps / leg_wall("conv", wall_c) / 1e9, 2), "unit": "GB/s",
                             "launch": leg_launch,
                             "call_us": stats_us(per_call_c), "kernel_us": round(kc * 1e6, 3),
                             "alu_achieved_tops": round(ops_c / kc / 1e12, 3),
                             "alu_frac": round(ops_c / kc / 1e12 / VALU_PEAK_TOPS, 4)}
    if not args.no_fwd:
        e_io = 2 if w.io_dtype == "bf16" else 4
        fbytes = (w.tokens_channels * 4 * e_io + 2 * w.batch * w.seqlen * 16 * e_io
                  + (w.d_inner * 16 + 2 * w.d_inner) * 4)
        ops_f = alu_ops_per_element(geometric, directions=1) * w.tokens_channels
        for name, label in (("fwd", "forward_only"), ("fwd_swap", "forward_only_aux_swap")):
            wall_f, per_call_f, per_scan_f = timed(name)
            kf = float(np.mean(per_scan_f))
            out[label] = {"what": "forward scan alone (vimscan_fwd)" + (", with the auxiliary-token swap"
                                                                         if name == "fwd_swap" else ""),
                          "value": round(fbytes * args.steps / leg_wall(name, wall_f) / 1e9, 2), "unit": "GB/s",
                          "launch": leg_launch,
                          "call_us": stats_us(per_call_f), "kernel_us": round(kf * 1e6, 3),
                          "alu_achieved_tops": round(ops_f / kf / 1e12, 3),
                          "alu_frac": round(ops_f / kf / 1e12 / VALU_PEAK_TOPS, 4),
                          "ops_per_element": alu_ops_per_element(geometric, directions=1)}
    if not args.no_order:
        wall_o, per_call_o, per_scan_o = timed("order")
        ko = float(np.mean(per_scan_o))
        obytes = nbytes + w.batch * w.seqlen * 4   # plus the order
        out["ordered"] = {"what": "the same scan in a given token order (vimscan_bidir_order_fwd): " + order_desc,
                          "value": round(obytes * args.steps / leg_wall("order", wall_o) / 1e9, 2), "unit": "GB/s",
                          "launch": leg_launch,
                          "call_us": stats_us(per_call_o), "kernel_us": round(ko * 1e6, 3),
                          "alu_achieved_tops": round(ops / ko / 1e12, 3),
                          "alu_frac": round(ops / ko / 1e12 / VALU_PEAK_TOPS, 4)}
    if not args.no_ncssd:
        out["ncssd"] = ncssd_leg(w, timed, stats_us, calls["ncssd"][0].plan, nc_bytes, nc_copies,
                                 value_wall=lambda eager: leg_wall("ncssd", eager, nc_copies), launch=leg_launch)
    if not args.no_copy:
        # measured HBM ceiling: a device copy of 512 MiB (read + write 1 GiB), outside the Infinity Cache
        n = 512 * 2 ** 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ceil_gbs = 2 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst
        out["roofline"]["copy_ceiling"] = round(ceil_gbs, 1)
        out["roofline"]["frac_of_copy"] = round(nbytes / kernel_s / 1e9 / ceil_gbs, 4)
        if "ncssd" in out:
            out["ncssd"]["roofline"]["copy_ceiling"] = round(ceil_gbs, 1)
            out["ncssd"]["roofline"]["frac_of_copy"] = round(out["ncssd"]["roofline"]["achieved"] / ceil_gbs, 4)
    if not args.no_shard and w.batch % 8 == 0 and w.batch >= 8:
        # one GPU's share of an 8-way data-parallel split: the first batch / 8 rows of the same inputs
        bs = w.batch // 8
        sh = [[t[:bs] for t in copies[i]] for i in range(ncopy)]
        plan_s = binding.launch_info(bs, w.seqlen, w.d_inner, 16, w.seg_len, w.io_dtype)
        ws_s = torch.empty(max(plan_s["workspace_bytes"], 1), dtype=torch.uint8, device=dev)
        calls["shard"] = [binding.PreparedCall(*sh[i], *params, seg_len=w.seg_len, out=outs[i][:bs], workspace=ws_s)
                          for i in range(ncopy)]
        wall_s, per_call_s, per_scan_s = timed("shard")
        mode_s = "eager library calls"
        if not args.no_graph:
            wall_s = graph_wall(lambda i, s: binding.PreparedCall(*sh[i], *params, seg_len=w.seg_len, out=outs[i][:bs],
                                                                  workspace=ws_s, stream=s))
            mode_s = "HIP graph replays of the whole call"
        ks = float(np.mean(per_scan_s))
        step_s = wall_s / args.steps
        sbytes = (nbytes - (2 * w.d_inner * 16 + 4 * w.d_inner) * 4) // 8 + (2 * w.d_inner * 16 + 4 * w.d_inner) * 4
        out["shard_1_of_8"] = {"what": f"the scan on one GPU's share of an 8-way batch split (batch {bs})",
                               "value": round(sbytes / step_s / 1e9, 2), "unit": "GB/s",
                               "step_us": round(step_s * 1e6, 3), "launch": mode_s,
                               "eager_call_us": stats_us(per_call_s),
                               # the chunked path: the chunk aggregates, the carry combine, then
                               # the scan kernel the library's events bracket
                               "scan_kernel_us": round(ks * 1e6, 3),
                               "alu_frac_step": round(ops / 8 / step_s / 1e12 / VALU_PEAK_TOPS, 4),
                               "plan": {k: plan_s[k] for k in ("chunks", "workgroups", "park_in_workspace")}}
    if not args.no_configs and not args.no_graph:
        out["configs"] = configs_leg(graph_wall, dev, args.steps, headline=(w.name, wall / args.steps),
                                     with_cpu=not args.no_cpu)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
