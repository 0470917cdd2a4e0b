"""Summaries of rocprofv3 output for profiles/.

  python profile_summary.py trace --stats <run_kernel_stats.csv> --cmd "<command>" --out profiles/<name>.txt
      [--dispatches <run_kernel_trace.csv> --legs <kernel substring>=<label>:<n>,<label>:<n>,...]
      per-kernel call count and average / min / max duration from a --kernel-trace --stats run;
      with --legs, the dispatches of one kernel name are also split, in launch order, into
      consecutive legs of the given sizes (e.g. a benchmark's automatic and forced-general runs
      of the same kernel) and each leg is summarised.

  python profile_summary.py traffic --fetch <fetch counter csv> --write <write counter csv>
      --calib-fetch <csv> --calib-write <csv> --calib-bytes N --kernel <substring>
      --workload <name> --source <kernel source file> --cmd "<commands>" --out profiles/<name>.json
      HBM traffic per dispatch of one kernel from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
      each scaled by what the same counter reads for a plain copy of N bytes.

  python profile_summary.py valu --pmc <counter csv> --kernel <substring> --cus 256 --cmd "<command>"
      --out profiles/<name>.txt
      VALU issue evidence for one kernel from SQ counters (per dispatch, averaged): instructions per
      wave, the fraction of time the VALU was busy (SQ_ACTIVE_INST_VALU is in quad-cycles per SIMD,
      so busy = sum / CUs / GRBM_GUI_ACTIVE of one XCD), the shader clock implied by
      GRBM_GUI_ACTIVE over the dispatch time, and the share of waves' time spent waiting.

  python profile_summary.py sweep --jsonl <bench.py --chunk-sweep output> --cmd "<command>"
      --out profiles/<name>.txt
      the forced-chunk sweep as a table: per shape the plan's chunking and time, the best forced
      chunk length and time, their ratio, and every forced length's time.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import statistics


def kernel_stats(path):
    rows = list(csv.DictReader(open(path)))
    return rows


def counter_per_dispatch(path, kernel_substr, counter):
    """Mean over dispatches of ``counter`` for kernels whose name contains kernel_substr."""
    per = collections.defaultdict(float)
    for r in csv.DictReader(open(path)):
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r} in {path}")
    return statistics.mean(per.values()), len(per)


def largest_kernel_counter(path, counter):
    """Counter value (per dispatch, mean) of the kernel with the largest value: the copy kernel of a
    calibration run."""
    per = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
    top = max(per.values())
    picked = [v for v in per.values() if v > 0.5 * top]
    return statistics.mean(picked), names[max(per, key=per.get)]


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--stats", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--dispatches", default=None)
    t.add_argument("--legs", default=None)
    t.add_argument("--bench-json", default=None, help="the JSON line bench.py printed in the traced run")
    f = sub.add_parser("traffic")
    for k in ("fetch", "write", "calib_fetch", "calib_write", "kernel", "workload", "source", "cmd", "out"):
        f.add_argument("--" + k.replace("_", "-"), required=True)
    f.add_argument("--calib-bytes", type=int, required=True)
    v = sub.add_parser("valu")
    for k in ("pmc", "kernel", "cmd", "out"):
        v.add_argument("--" + k, required=True)
    v.add_argument("--cus", type=int, default=256)
    v.add_argument("--skip", type=int, default=0, help="ignore the first N dispatches of the kernel")
    v.add_argument("--take", type=int, default=0, help="then use N dispatches (0: all the rest)")
    v.add_argument("--xcds", type=int, default=8)
    w = sub.add_parser("sweep")
    for k in ("jsonl", "cmd", "out"):
        w.add_argument("--" + k, required=True)
    a = ap.parse_args()

    if a.what == "sweep":
        recs = [json.loads(x) for x in open(a.jsonl) if x.strip().startswith("{")]
        shapes = [r for r in recs if "shape" in r]
        lines = [f"command: {a.cmd}", "",
                 "HIP graph replays of the whole call (all kernels of the plan), rotating input copies; us per call.",
                 "plan = the library's own chunking (chunk_len 0); forced = each even split into K chunks.", "",
                 f"{'shape (batch, tokens, d_inner, io, seg_len, fwd)':50s} {'plan T x K':>11s} {'kern':>4s} "
                 f"{'plan_us':>8s} {'best T':>6s} {'best_us':>8s} {'plan/best':>9s}"]
        for r in shapes:
            sh = r["shape"]
            name = (f"({sh['batch']}, {sh['seqlen']}, {sh['d_inner']}, {sh['io']}, {sh['seg_len']}, "
                    f"{'fwd' if sh.get('forward_only') else 'bidir'})")
            pl = r["plan"]
            lines.append(f"{name:50s} {str(pl['chunk_len']) + ' x ' + str(pl['chunks']):>11s} {pl['kernels']:4d} "
                         f"{r['plan_us']:8.2f} {r['best_chunk_len']:6d} {r['best_us']:8.2f} {r['plan_over_best']:9.4f}")
        n3 = sum(r["plan_over_best"] <= 1.03 for r in shapes)
        lines += ["", f"plan within 3% of the best forced chunk length: {n3} of {len(shapes)} shapes; "
                      f"worst plan/best {max(r['plan_over_best'] for r in shapes):.4f}", "",
                  "every forced chunk length (T: us per call):"]
        for r in shapes:
            sh = r["shape"]
            lines.append(f"  ({sh['batch']}, {sh['seqlen']}, {sh['d_inner']}, {sh['io']}, {sh['seg_len']}, "
                         f"{'fwd' if sh.get('forward_only') else 'bidir'}): " +
                         " ".join(f"{t}:{v}" for t, v in r["us_by_chunk_len"].items()))
        open(a.out, "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return

    if a.what == "valu":
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        dur = {}
        for r in csv.DictReader(open(a.pmc)):
            if a.kernel in r["Kernel_Name"]:
                per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
                dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        order = sorted(per, key=int)[a.skip:]
        if a.take:
            order = order[:a.take]
        per = {k: per[k] for k in order}
        dur = {k: dur[k] for k in order}
        if not per:
            raise SystemExit(f"no dispatches of {a.kernel!r} in {a.pmc}")
        names = sorted({k for d in per.values() for k in d})
        mean = {k: statistics.mean(d[k] for d in per.values()) for k in names}
        dns = statistics.mean(dur.values())
        gui = mean["GRBM_GUI_ACTIVE"] / a.xcds            # cycles of one XCD (the counter sums the XCDs)
        waves = mean["SQ_WAVES"]
        lines = [f"command: {a.cmd}",
                 f"kernel: {a.kernel} (dispatches {a.skip + 1}..{a.skip + len(per)} of the run, averaged)", "",
                 "raw counters per dispatch:"]
        lines += [f"  {k:28s} {mean[k]:16.0f}" for k in names]
        lines += ["", "derived:",
                  f"  dispatch time (profiled)      {dns / 1e3:10.2f} us",
                  f"  shader clock                  {gui / dns:10.3f} GHz  (GRBM_GUI_ACTIVE per XCD / time)",
                  f"  VALU instructions per wave    {mean['SQ_INSTS_VALU'] / waves:10.0f}"]
        if "SQ_INSTS_VALU_TRANS_F32" in mean:
            lines.append(f"  of them transcendental       {mean['SQ_INSTS_VALU_TRANS_F32'] / waves:10.0f}")
        if "SQ_INSTS_SALU" in mean:
            lines.append(f"  SALU instructions per wave    {mean['SQ_INSTS_SALU'] / waves:10.0f}")
        lines += [f"  VALU busy                     {100 * mean['SQ_ACTIVE_INST_VALU'] / a.cus / gui:10.1f} %"
                  "  (sum SQ_ACTIVE_INST_VALU / CUs / GRBM_GUI_ACTIVE per XCD)",
                  f"  cycles per VALU instruction   {4 * mean['SQ_ACTIVE_INST_VALU'] / mean['SQ_INSTS_VALU']:10.2f}"
                  "  (per SIMD while busy)"]
        if "SQ_WAIT_INST_ANY" in mean and "SQ_WAVE_CYCLES" in mean:
            lines.append(f"  waves waiting (any)           {100 * mean['SQ_WAIT_INST_ANY'] / mean['SQ_WAVE_CYCLES']:10.1f} %"
                         "  of wave lifetime")
        open(a.out, "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return

    if a.what == "trace":
        rows = kernel_stats(a.stats)
        lines = [f"command: {a.cmd}", "",
                 f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share':>7s}"]
        for r in rows:
            name = r["Name"]
            short = name if len(name) <= 70 else name[:67] + "..."
            lines.append(f"{short:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.3f} "
                         f"{float(r['MinNs']) / 1e3:10.3f} {float(r['MaxNs']) / 1e3:10.3f} "
                         f"{float(r['Percentage']):6.2f}%")
        if a.dispatches and a.legs:
            sub, spec = a.legs.split("=", 1)
            durs = []
            for r in csv.DictReader(open(a.dispatches)):
                if sub in r["Kernel_Name"]:
                    durs.append((int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
            durs = [d for _, d in sorted(durs)]
            lines += ["", f"dispatches of the kernel whose name contains {sub!r}, in launch order:",
                      f"{'leg':>12s} {'calls':>6s} {'avg_us':>10s} {'median_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
            i = 0
            for part in spec.split(","):
                label, n = part.split(":")
                leg = durs[i:i + int(n)]
                i += int(n)
                lines.append(f"{label:>12s} {len(leg):6d} {statistics.mean(leg) / 1e3:10.3f} "
                             f"{statistics.median(leg) / 1e3:10.3f} {min(leg) / 1e3:10.3f} {max(leg) / 1e3:10.3f}")
        if a.bench_json:
            b = json.loads(open(a.bench_json).read().strip().splitlines()[-1])
            lines += ["", "bench.py in the traced run (HIP events the library records around the scan kernel):",
                      f"  automatic transitions   kernel_us mean {b['kernel_us']:.3f}, "
                      f"median {b['scan_kernel_us']['median']:.3f}"]
            labels = {"general_decay": "forced general", "conv_fused": "with the convolution",
                      "forward_only": "forward only", "forward_only_aux_swap": "forward only + swap",
                      "ordered": "in a given order", "ncssd": "NC-SSD (whole call)"}
            for key, label in labels.items():
                if key in b:
                    lines.append(f"  {label:23s} kernel_us mean {b[key]['kernel_us']:.3f}")
        open(a.out, "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))
        return

    fetch_kib, n1 = counter_per_dispatch(a.fetch, a.kernel, "FETCH_SIZE")
    write_kib, n2 = counter_per_dispatch(a.write, a.kernel, "WRITE_SIZE")
    cf_kib, cf_name = largest_kernel_counter(a.calib_fetch, "FETCH_SIZE")
    cw_kib, cw_name = largest_kernel_counter(a.calib_write, "WRITE_SIZE")
    f_scale = a.calib_bytes / (cf_kib * 1024.0)
    w_scale = a.calib_bytes / (cw_kib * 1024.0)
    rec = {
        "workload": a.workload,
        "kernel": a.kernel,
        "kernel_source_sha256_16": hashlib.sha256(open(a.source, "rb").read()).hexdigest()[:16],
        "fetch_kib_per_dispatch": round(fetch_kib, 1),
        "write_kib_per_dispatch": round(write_kib, 1),
        "dispatches": [n1, n2],
        "calibration": {"bytes": a.calib_bytes, "fetch_kib": round(cf_kib, 1), "write_kib": round(cw_kib, 1),
                        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                        "copy_kernel": cf_name[:80]},
        "fetch_bytes_per_launch": int(fetch_kib * 1024 * f_scale),
        "write_bytes_per_launch": int(write_kib * 1024 * w_scale),
        "bytes_per_launch": int(fetch_kib * 1024 * f_scale + write_kib * 1024 * w_scale),
        "command": a.cmd,
    }
    json.dump(rec, open(a.out, "w"), indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
