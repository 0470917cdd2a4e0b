"""Host logic of bench.py: the one-GPU guard, the counter-traffic record's source check, and the
lane-operation counts the ALU roofline divides by."""
import json
import subprocess
import sys

import bench


def test_more_than_one_gpu_is_refused_without_touching_a_device():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=bench.ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_is_used_only_for_the_source_it_was_taken_on(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("kernel source, first version\n")
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps({"workload": "w", "kernel_source_sha256_16": bench.kernel_source_hash(str(src)),
                               "bytes_per_launch": 12345}))
    assert bench.load_traffic("w", str(rec), str(src)) == 12345
    assert bench.load_traffic("other", str(rec), str(src)) is None
    src.write_text("kernel source, changed\n")
    assert bench.load_traffic("w", str(rec), str(src)) is None
    assert bench.load_traffic("w", str(tmp_path / "missing.json"), str(src)) is None


def test_lane_operation_counts_are_consistent():
    geo, gen = bench.alu_ops_per_element(True), bench.alu_ops_per_element(False)
    geo1, gen1 = bench.alu_ops_per_element(True, 1), bench.alu_ops_per_element(False, 1)
    # general transitions: 15 more exponentials per direction than the geometric form
    assert gen - geo == 2 * 15 * bench.TRANS_OPS
    assert gen1 - geo1 == 15 * bench.TRANS_OPS
    # the bidirectional path is the forward one plus a second direction and the add of the branches
    per_dir_geo = geo1 - (5 + 2 * bench.TRANS_OPS)
    assert geo == geo1 + per_dir_geo + 1
    assert geo == 162 and geo1 == 85
