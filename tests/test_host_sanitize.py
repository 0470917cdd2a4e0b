"""The host side of the library (csrc/plan.cpp: the plans and argument checks every entry point
runs before its first HIP call, and the host-only entry points) built with the address and
undefined-behaviour sanitizers and driven through millions of plan calls and every argument error
(tests/sanitize/host_driver.cpp). plan.cpp is plain C++, so this needs no GPU and no HIP."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _build(tmp_path, sources, name):
    exe = str(tmp_path / name)
    cmd = ["g++"] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", exe] + sources
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path, [os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
                            os.path.join(ROOT, "bidirectional_selective_scan_amd", "csrc", "plan.cpp")], "host_driver")
    r = _run(exe)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "host driver ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_the_sanitizers_are_active(tmp_path):
    """The same flags on a program with a planted heap overflow and a planted signed overflow: both
    are reported (so a clean run above means something)."""
    src = tmp_path / "planted.cpp"
    src.write_text("#include <cstdlib>\n#include <climits>\nint main(int argc, char** argv) {\n"
                   "  int* p = static_cast<int*>(std::malloc(4 * sizeof(int)));\n"
                   "  int k = INT_MAX - 1 + argc;  // argc == 1: INT_MAX, no overflow yet\n"
                   "  if (argc > 1) { k += argc; return k; }\n"
                   "  p[argc + 3] = 1;  // one past the end\n  int r = p[0];\n  std::free(p);\n  return r;\n}\n")
    exe = _build(tmp_path, [str(src)], "planted")
    r = _run(exe)
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "runtime error: store" in r.stderr)
    r = subprocess.run([exe, "x"], capture_output=True, text=True, timeout=60,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode != 0 and "signed integer overflow" in r.stderr
