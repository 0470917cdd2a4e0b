"""The C ABI without a GPU: the library loads, exports every function include/vimscan.h declares,
plans launches, and rejects bad arguments with the documented status before any HIP call.

Every call here fails validation (or is host-only), so nothing reaches the device."""
import ctypes
import os
import re

import pytest

from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.configs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vimscan.h")

OK, NULL, SHAPE, SEGLEN, DTYPE, ALIGN, ALIAS, WORKSPACE, HIP, CHUNK, FLAGS, CONV, SCRATCH = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11, -12)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vimscan_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert "vimscan_bidir_fwd" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.EXPORTED)


def test_wait_timeouts_rejects_null_before_any_hip_call(lib):
    assert lib.vimscan_wait_timeouts(None) == NULL


def test_status_strings(lib):
    for code in range(0, -13, -1):
        s = binding.status_string(code)
        assert s and s != "unknown status"
    assert binding.status_string(-99) == "unknown status"
    assert binding.status_string(5) == "unknown status"
    assert b"gfx950" in lib.vimscan_version()


def test_plans_for_the_workloads(lib):
    plans = {w.name: binding.launch_info(w.batch, w.seqlen, w.d_inner, 16, w.seg_len, w.io_dtype) for w in WORKLOADS}
    vim_s = plans["vim_s_b128_l197_d768_bf16"]
    # one pass, one kernel (the B and C rows are staged in LDS by the scan itself, bf16 included)
    assert (vim_s["chunks"], vim_s["kernels"], vim_s["park_in_workspace"]) == (1, 1, 1)
    assert vim_s["workgroups"] == 128 * 6     # 4 waves: 2 channel blocks x 2 directions
    park = 128 * 12 * 197 * 64 * 4        # the park: one fp32 per token and lane
    assert vim_s["workspace_bytes"] == park
    folded = plans["folded_256x51_d1536_bf16"]
    assert (folded["sequences"], folded["seq_tokens"], folded["chunks"]) == (256, 51, 1)
    assert folded["park_in_workspace"] == 0 and folded["kernels"] == 1
    assert folded["workspace_bytes"] == 0
    hi = plans["highres_b8_l1025_d768_bf16"]
    # chunked, one kernel: the chunks hand their aggregates over through the workspace (carries,
    # delta sums and a tag word per direction, sequence, chunk and channel block)
    assert hi["chunks"] > 1 and hi["kernels"] == 1 and hi["workspace_bytes"] > 0
    assert hi["chunk_len"] * hi["chunks"] >= 1025 > hi["chunk_len"] * (hi["chunks"] - 1)
    assert hi["park_in_workspace"] == 0
    carry = 2 * 8 * hi["chunks"] * 16 * 768 * 4
    dsum = 2 * 8 * hi["chunks"] * 768 * 4
    tags = 2 * 8 * hi["chunks"] * 12 * 8
    assert hi["workspace_bytes"] == carry + dsum + tags
    # Vim-Ti in one pass would be 192 workgroups, one per CU at most: it is cut into 4 chunks of 50
    # (768 workgroups), with the carries, delta sums and tags in the workspace and the park in LDS
    ti = binding.launch_info(64, 197, 384, 16, 0, "f32")
    assert (ti["chunk_len"], ti["chunks"], ti["workgroups"], ti["kernels"]) == (50, 4, 768, 1)
    carry, dsum, tags = 2 * 64 * 4 * 16 * 384 * 4, 2 * 64 * 4 * 384 * 4, 2 * 64 * 4 * 6 * 8
    assert ti["park_in_workspace"] == 0 and ti["workspace_bytes"] == carry + dsum + tags
    one_pass = binding.launch_info(64, 197, 384, 16, 0, "f32", chunk_len=197)
    assert one_pass["kernels"] == 1 and one_pass["workspace_bytes"] == one_pass["workgroups"] * 2 * 197 * 64 * 4
    # a forced chunk length is honoured and capped at 256 tokens
    assert binding.launch_info(2, 197, 64, chunk_len=16)["chunks"] == 13
    assert binding.launch_info(1, 1000, 64, chunk_len=5000)["chunk_len"] == 256


def test_chunk_count_follows_the_cost_model():
    """The bidirectional plan takes the chunk count of least modelled time (plan.cpp plan_cost:
    scan rounds, the one-pass kernel's aggregate walk and hand-over up to 16 chunks, the aggregate
    pass, combine and launches past that), fitted to a forced-chunk sweep on an MI355X; forward
    only keeps its rule. Choices below were each measured against every forced chunk count
    (bench.py --chunk-sweep): Vim-Ti 4 x 50 (46.6 us, best of 15), the high-res batch 16 x 65
    (62.5 us, best), one 1025-token sequence 41 x 25 (31.7 us; best 31.5 at 40 x 26), a 4097-token
    pair 64 x 65 (67.1 us, best), a 16-image Vim-S shard 5 x 40 (31.7 us, best), 8 x 577 tokens
    10 x 58 (43.4 us, best), the tiny case 9 x 8 (11.7 us, best; one pass 22 us)."""
    def plan(*shape, fwd=False):
        i = binding.launch_info(*shape, forward_only=fwd)
        return i["chunk_len"], i["chunks"], i["workgroups"]
    assert plan(64, 197, 384, 16, 0, "f32")[:2] == (50, 4)
    assert plan(8, 1025, 768, 16, 0, "bf16")[:2] == (65, 16)
    assert plan(1, 1025, 768, 16, 0, "bf16")[:2] == (25, 41)
    assert plan(2, 4097, 768, 16, 0, "bf16")[:2] == (65, 64)
    assert plan(16, 197, 768, 16, 0, "bf16")[:2] == (40, 5)
    assert plan(8, 577, 768, 16, 0, "bf16")[:2] == (58, 10)
    assert plan(2, 65, 32, 16, 0, "f32")[:2] == (8, 9)
    # enough workgroups for the chip: one pass (Vim-S, the folded stream)
    assert plan(128, 197, 768, 16, 0, "bf16")[:2] == (197, 1)
    assert plan(1, 13056, 1536, 16, 51, "bf16")[:2] == (51, 1)
    # forward only: a single pass from 1024 waves on (Vim-S: 64.5 us, best of 15); Vim-Ti 4 x 50
    # (38.2 us, best); the rule's round-filling refinement (a 16-image shard: 10 x 20)
    assert plan(128, 197, 768, 16, 0, "bf16", fwd=True)[:2] == (197, 1)
    assert plan(64, 197, 384, 16, 0, "f32", fwd=True) == (50, 4, 512)
    assert plan(16, 197, 768, 16, 0, "bf16", fwd=True) == (20, 10, 480)
    for shape in ((2, 400, 64), (1, 1025, 64), (4, 512, 768), (8, 1025, 768)):
        for fwd in (False, True):
            T, K, _ = plan(*shape, 16, 0, "bf16", fwd=fwd)
            assert 8 <= T <= 256 and K == -(-shape[1] // T)
    # up to 16 chunks one kernel computes, hands over and folds the aggregates itself (no aggregate
    # or carry-combine kernel); past that the aggregate pass, the combine and the scan
    assert binding.launch_info(16, 197, 768, 16, 0, "bf16")["kernels"] == 1
    assert binding.launch_info(8, 1025, 768, 16, 0, "bf16")["kernels"] == 1
    assert [binding.launch_info(1, 256, 64, 16, 0, "f32", chunk_len=t)["kernels"] for t in (256, 128, 16, 15)] == \
        [1, 1, 1, 3]
    # the element limit: chunks of at most 256 tokens, many rounds of workgroups, the combine kernel
    T, K, _ = plan(1, 2097151, 1024, 16, 0, "bf16")
    assert T <= 256 and K == -(-2097151 // T) and binding.launch_info(1, 2097151, 1024, 16, 0, "bf16")["kernels"] == 3


def _launch(**kw):
    base = dict(batch=2, seqlen=12, d_inner=64, d_state=16, io_dtype=binding.VIMSCAN_F32, chunk_len=0,
                general_decay=False, workspace=0, workspace_bytes=0, stream=0)
    base.update(kw)
    return binding.make_launch(**base)


def _call(lib, launch, ptrs=None, seg_len=0, y=None):
    # distinct, far-apart fake device addresses: never dereferenced, every case fails validation
    p = ptrs or [0x10000000 * (i + 1) for i in range(13)]
    y = 0x7F0000000 if y is None else y
    return lib.vimscan_bidir_fwd(*p, seg_len, y, ctypes.byref(launch) if launch is not None else None)


def test_null_arguments(lib):
    assert _call(lib, None) == NULL
    ptrs = [0x10000000 * (i + 1) for i in range(13)]
    for i in range(13):
        p = list(ptrs)
        p[i] = 0
        assert _call(lib, _launch(d_state=7), p) == SHAPE   # shape is checked first
        assert _call(lib, _launch(seqlen=12), p, seg_len=5) == SEGLEN
    # empty shapes launch nothing and accept NULL pointers
    assert _call(lib, _launch(batch=0), [0] * 13, y=0) == OK
    assert _call(lib, _launch(d_inner=0), [0] * 13, y=0) == OK
    assert _call(lib, _launch(batch=0, d_state=3), [0] * 13, y=0) == SHAPE
    p = list(ptrs)
    p[4] = 0
    launch = _launch(batch=1, seqlen=1, d_inner=1)
    assert _call(lib, launch, p) == NULL
    assert _call(lib, launch, ptrs, y=0) == NULL


@pytest.mark.parametrize("kw,code", [
    (dict(d_state=8), SHAPE), (dict(batch=-1), SHAPE), (dict(seqlen=-3), SHAPE), (dict(d_inner=-1), SHAPE),
    (dict(batch=1 << 20, seqlen=1 << 10, d_inner=1 << 2), SHAPE),
    (dict(io_dtype=2), DTYPE), (dict(chunk_len=-1), CHUNK), (dict(flags_raw=4), FLAGS),
])
def test_bad_launch_fields(lib, kw, code):
    flags = kw.pop("flags_raw", None)
    launch = _launch(**kw)
    if flags is not None:
        launch.flags = flags
    assert _call(lib, launch) == code


def test_seg_len(lib):
    assert _call(lib, _launch(seqlen=12), seg_len=-1) == SEGLEN
    assert _call(lib, _launch(seqlen=12), seg_len=5) == SEGLEN
    assert _call(lib, _launch(seqlen=12), seg_len=24) == SEGLEN


def test_alignment(lib):
    ptrs = [0x10000000 * (i + 1) for i in range(13)]
    bad = list(ptrs)
    bad[0] += 2                                   # fp32 x on a 2-byte boundary
    assert _call(lib, _launch(), bad) == ALIGN
    bad = list(ptrs)
    bad[3] += 2                                   # B_f must be 4-byte aligned even for bf16
    assert _call(lib, _launch(io_dtype=binding.VIMSCAN_BF16), bad) == ALIGN
    bad = list(ptrs)
    bad[7] += 1                                   # A_f
    assert _call(lib, _launch(), bad) == ALIGN
    assert _call(lib, _launch(), ptrs, y=0x7F0000001) == ALIGN


def test_alias(lib):
    ptrs = [0x10000000 * (i + 1) for i in range(13)]
    # y starts inside x's range (x holds 2*12*64*4 bytes)
    assert _call(lib, _launch(), ptrs, y=ptrs[0] + 256) == ALIAS
    # y ends inside A_b
    S = 2 * 12 * 64 * 4
    assert _call(lib, _launch(), ptrs, y=ptrs[8] - S + 4) == ALIAS
    # disjoint: touching but not overlapping is fine -> would launch, so only check the plan here


def test_workspace_required_for_chunked_plans(lib):
    launch = _launch(batch=1, seqlen=1025, d_inner=64)
    need = ctypes.c_size_t(0)
    assert lib.vimscan_workspace_bytes(ctypes.byref(launch), 0, ctypes.byref(need)) == OK and need.value > 0
    assert _call(lib, launch) == WORKSPACE
    launch.workspace = 0x50000000
    launch.workspace_bytes = need.value - 4
    assert _call(lib, launch) == WORKSPACE
    launch.workspace_bytes = need.value
    launch.workspace = 0x10000000 + 64       # overlaps x
    assert _call(lib, launch) == ALIAS


def test_noalloc_entry_point_arguments(lib):
    """vimscan_bidir_fwd_noalloc: the arguments of vimscan_bidir_fwd, checked the same way before
    any HIP call; a plan whose scratch exceeds the static array is VIMSCAN_ERR_SCRATCH."""
    ptrs = [0x10000000 * (i + 1) for i in range(13)]
    y = 0x7F000000

    def call(launch, p=ptrs, seg_len=0, yy=y):
        return lib.vimscan_bidir_fwd_noalloc(*p, seg_len, yy, ctypes.byref(launch) if launch is not None else None)

    assert call(None) == NULL
    assert call(_launch(d_state=8)) == SHAPE
    assert call(_launch(seqlen=12), seg_len=5) == SEGLEN
    assert call(_launch(io_dtype=2)) == DTYPE
    bad = list(ptrs)
    bad[0] += 2
    assert call(_launch(), bad) == ALIGN
    assert call(_launch(), ptrs, yy=ptrs[0] + 256) == ALIAS
    launch = _launch()
    launch.flags = binding.VIMSCAN_FLAG_FORWARD_ONLY
    assert call(launch) == FLAGS
    assert call(_launch(batch=0), [0] * 13, yy=0) == OK   # empty: nothing launched
    # Vim-S at batch 256: a 155 MB park, more than the 96 MiB array (x etc. spaced far apart)
    big = _launch(batch=256, seqlen=197, d_inner=768, io_dtype=binding.VIMSCAN_BF16)
    need = ctypes.c_size_t(0)
    assert lib.vimscan_workspace_bytes(ctypes.byref(big), 0, ctypes.byref(need)) == OK
    assert need.value > binding.NOALLOC_SCRATCH_BYTES
    far = [0x100000000 * (i + 1) for i in range(13)]
    assert call(big, far, yy=0x100000000 * 20) == SCRATCH
    # the batch-128 workload fits
    vim_s = _launch(batch=128, seqlen=197, d_inner=768, io_dtype=binding.VIMSCAN_BF16)
    assert lib.vimscan_workspace_bytes(ctypes.byref(vim_s), 0, ctypes.byref(need)) == OK
    assert 0 < need.value <= binding.NOALLOC_SCRATCH_BYTES


def test_workspace_bytes_rejects_bad_shapes(lib):
    need = ctypes.c_size_t(0)
    assert lib.vimscan_workspace_bytes(ctypes.byref(_launch(d_state=4)), 0, ctypes.byref(need)) == SHAPE
    assert lib.vimscan_workspace_bytes(ctypes.byref(_launch()), 0, None) == NULL
    assert lib.vimscan_workspace_bytes(None, 0, ctypes.byref(need)) == NULL


def _c_layout(struct, fields, tmp_path):
    """sizeof and offsetof of a header struct, from a C program compiled against the header."""
    import subprocess
    src = tmp_path / "layout.c"
    body = "".join(f'    printf("%zu\\n", offsetof({struct}, {f}));\n' for f in fields)
    src.write_text(f'#include <stddef.h>\n#include <stdio.h>\n#include "vimscan.h"\nint main(void) {{\n'
                   f'    printf("%zu\\n", sizeof({struct}));\n{body}    return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    return [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]


@pytest.mark.parametrize("cstruct,pystruct", [("vimscan_launch", binding._Launch), ("vimscan_plan", binding._Plan),
                                               ("vimscan_conv", binding._Conv)])
def test_binding_structs_match_the_header(cstruct, pystruct, tmp_path):
    fields = [f for f, _ in pystruct._fields_]
    size, *offsets = _c_layout(cstruct, fields, tmp_path)
    assert size == ctypes.sizeof(pystruct)
    assert offsets == [getattr(pystruct, f).offset for f in fields]


def _conv(k=4, base=0x60000000):
    return binding._Conv(base, base + 0x1000000, base + 0x2000000, base + 0x3000000, k)


def _call_conv(lib, launch, conv, ptrs=None, seg_len=0, y=None):
    p = ptrs or [0x10000000 * (i + 1) for i in range(13)]
    y = 0x7F0000000 if y is None else y
    return lib.vimscan_bidir_conv_fwd(p[0], ctypes.byref(conv) if conv is not None else None, *p[1:], seg_len, y,
                                      ctypes.byref(launch) if launch is not None else None)


def test_conv_arguments(lib):
    assert _call_conv(lib, _launch(), None) == NULL
    assert _call_conv(lib, None, _conv()) == NULL
    for k in (0, 5, -1):
        assert _call_conv(lib, _launch(d_state=3), _conv(k)) == CONV      # checked before the shape
    assert _call_conv(lib, _launch(d_state=3), _conv(4)) == SHAPE
    for f in ("w_f", "bias_f", "w_b", "bias_b"):
        c = _conv()
        setattr(c, f, 0)
        assert _call_conv(lib, _launch(), c) == NULL
        c = _conv()
        setattr(c, f, getattr(c, f) + 2)
        assert _call_conv(lib, _launch(), c) == ALIGN
    # y (2*12*64 fp32) overlapping the backward taps (64*4 fp32)
    c = _conv()
    assert _call_conv(lib, _launch(), c, y=c.w_b - 4 * 2 * 12 * 64 + 4) == ALIAS
    # the workspace overlapping a bias
    launch = _launch(batch=1, seqlen=1025, d_inner=64)
    need = ctypes.c_size_t(0)
    assert lib.vimscan_workspace_bytes(ctypes.byref(launch), 0, ctypes.byref(need)) == OK
    launch.workspace = c.bias_f - 64
    launch.workspace_bytes = need.value
    assert _call_conv(lib, launch, c) == ALIAS
    # empty shapes still accept NULL arrays once conv itself is valid
    assert _call_conv(lib, _launch(batch=0), _conv(), [0] * 13, y=0) == OK


def test_forward_only_plans(lib):
    f = binding.launch_info(128, 197, 768, 16, 0, "bf16", forward_only=True)
    b = binding.launch_info(128, 197, 768, 16, 0, "bf16")
    # one wave per channel block: 4 blocks per workgroup; no park, so no workspace in one pass
    assert f["park_in_workspace"] == 0
    ncb = 768 // 64
    assert f["workgroups"] == 128 * f["chunks"] * (ncb // 4)
    if f["chunks"] == 1:
        assert f["workspace_bytes"] == 0 and f["kernels"] == 1
    assert b["workspace_bytes"] > f["workspace_bytes"]
    s = binding.launch_info(128, 197, 768, 16, 0, "bf16", forward_only=True, aux_swap=True)
    assert s["kernels"] == f["kernels"] + 1
    hi = binding.launch_info(8, 1025, 768, 16, 0, "bf16", forward_only=True)
    assert hi["chunks"] > 1 and hi["kernels"] == (1 if hi["chunks"] <= 16 else 3)
    carry = 8 * hi["chunks"] * 16 * 768 * 4
    dsum = 8 * hi["chunks"] * 768 * 4
    tags = 8 * hi["chunks"] * 12 * 8 if hi["chunks"] <= 16 else 0
    assert hi["workspace_bytes"] == carry + dsum + tags
    # up to 16 chunks forward only is one kernel too (k_fwd_chain), with its tag words
    ti = binding.launch_info(64, 197, 384, 16, 0, "f32", forward_only=True)
    assert (ti["chunks"], ti["kernels"]) == (4, 1)
    assert ti["workspace_bytes"] == 64 * 4 * 17 * 384 * 4 + 64 * 4 * 6 * 8


def _call_fwd(lib, launch, ptrs=None, seg_len=0, y=None):
    p = ptrs or [0x10000000 * (i + 1) for i in range(8)]
    y = 0x7F0000000 if y is None else y
    return lib.vimscan_fwd(*p, seg_len, y, ctypes.byref(launch) if launch is not None else None)


def test_forward_only_arguments(lib):
    assert _call_fwd(lib, None) == NULL
    assert _call_fwd(lib, _launch(d_state=8)) == SHAPE
    assert _call_fwd(lib, _launch(seqlen=12), seg_len=5) == SEGLEN
    for i in range(8):
        p = [0x10000000 * (j + 1) for j in range(8)]
        p[i] = 0
        assert _call_fwd(lib, _launch(), p) == NULL
    assert _call_fwd(lib, _launch(batch=0), [0] * 8, y=0) == OK
    launch = _launch()
    launch.flags = 8
    assert _call_fwd(lib, launch) == FLAGS
    # the bidirectional entry points reject a forward-only launch
    launch = _launch()
    launch.flags = binding.VIMSCAN_FLAG_FORWARD_ONLY
    assert _call(lib, launch) == FLAGS
    assert _call_conv(lib, launch, _conv()) == FLAGS
    # y overlapping B (2*12*16 fp32)
    p = [0x10000000 * (j + 1) for j in range(8)]
    assert _call_fwd(lib, _launch(), p, y=p[3] + 64) == ALIAS


def test_ncssd_plans(lib):
    v = binding.ncssd_info(128, 197, 768, 16, 0, "bf16")
    # one workgroup per (sequence, 64 channels) holds the whole sequence: one kernel, no workspace
    assert (v["chunks"], v["kernels"], v["workgroups"], v["workspace_bytes"]) == (1, 1, 128 * 12, 0)
    f = binding.ncssd_info(1, 256 * 51, 1536, 16, 51, "bf16")
    assert (f["sequences"], f["seq_tokens"], f["kernels"], f["workspace_bytes"]) == (256, 51, 1, 0)
    h = binding.ncssd_info(8, 1025, 768, 16, 0, "bf16")
    # 96 (sequence, channel block) pairs are too few: the sequences are split
    assert h["chunks"] > 1 and h["kernels"] == 3 and h["chunk_len"] % 64 == 0
    assert h["chunks"] == -(-1025 // h["chunk_len"])
    hsz = 8 * 16 * 768 * 4
    assert h["workspace_bytes"] == -(-hsz * h["chunks"] // 256) * 256 + hsz
    c = binding.ncssd_info(2, 65, 32, 64, 0, "f32", chunk_len=20)   # rounded up to 32 tokens
    assert (c["chunk_len"], c["chunks"], c["kernels"]) == (32, 3, 3)
    assert c["workspace_bytes"] == 3 * 2 * 64 * 32 * 4 + 2 * 64 * 32 * 4
    assert binding.ncssd_info(2, 65, 32, 32, 0, "f32", chunk_len=1000)["chunks"] == 1


def _nc_launch(**kw):
    base = dict(batch=2, seqlen=12, d_inner=64, d_state=16, io_dtype=binding.VIMSCAN_F32, chunk_len=0,
                general_decay=False, workspace=0, workspace_bytes=0, stream=0)
    base.update(kw)
    return binding.make_launch(**base)


def _nc_plan(lib, launch, seg_len=0):
    plan = binding._Plan()
    return lib.vimscan_ncssd_plan(ctypes.byref(launch) if launch is not None else None, seg_len, ctypes.byref(plan))


@pytest.mark.parametrize("kw,code", [(dict(d_state=8), SHAPE), (dict(d_state=48), SHAPE), (dict(d_inner=40), SHAPE),
                                     (dict(batch=-1), SHAPE), (dict(io_dtype=7), DTYPE), (dict(chunk_len=-1), CHUNK),
                                     (dict(general_decay=True), FLAGS), (dict(d_state=64), OK), (dict(d_state=32), OK)])
def test_ncssd_plan_rejects_bad_launches(lib, kw, code):
    assert _nc_plan(lib, _nc_launch(**kw)) == code


def _call_nc(lib, launch, ptrs=None, seg_len=0, y=None):
    p = ptrs or [0x10000000 * (i + 1) for i in range(4)]
    y = 0x7F0000000 if y is None else y
    return lib.vimscan_ncssd_fwd(*p, seg_len, y, ctypes.byref(launch) if launch is not None else None)


def test_ncssd_arguments(lib):
    assert _call_nc(lib, None) == NULL
    assert _nc_plan(lib, None) == NULL
    assert _call_nc(lib, _nc_launch(seqlen=12), seg_len=5) == SEGLEN
    assert _nc_plan(lib, _nc_launch(seqlen=12), seg_len=5) == SEGLEN
    for i in range(4):
        p = [0x10000000 * (j + 1) for j in range(4)]
        p[i] = 0
        assert _call_nc(lib, _nc_launch(), p) == NULL
    assert _call_nc(lib, _nc_launch(), y=0) == NULL
    assert _call_nc(lib, _nc_launch(batch=0), [0] * 4, y=0) == OK
    # x and y need 16 bytes; C 8 (bf16) or 16 (fp32); fp32 B and m need 4
    for i, off, io in ((0, 8, binding.VIMSCAN_F32), (2, 4, binding.VIMSCAN_BF16), (2, 8, binding.VIMSCAN_F32),
                       (1, 2, binding.VIMSCAN_F32), (3, 2, binding.VIMSCAN_F32)):
        p = [0x10000000 * (j + 1) for j in range(4)]
        p[i] += off
        assert _call_nc(lib, _nc_launch(io_dtype=io), p) == ALIGN
    assert _call_nc(lib, _nc_launch(), y=0x7F0000008) == ALIGN
    # y overlapping x, or m
    p = [0x10000000 * (j + 1) for j in range(4)]
    assert _call_nc(lib, _nc_launch(), p, y=p[0] + 256) == ALIAS
    assert _call_nc(lib, _nc_launch(), p, y=p[3] - 64) == ALIAS
    # a split plan needs its workspace
    assert _call_nc(lib, _nc_launch(seqlen=64, chunk_len=16)) == WORKSPACE
    launch = _nc_launch(seqlen=64, chunk_len=16, workspace=0x50000000, workspace_bytes=16)
    assert _call_nc(lib, launch) == WORKSPACE


def _call_ord(lib, launch, ptrs=None, order=0x70000000, seg_len=0, y=None):
    p = ptrs or [0x10000000 * (i + 1) for i in range(13)]
    y = 0x7F0000000 if y is None else y
    return lib.vimscan_bidir_order_fwd(*p, order, seg_len, y, ctypes.byref(launch) if launch is not None else None)


def test_order_arguments(lib):
    assert _call_ord(lib, None) == NULL
    assert _call_ord(lib, _launch(), order=0) == NULL
    assert _call_ord(lib, _launch(batch=0), [0] * 13, order=0, y=0) == OK
    assert _call_ord(lib, _launch(), order=0x70000002) == ALIGN
    assert _call_ord(lib, _launch(d_state=8)) == SHAPE
    assert _call_ord(lib, _launch(seqlen=12), seg_len=5) == SEGLEN
    launch = _launch()
    launch.flags = binding.VIMSCAN_FLAG_FORWARD_ONLY
    assert _call_ord(lib, launch) == FLAGS
    # y overlapping the order (2 x 12 int32)
    assert _call_ord(lib, _launch(), y=0x70000000 - 64) == ALIAS
    # a walk in a given order spans a whole sequence: 2^18 tokens x 4096 fp32 channels is 4 GiB
    assert _call_ord(lib, _launch(batch=1, seqlen=1 << 18, d_inner=4096)) == SHAPE
    # the same shape in raster order passes the shape check (and then needs its workspace)
    assert _call(lib, _launch(batch=1, seqlen=1 << 18, d_inner=4096)) == WORKSPACE
