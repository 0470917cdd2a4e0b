"""Host replay of the memory indices the HIP kernels form, checked against the sizes of the
buffers they address, without a GPU.

For every launch of a call -- the scan kernels (plain, with the convolution, in a given order,
forward only), the chunk-aggregate pass, the carry fold and the carry-combine kernel, the
auxiliary swap, and the three NC-SSD passes -- this file recomputes, from the library's own plan
(vimscan_plan_launch / vimscan_ncssd_plan), the indices each workgroup, wave and lane forms:

* raw global loads and stores (row staging, order lookups, parameter rows, carries, delta sums,
  convolution window, swap, NC-SSD tiles, partial states and H), as element ranges of the tensor
  or workspace region they address;
* buffer resources (x, dt, z, y, the park): base offset plus range inside the tensor or region,
  and every offset formed against them inside the range (out-of-range buffer offsets would be
  dropped by the hardware, so they would lose data rather than fault: they must not occur either);
* LDS addresses against the dynamic LDS size of the launch and the 160 KB of a CU;
* the workspace layout against vimscan_workspace_bytes, the XCD remap of workgroup ids as a
  permutation of the grid, and the one-pass chunked kernel's workgroup order (a bijection onto
  sequence x channel-block group x chunk, chunk fastest) and tag words.

The index formulas restate the kernel code (vimscan.hip: wg_coords, stage_rows,
stage_rows_ordered, walk, fold_carry, k_chunk_aggregate, k_bidir_chain, k_fwd_chain, tag_word,
wait_published,
k_carry_combine, k_aux_swap; ncssd.hip:
state_tiles, load_c, out_tiles, k_ncssd_state, k_ncssd_reduce, k_ncssd_out). Extremes over lanes
and steps are taken analytically where an index is monotone in them (as every one is), so the
element-limit shape (65,536 workgroups) replays in well under a second.

Shapes: the five workloads, every shape of the GPU parity sweeps (with their forced chunk
lengths), the 2-3-...-33-chunk fold boundaries, and the element limit (2^31 - 1024 elements).
"""
import numpy as np
import pytest

from bidirectional_selective_scan_amd import binding
from bidirectional_selective_scan_amd.configs import WORKLOADS

N = 16
WAVE = 64
LDS_PER_CU = 160 * 1024
FOLD_MAX = 16


def xcd_remap(i, n):
    q, r = n >> 3, n & 7
    x, k = i & 7, i >> 3
    return np.where(x < r, x * (q + 1), r * (q + 1) + (x - r) * q) + k


def ceil_div(a, b):
    return -(-a // b)


def round_up(v, a):
    return ceil_div(v, a) * a


class Checks:
    """Collects (what, lo, hi, limit): every index of `what` must lie in [0, limit). lo, hi and
    limit may be arrays (per workgroup and wave); they are compared elementwise."""

    def __init__(self, case):
        self.case = case
        self.items = []

    def add(self, what, lo, hi, limit):
        lo, hi, limit = np.asarray(lo), np.asarray(hi), np.asarray(limit)
        bad = bool(np.any(lo < 0) or np.any(hi >= limit))
        self.items.append((what, int(lo.min()), int(hi.max()), int(limit.min()), bad))

    def verify(self):
        bad = [(w, lo, hi, lim) for w, lo, hi, lim, b in self.items if b]
        assert not bad, f"{self.case}: out of range (what, min index, max index, smallest limit): {bad[:5]}"
        return len(self.items)


def scan_plan(B, L, Di, io, seg, chunk, uni, ordered=False):
    info = binding.launch_info(B, L, Di, 16, seg, io, chunk_len=chunk, forward_only=uni)
    p = dict(info)
    p["ncb"] = ceil_div(Di, WAVE)
    p["subs"] = (min(p["ncb"], 4) if uni else (2 if p["ncb"] >= 2 else 1))
    p["K"], p["T"], p["Lp"], p["nseq"] = info["chunks"], info["chunk_len"], info["seq_tokens"], info["sequences"]
    p["wpc"] = ceil_div(p["ncb"], p["subs"])
    assert p["workgroups"] == p["nseq"] * p["K"] * p["wpc"], p
    assert p["K"] == ceil_div(p["Lp"], p["T"]) and p["T"] <= 256
    p["fold"] = 1 < p["K"] <= FOLD_MAX
    p["chain"] = p["fold"]                         # one kernel: k_bidir_chain / k_fwd_chain
    assert info["kernels"] == (1 if p["K"] == 1 or p["chain"] else 3), info
    ndir = 1 if uni else 2
    f = 4
    carry = ndir * p["nseq"] * p["K"] * N * Di * f if p["K"] > 1 else 0
    dsum = ndir * p["nseq"] * p["K"] * Di * f if p["K"] > 1 else 0
    park = p["workgroups"] * p["subs"] * p["T"] * WAVE * f if p["park_in_workspace"] else 0
    tags = ndir * p["nseq"] * p["K"] * p["ncb"] * 8 if p["chain"] else 0
    off_dsum = round_up(carry, 256)
    off_park = round_up(off_dsum + dsum, 256)
    off_tags = round_up(off_park + park, 256)
    ws = off_tags + tags if carry + dsum + park + tags > 0 else 0
    assert ws == info["workspace_bytes"], (ws, info)
    assert bool(p["park_in_workspace"]) == (not uni and p["T"] * WAVE * 4 > 20 * 1024)
    p.update(ndir=ndir, carry_floats=carry // f, dsum_floats=dsum // f, park_floats=park // f, tag_words=tags // 8,
             off_dsum=off_dsum, off_park=off_park, off_tags=off_tags, ws=ws)
    return p


def coords(p, uni, waves):
    """wg_coords for every (workgroup, wave): arrays over hardware ids bid (grid order) x waves."""
    grid = p["workgroups"]
    bid = np.arange(grid, dtype=np.int64)
    ncbw = p["wpc"]
    if p.get("chain"):
        # k_bidir_chain: hardware order, chunk fastest, then the channel-block group
        lid = bid
        chunk = lid % p["K"]
        rest = lid // p["K"]
        cbw = rest % ncbw
        seq = rest // ncbw
        key = (seq * ncbw + cbw) * p["K"] + chunk
        assert np.array_equal(np.sort(key), bid), "chain workgroups do not cover sequence x group x chunk once"
    else:
        lid = xcd_remap(bid, grid)
        assert np.array_equal(np.sort(lid), bid), "the XCD remap is not a permutation of the grid"
        cbw = lid % ncbw
        rest = lid // ncbw
        chunk = rest % p["K"]
        seq = rest // p["K"]
    wave = np.arange(waves, dtype=np.int64)
    c = {}
    c["lid"] = lid[:, None]
    c["seq"] = seq[:, None]
    c["chunk"] = chunk[:, None]
    c["dir"] = np.zeros_like(wave)[None, :] if uni else (wave & 1)[None, :]
    c["sub"] = wave[None, :] if uni else (wave >> 1)[None, :]
    c["slot"] = c["lid"] * p["subs"] + c["sub"]
    c["cb"] = cbw[:, None] * p["subs"] + c["sub"]
    c["t0"] = c["chunk"] * p["T"]
    c["t1"] = np.minimum(c["t0"] + p["T"], p["Lp"])
    c["len"] = c["t1"] - c["t0"]
    return c


def lane_dc(c, Di):
    """Smallest and largest channel dc = min(cb * 64 + lane, Di - 1) over the 64 lanes."""
    lo = np.minimum(c["cb"] * WAVE, Di - 1)
    hi = np.minimum(c["cb"] * WAVE + WAVE - 1, Di - 1)
    return lo, hi


def replay_scan(B, L, Di, io, seg=0, chunk=0, variant="plain", taps=4):
    uni = variant in ("fwd", "fwd_swap")
    ordered = variant == "ordered"
    conv = variant == "conv"
    swap = variant == "fwd_swap"
    p = scan_plan(B, L, Di, io, seg, chunk, uni, ordered)
    e = 4 if io == "f32" else 2
    kpw = 4 // e                      # values per 32-bit word
    S = B * L * Di                    # elements of x, dt, z, y
    rows_el = B * L * N               # elements of each B / C tensor
    ck = Checks(f"{variant} B={B} L={L} Di={Di} {io} seg={seg} chunk={chunk}")
    waves = p["subs"] * (1 if uni else 2)
    c = coords(p, uni, waves)
    Lp, T, K, nseq = p["Lp"], p["T"], p["K"], p["nseq"]
    ck.add("sequence of a workgroup", c["seq"], c["seq"], nseq)
    ck.add("chunk of a workgroup", c["chunk"], c["chunk"], K)
    ck.add("chunk length - 1", c["len"] - 1, c["len"] - 1, T)
    dlo, dhi = lane_dc(c, Di)
    ck.add("lane channel dc", dlo, dhi, Di)

    # -- LDS of each kernel
    regions = 2 if uni else 4
    lds_park = (not uni) and not p["park_in_workspace"]
    scan_lds = (regions * T * N + (T if ordered else 0) + (p["subs"] * T * WAVE if lds_park else 0)) * 4
    agg_lds = (p["ndir"] * T * N + (T if ordered else 0)) * 4
    ck.add("scan kernel LDS bytes", 0, scan_lds - 1, LDS_PER_CU)
    if K > 1 and not p["chain"]:
        ck.add("aggregate kernel LDS bytes", 0, agg_lds - 1, LDS_PER_CU)
    # staged rows: region r, local row < len, 16 values; order copy after the rows; the LDS park
    ck.add("LDS row staging (floats)", 0, (regions - 1) * T * N + c["len"] * N - 1, scan_lds // 4)
    if ordered:
        ck.add("LDS order copy (ints)", regions * T * N, regions * T * N + c["len"] - 1, scan_lds // 4)
    if lds_park:
        base = regions * T * N + (T if ordered else 0)
        ck.add("LDS park (floats)", base + c["sub"] * T * WAVE,
               base + c["sub"] * T * WAVE + (c["len"] - 1) * WAVE + WAVE - 1, scan_lds // 4)

    # -- row staging from global memory (32-bit words of the B / C tensors)
    words = rows_el // kpw
    if not ordered:
        off = (c["seq"] * Lp + c["t0"]) * N          # element offset of the chunk's first row
        wpd = c["len"] * N // kpw
        ck.add("stage_rows words", off // kpw, off // kpw + wpd - 1, words)
        assert np.all((off % kpw) == 0)
    else:
        srow = c["seq"] * Lp
        ck.add("order entries read", srow + c["t0"], srow + c["t0"] + c["len"] - 1, B * L)
        # a clamped token 0..Lp-1 of the sequence: its row's words
        ck.add("stage_rows_ordered words", srow * (N // kpw), (srow + Lp - 1) * (N // kpw) + N // kpw - 1, words)

    # -- parameters: A rows, D, dt_bias, convolution taps
    ck.add("A row elements", dlo * N, dhi * N + N - 1, Di * N)
    ck.add("D / dt_bias elements", dlo, dhi, Di)
    if conv:
        ck.add("conv taps", dlo * taps, dhi * taps + taps - 1, Di * taps)

    # -- the walk's buffer resources: base (elements) and range (bytes) inside the tensor, and
    # every offset vo + so + e within the range
    rbase = c["seq"] * Lp if ordered else c["seq"] * Lp + c["t0"]
    span = (Lp if ordered else c["len"]) * Di * e
    assert np.all(span < 2 ** 32)
    ck.add("x/dt/z/y buffer end (bytes)", rbase * Di * e, rbase * Di * e + span - 1, S * e)
    max_row = (Lp - 1) if ordered else (c["len"] - 1)
    ck.add("x/dt/z/y buffer offsets (bytes)", 0 * span, max_row * Di * e + dhi * e + e - 1, span)
    if p["park_in_workspace"]:
        pbase = c["slot"] * T * WAVE
        ck.add("park region (floats)", pbase, pbase + T * WAVE - 1, p["park_floats"])
        ck.add("park offsets (bytes)", 0 * pbase, (c["len"] - 1) * WAVE * 4 + (WAVE - 1) * 4 + 3, T * WAVE * 4)
        ck.add("park inside the workspace (bytes)", p["off_park"], p["off_park"] + p["park_floats"] * 4 - 1, p["ws"])
    if conv:
        # the window of the three tokens before a walk's first step, read only inside the sequence
        tok = np.stack([c["t0"] + j for j in range(-3, T + 3)], axis=-1)
        inside = (tok >= 0) & (tok < Lp)
        idx = np.where(inside, (c["seq"][..., None] * Lp + tok) * Di, 0)
        ck.add("conv window x elements", idx.min(), idx.max() + Di - 1, S)

    # -- chunk carries
    if K > 1:
        ck.add("delta sums inside the workspace", p["off_dsum"], p["off_dsum"] + p["dsum_floats"] * 4 - 1, p["ws"])
        ck.add("carries inside the workspace", 0, p["carry_floats"] * 4 - 1, p["off_dsum"] if p["dsum_floats"] else p["ws"])
        base = (c["dir"] * nseq + c["seq"]) * K
        # aggregate stores (every chunk but the last in scan order) and the carry read of the
        # non-fold scan: slot = base + chunk
        slot = base + c["chunk"]
        ck.add("carry slot", slot, slot, p["ndir"] * nseq * K)
        ck.add("carry elements", (slot * N) * Di + dlo, (slot * N + N - 1) * Di + dhi, p["carry_floats"])
        ck.add("delta-sum elements", slot * Di + dlo, slot * Di + dhi, p["dsum_floats"])
        if p["fold"]:
            # fold_carry: batches of 4 loads, clamped to chunks that have an aggregate
            # forward: k = min(j0 + j, K - 2) over j0 + j < round_up(cnt, 4); backward:
            # k = max(K - 1 - j0 - j, 1); no loads when cnt = 0
            cnt = np.where(c["dir"] == 0, c["chunk"], K - 1 - c["chunk"])
            jmax = round_up(np.maximum(cnt, 1), 4) - 1      # last j0 + j a batch issues
            fwd = c["dir"] == 0
            lo_k = np.where(fwd, 0, np.maximum(K - 1 - jmax, 1))
            hi_k = np.where(fwd, np.minimum(jmax, K - 2), K - 1)
            lo_k = np.where(cnt > 0, lo_k, np.where(fwd, 0, K - 1))
            hi_k = np.where(cnt > 0, hi_k, np.where(fwd, 0, K - 1))
            ck.add("fold slot", base + lo_k, base + hi_k, p["ndir"] * nseq * K)
            ck.add("fold carry elements", ((base + lo_k) * N) * Di + dlo, ((base + hi_k) * N + N - 1) * Di + dhi,
                   p["carry_floats"])
        if p["chain"]:
            # k_bidir_chain: a live wave (cb < ncb) publishes tag_word(dir, seq, chunk, cb) and
            # waits on the words of chunks 0..cnt-1 (forward) or K-cnt..K-1 (backward)
            live = c["cb"] < p["ncb"]
            cnt = np.where(c["dir"] == 0, c["chunk"], K - 1 - c["chunk"])
            fwd = c["dir"] == 0
            k_lo = np.where(cnt > 0, np.where(fwd, 0, K - cnt), c["chunk"])
            k_hi = np.where(cnt > 0, np.where(fwd, cnt - 1, K - 1), c["chunk"])
            word = lambda k: ((c["dir"] * nseq + c["seq"]) * K + k) * p["ncb"] + c["cb"]
            cb_live = np.where(live, c["cb"], 0)
            ck.add("live channel block", cb_live, cb_live, p["ncb"])
            ck.add("published tag word", np.where(live, word(c["chunk"]), 0), np.where(live, word(c["chunk"]), 0),
                   p["tag_words"])
            ck.add("awaited tag words", np.where(live, word(k_lo), 0), np.where(live, word(k_hi), 0), p["tag_words"])
            ck.add("lanes watching tag words", 0, np.max(cnt), WAVE)
            ck.add("tags inside the workspace (bytes)", p["off_tags"], p["off_tags"] + p["tag_words"] * 8 - 1, p["ws"])
        else:
            # k_carry_combine: grid (ncb * ndir * nseq, 4), 256 threads = 64 channels x 4 states
            gx = p["ncb"] * p["ndir"] * nseq
            assert gx < 2 ** 31
            bx = np.arange(gx, dtype=np.int64)
            zz = bx // p["ncb"]
            d_hi = np.minimum((bx % p["ncb"]) * WAVE + WAVE - 1, Di - 1)
            dirs = np.zeros_like(zz) if uni else zz & 1
            seqs = zz if uni else zz >> 1
            cbase = (dirs * nseq + seqs) * K
            ck.add("combine sequence", seqs, seqs, nseq)
            ck.add("combine carry elements", (cbase * N) * Di, ((cbase + K - 1) * N + N - 1) * Di + d_hi,
                   p["carry_floats"])
            ck.add("combine delta-sum elements", cbase * Di, (cbase + K - 1) * Di + d_hi, p["dsum_floats"])
    if swap:
        groups = ceil_div(Di, 256)
        gs = groups * nseq
        bidx = np.arange(gs, dtype=np.int64)
        sq = bidx // groups
        d_hi = np.minimum((bidx % groups) * 256 + 255, Di - 1)
        ck.add("swap elements", sq * Lp * Di, sq * Lp * Di + (Lp - 1) * Di + d_hi, S)
    return ck.verify()


def replay_ncssd(B, L, Di, Nst, io, seg=0, chunk=0):
    launch = binding.make_launch(B, L, Di, Nst, binding.VIMSCAN_BF16 if io == "bf16" else binding.VIMSCAN_F32,
                                 chunk)
    import ctypes
    plan = binding._Plan()
    binding._check(binding.load_library().vimscan_ncssd_plan(ctypes.byref(launch), int(seg), ctypes.byref(plan)))
    nseq, T, span, splits = plan.sequences, plan.seq_tokens, plan.chunk_len, plan.chunks
    ncb = ceil_div(Di, 64)
    groups = ceil_div(T, 128)
    ck = Checks(f"ncssd B={B} L={L} Di={Di} N={Nst} {io} seg={seg} chunk={chunk}")
    assert plan.workgroups == nseq * ncb * splits
    assert splits == ceil_div(T, span) and span % 16 == 0
    S, rows = B * L * Di, B * L
    vec = 4                                           # channels a lane reads per x load
    tiles = [(0, T)] if splits == 1 else [(s * span, min(s * span + span, T)) for s in range(splits)]
    for tb, te in tiles:
        if te <= tb:
            continue
        row_hi = (nseq - 1) * T + te - 1               # rows are clamped to te - 1
        ck.add("x elements", 0, row_hi * Di + Di - 4 + vec - 1, S)
        ck.add("m elements", 0, row_hi, rows)
        ck.add("B elements", 0, row_hi * Nst + Nst - 1, rows * Nst)
    ck.add("C elements", 0, ((nseq - 1) * T + T - 1) * Nst + Nst - 1, rows * Nst)
    # stores are guarded by t < ge and channel < Di; y rows are those of the sequence
    ck.add("y elements", 0, ((nseq - 1) * T + T - 1) * Di + Di - 1, S)
    if splits > 1:
        hsz = nseq * Nst * Di
        off_H = round_up(hsz * 4 * splits, 256)
        assert plan.workspace_bytes == off_H + hsz * 4
        ck.add("partial states (floats)", 0, ((nseq - 1) * splits + splits - 1) * Nst * Di + (Nst - 1) * Di + Di - 1,
               hsz * splits)
        ck.add("H (floats)", 0, (nseq - 1) * Nst * Di + (Nst - 1) * Di + Di - 1, hsz)
        ck.add("partials inside the workspace", 0, hsz * splits * 4 - 1, off_H)
        ck.add("H inside the workspace", off_H, off_H + hsz * 4 - 1, plan.workspace_bytes)
        ck.add("pass-2 token groups", 0, (groups - 1) * 128, T)
    return ck.verify()


PARITY_SHAPES = [  # tests/test_parity_gpu.py SHAPES
    (1, 1, 1, 0, 0), (2, 2, 3, 0, 0), (1, 3, 64, 0, 0), (3, 63, 65, 0, 0), (2, 64, 128, 0, 0), (2, 65, 130, 0, 0),
    (1, 200, 70, 0, 0), (2, 257, 64, 0, 0), (1, 300, 96, 0, 0), (1, 1025, 64, 0, 0), (2, 197, 64, 0, 16),
    (2, 197, 64, 0, 1), (2, 197, 100, 0, 64), (2, 400, 64, 0, 150), (1, 120, 64, 12, 0), (1, 120, 64, 12, 5),
    (2, 102, 33, 51, 0), (1, 60, 64, 1, 0), (3, 256, 64, 0, 0), (1, 512, 64, 0, 256),
    (1, 32768, 64, 0, 0), (2, 64, 4096, 0, 0), (1, 3, 8192, 0, 0), (1, 140000, 32, 2, 1),
]
VARIANTS = ("plain", "conv", "ordered", "fwd", "fwd_swap")
LIMIT = (1, (1 << 31) // 1024 - 1, 1024)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
def test_workloads(w, variant):
    assert replay_scan(w.batch, w.seqlen, w.d_inner, w.io_dtype, w.seg_len, 0, variant) > 10


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_parity_sweep_shapes(io, variant):
    for B, L, Di, seg, chunk in PARITY_SHAPES:
        replay_scan(B, L, Di, io, seg, chunk, variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_random_sweep_and_fold_boundaries(variant):
    rng = np.random.Generator(np.random.PCG64(7))
    for _ in range(40):
        B = int(rng.integers(1, 4))
        if rng.random() < 0.35:
            T = int(rng.integers(1, 80))
            L, seg = T * int(rng.integers(1, 7)), T
        else:
            L, seg = int(rng.integers(1, 600)), 0
        Di = int(rng.integers(1, 200))
        chunk = int(rng.integers(1, min(seg or L, 256) + 1)) if rng.random() < 0.4 else 0
        replay_scan(B, L, Di, ("f32", "bf16")[int(rng.integers(2))], seg, chunk, variant, int(rng.integers(1, 5)))
    for k in (2, 3, 4, 5, 6, 9, 13, 16, 17, 32, 33):    # 7-token chunks: fold batches and the combine
        replay_scan(2, 7 * k - 3, 96, "bf16", 0, 7, variant)


@pytest.mark.parametrize("variant", ("plain", "ordered", "fwd"))
def test_element_limit(variant):
    B, L, Di = LIMIT
    assert B * L * Di == 2 ** 31 - 1024
    replay_scan(B, L, Di, "bf16", 0, 0, variant)
    replay_scan(B, L, Di, "bf16", 0, 256, variant)


def test_ncssd_shapes():
    for w in WORKLOADS:
        replay_ncssd(w.batch, w.seqlen, w.d_inner - w.d_inner % 16 or 16, 16, w.io_dtype, w.seg_len)
    for Nst in (16, 32, 64):
        for io in ("f32", "bf16"):
            for B, L, Di, seg, chunk in [(2, 65, 32, 0, 0), (1, 1, 16, 0, 0), (1, 1025, 64, 0, 0), (2, 300, 48, 0, 64),
                                         (1, 120, 64, 12, 0), (3, 777, 80, 0, 16), (8, 1025, 768, 0, 0)]:
                replay_ncssd(B, L, Di, Nst, io, seg, chunk)
    B, L, Di = LIMIT
    replay_ncssd(B, L, Di, 16, "bf16")


def test_a_planted_index_error_is_caught(monkeypatch):
    """The replay itself: an index one past a buffer fails, and so do plans whose workspace regions
    are one element short of what the kernels address (a park, the carries, the delta sums, the
    one-pass kernel's tag words)."""
    ck = Checks("planted")
    ck.add("one past the end", 0, 10, 10)
    with pytest.raises(AssertionError):
        ck.verify()
    real = scan_plan
    for key, shape in (("park_floats", (2, 400, 64, "bf16", 0, 150)), ("carry_floats", (2, 1025, 64, "bf16", 0, 0)),
                       ("dsum_floats", (1, 40000, 64, "f32", 0, 0)), ("tag_words", (2, 400, 64, "bf16", 0, 50))):
        B, L, Di, io, seg, chunk = shape
        assert real(B, L, Di, io, seg, chunk, False)[key] > 0   # the region exists in this plan

        def short(*a, key=key, **kw):
            p = real(*a, **kw)
            p[key] -= 1
            return p
        monkeypatch.setattr(__import__(__name__), "scan_plan", short)
        with pytest.raises(AssertionError):
            replay_scan(*shape)
        monkeypatch.setattr(__import__(__name__), "scan_plan", real)
    replay_scan(8, 197, 128, "bf16")
