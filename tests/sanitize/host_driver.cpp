// Drives the host side of libvimscan (csrc/plan.cpp: plans and argument checks of every entry
// point, the host-only entry points of include/vimscan.h) through many shapes, including sizes at
// and past every limit, and every argument error, so that a build with the address and
// undefined-behaviour sanitizers checks that code for out-of-bounds accesses, signed overflow and
// other undefined behaviour. No HIP call is involved: plan.cpp is plain C++.
// Exit status 0 and "host driver ok" on success; a sanitizer report aborts the program.
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>

#include "../../bidirectional_selective_scan_amd/csrc/plan.h"
#include "vimscan.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int64_t a, int64_t b, int64_t c) {
    if (!ok) {
        ++failures;
        std::printf("FAIL %s (%" PRId64 ", %" PRId64 ", %" PRId64 ")\n", what, a, b, c);
    }
}

vimscan_launch launch(int64_t B, int64_t L, int64_t D, int64_t N, int io, int flags, int64_t chunk) {
    vimscan_launch l;
    std::memset(&l, 0, sizeof(l));
    l.batch = B;
    l.seqlen = L;
    l.d_inner = D;
    l.d_state = N;
    l.io_dtype = io;
    l.flags = flags;
    l.chunk_len = chunk;
    return l;
}

// A plan must be self-consistent whenever the call is accepted.
void check_scan_plan(const vimscan_launch& l, int64_t seg) {
    vimscan_plan p;
    const int rc = vimscan_plan_launch(&l, seg, &p);
    size_t ws = 0;
    const int rc2 = vimscan_workspace_bytes(&l, seg, &ws);
    expect(rc == rc2, "plan and workspace_bytes agree on the status", l.batch, l.seqlen, l.d_inner);
    if (rc != VIMSCAN_OK) {
        expect(rc < 0 && std::strcmp(vimscan_status_string(rc), "unknown status") != 0, "documented status", rc,
               l.batch, l.seqlen);
        return;
    }
    expect(ws == p.workspace_bytes, "workspace bytes", static_cast<int64_t>(ws), l.batch, l.seqlen);
    if (l.batch == 0 || l.seqlen == 0 || l.d_inner == 0) {
        expect(p.chunks == 0 && p.workgroups == 0 && ws == 0, "empty plan", l.batch, l.seqlen, l.d_inner);
        return;
    }
    const int64_t T = seg > 0 ? seg : l.seqlen;
    expect(p.seq_tokens == T && p.sequences * T == l.batch * l.seqlen, "sequences", p.sequences, T, l.batch);
    expect(p.chunk_len >= 1 && p.chunk_len <= vimscan_host::kMaxChunk && p.chunk_len <= T, "chunk length",
           p.chunk_len, T, l.chunk_len);
    expect(p.chunks == (T + p.chunk_len - 1) / p.chunk_len, "chunk count", p.chunks, T, p.chunk_len);
    expect(p.workgroups > 0 && p.workgroups < (int64_t(1) << 31), "grid size", p.workgroups, T, l.d_inner);
    expect(p.kernels >= 1 && p.kernels <= 4, "kernel count", p.kernels, p.chunks, 0);
}

void check_nc_plan(const vimscan_launch& l, int64_t seg) {
    vimscan_plan p;
    const int rc = vimscan_ncssd_plan(&l, seg, &p);
    if (rc != VIMSCAN_OK) {
        expect(rc < 0, "ncssd status", rc, l.batch, l.seqlen);
        return;
    }
    if (l.batch == 0 || l.seqlen == 0 || l.d_inner == 0) return;
    expect(p.chunk_len % 16 == 0 && p.chunk_len >= 16, "ncssd span", p.chunk_len, l.seqlen, 0);
    expect(p.chunks * p.chunk_len >= p.seq_tokens, "ncssd splits cover the sequence", p.chunks, p.chunk_len,
           p.seq_tokens);
}

}  // namespace

int main() {
    const int64_t big = std::numeric_limits<int64_t>::max();
    const int64_t Bs[] = {0, 1, 2, 3, 8, 64, 128, 256, 70000, int64_t(1) << 20, int64_t(1) << 31, big, -1};
    const int64_t Ls[] = {0, 1, 2, 13, 31, 32, 33, 51, 63, 64, 65, 80, 81, 197, 256, 257, 1025, 13056,
                          32768, (int64_t(1) << 21) - 1, int64_t(1) << 31, big, -5};
    const int64_t Ds[] = {0, 1, 16, 32, 63, 64, 65, 130, 384, 768, 1024, 1536, 4096, 8192,
                          (int64_t(1) << 22) - 1, int64_t(1) << 22, big, -1};
    int calls = 0;
    for (int64_t B : Bs)
        for (int64_t L : Ls)
            for (int64_t D : Ds)
                for (int io = 0; io < 3; io += 1)
                    for (int flags : {0, 1, 2, 4, 6, 8}) {
                        for (int64_t chunk : {int64_t(0), int64_t(1), int64_t(17), int64_t(256), int64_t(4000),
                                              int64_t(-1)}) {
                            const vimscan_launch l = launch(B, L, D, 16, io, flags, chunk);
                            check_scan_plan(l, 0);
                            if (L > 0 && L % 51 == 0) check_scan_plan(l, 51);
                            if (L > 1) check_scan_plan(l, 1);
                            check_scan_plan(l, -3);
                            calls += 4;
                        }
                        for (int64_t N : {8, 16, 32, 64}) {
                            const vimscan_launch l = launch(B, L, D, N, io, flags == 8 ? 0 : flags, 0);
                            check_nc_plan(l, 0);
                            ++calls;
                        }
                    }
    // random shapes inside the limits, with seg_len divisors and forced chunks
    std::mt19937_64 rng(12345);
    for (int i = 0; i < 200000; ++i) {
        const int64_t B = 1 + static_cast<int64_t>(rng() % 300);
        const int64_t T = 1 + static_cast<int64_t>(rng() % 3000);
        const int64_t m = 1 + static_cast<int64_t>(rng() % 8);
        const int64_t D = 1 + static_cast<int64_t>(rng() % 5000);
        const int io = static_cast<int>(rng() % 2);
        const int64_t chunk = (rng() % 3 == 0) ? static_cast<int64_t>(rng() % 300) : 0;
        const int flags = static_cast<int>(rng() % 8);
        vimscan_launch l = launch(B, T * m, D, 16, io, flags, chunk);
        check_scan_plan(l, (rng() % 2) ? T : 0);
        l.d_state = 16 << (rng() % 3);
        l.d_inner = 16 * (1 + static_cast<int64_t>(rng() % 300));
        l.flags = 0;
        check_nc_plan(l, (rng() % 2) ? T : 0);
        calls += 2;
    }
    // the argument checks of a non-empty call: NULL, alignment, aliasing, workspace, scratch limit
    {
        const vimscan_launch l = launch(2, 300, 96, 16, VIMSCAN_BF16, 0, 0);
        vimscan_host::ScanPlan p;
        expect(vimscan_host::make_scan_plan(&l, 0, &p) == VIMSCAN_OK, "plan", 0, 0, 0);
        uintptr_t base = 0x100000000ull;
        const void* q[13];
        for (int i = 0; i < 13; ++i) q[i] = reinterpret_cast<const void*>(base * (i + 1));
        void* y = reinterpret_cast<void*>(base * 20);
        auto call = [&](const void* const* a, void* yy, const vimscan_launch& ll, const vimscan_conv* conv,
                        const int32_t* order, bool scratch) {
            return vimscan_host::check_scan_call(a[0], a[1], a[2], a[3], a[4], a[5], a[6],
                                                 static_cast<const float*>(a[7]), static_cast<const float*>(a[8]),
                                                 static_cast<const float*>(a[9]), static_cast<const float*>(a[10]),
                                                 static_cast<const float*>(a[11]), static_cast<const float*>(a[12]),
                                                 conv, order, yy, &ll, p, scratch);
        };
        expect(call(q, y, l, nullptr, nullptr, false) == VIMSCAN_ERR_WORKSPACE, "workspace needed", 0, 0, 0);
        expect(call(q, y, l, nullptr, nullptr, true) == VIMSCAN_OK, "scratch fits", 0, 0, 0);
        vimscan_launch lw = l;
        lw.workspace = reinterpret_cast<void*>(base * 30);
        lw.workspace_bytes = p.ws;
        expect(call(q, y, lw, nullptr, nullptr, false) == VIMSCAN_OK, "valid call", 0, 0, 0);
        lw.workspace_bytes = p.ws - 1;
        expect(call(q, y, lw, nullptr, nullptr, false) == VIMSCAN_ERR_WORKSPACE, "short workspace", 0, 0, 0);
        lw.workspace_bytes = p.ws;
        lw.workspace = const_cast<void*>(q[3]);
        expect(call(q, y, lw, nullptr, nullptr, false) == VIMSCAN_ERR_ALIAS, "workspace over B_f", 0, 0, 0);
        for (int i = 0; i < 13; ++i) {
            const void* bad[13];
            std::memcpy(bad, q, sizeof(q));
            bad[i] = nullptr;
            expect(call(bad, y, l, nullptr, nullptr, true) == VIMSCAN_ERR_NULL, "null input", i, 0, 0);
            std::memcpy(bad, q, sizeof(q));
            bad[i] = reinterpret_cast<const char*>(q[i]) + 1;
            expect(call(bad, y, l, nullptr, nullptr, true) == VIMSCAN_ERR_ALIGN, "misaligned input", i, 0, 0);
            expect(call(q, const_cast<void*>(q[i]), l, nullptr, nullptr, true) == VIMSCAN_ERR_ALIAS, "y over input",
                   i, 0, 0);
        }
        const float* w = reinterpret_cast<const float*>(base * 40);
        vimscan_conv conv = {w, w + 1024, w + 2048, w + 4096, 4};
        expect(call(q, y, l, &conv, nullptr, true) == VIMSCAN_OK, "conv call", 0, 0, 0);
        conv.bias_b = nullptr;
        expect(call(q, y, l, &conv, nullptr, true) == VIMSCAN_ERR_NULL, "conv null", 0, 0, 0);
        const int32_t* ord = reinterpret_cast<const int32_t*>(base * 50);
        expect(call(q, y, l, nullptr, ord, true) == VIMSCAN_OK, "order call", 0, 0, 0);
        expect(call(q, y, l, nullptr, ord + 1, true) == VIMSCAN_OK, "order 4-byte aligned", 0, 0, 0);
        expect(call(q, y, l, nullptr, reinterpret_cast<const int32_t*>(reinterpret_cast<uintptr_t>(ord) + 2), true) ==
                   VIMSCAN_ERR_ALIGN,
               "order misaligned", 0, 0, 0);
        // a plan larger than the static scratch
        const vimscan_launch lb = launch(256, 197, 768, 16, VIMSCAN_BF16, 0, 0);
        vimscan_host::ScanPlan pb;
        expect(vimscan_host::make_scan_plan(&lb, 0, &pb) == VIMSCAN_OK && pb.ws > VIMSCAN_NOALLOC_SCRATCH_BYTES,
               "big plan", 0, 0, 0);
        expect(vimscan_host::check_scan_call(q[0], q[1], q[2], q[3], q[4], q[5], q[6],
                                             static_cast<const float*>(q[7]), static_cast<const float*>(q[8]),
                                             static_cast<const float*>(q[9]), static_cast<const float*>(q[10]),
                                             static_cast<const float*>(q[11]), static_cast<const float*>(q[12]),
                                             nullptr, nullptr, y, &lb, pb, true) == VIMSCAN_ERR_SCRATCH,
               "scratch limit", 0, 0, 0);
        // NC-SSD
        const vimscan_launch ln = launch(4, 1025, 64, 32, VIMSCAN_BF16, 0, 0);
        vimscan_host::NcPlan np;
        expect(vimscan_host::make_nc_plan(&ln, 0, &np) == VIMSCAN_OK && np.splits > 1, "ncssd split plan", 0, 0, 0);
        const float* m = reinterpret_cast<const float*>(base * 60);
        expect(vimscan_host::check_ncssd_call(q[0], q[1], q[2], m, y, &ln, np) == VIMSCAN_ERR_WORKSPACE,
               "ncssd workspace", 0, 0, 0);
        vimscan_launch lnw = ln;
        lnw.workspace = reinterpret_cast<void*>(base * 70);
        lnw.workspace_bytes = np.ws;
        expect(vimscan_host::check_ncssd_call(q[0], q[1], q[2], m, y, &lnw, np) == VIMSCAN_OK, "ncssd call", 0, 0, 0);
        expect(vimscan_host::check_ncssd_call(q[0], q[1], q[2], m, const_cast<void*>(q[1]), &lnw, np) ==
                   VIMSCAN_ERR_ALIAS,
               "ncssd alias", 0, 0, 0);
        expect(vimscan_host::check_ncssd_call(reinterpret_cast<const char*>(q[0]) + 8, q[1], q[2], m, y, &lnw, np) ==
                   VIMSCAN_ERR_ALIGN,
               "ncssd align", 0, 0, 0);
    }
    for (int s = -20; s <= 5; ++s) expect(vimscan_status_string(s) != nullptr, "status text", s, 0, 0);
    expect(std::strstr(vimscan_version(), "gfx950") != nullptr, "version", 0, 0, 0);
    std::printf("host driver %s: %d plan calls\n", failures ? "FAILED" : "ok", calls);
    return failures ? 1 : 0;
}
