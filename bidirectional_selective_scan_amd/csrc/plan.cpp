// Host side of libvimscan (see plan.h): execution plans and argument checks of the scan and NC-SSD
// entry points, and the host-only entry points of include/vimscan.h (plans, workspace size, status
// text, version).

#include "plan.h"

#include <algorithm>
#include <cstring>

namespace vimscan_host {
namespace {



// An MI355X: 256 compute units with 160 KB of LDS each.
constexpr int64_t kCus = 256;
constexpr int64_t kLdsPerCu = 160 * 1024;

// Workgroups of a chunked scan pass that one CU holds at once. The register budget of the scan
// kernels (150-161 VGPRs with either io dtype) allows 3 waves per SIMD, one wave of each
// workgroup on each SIMD; the bidirectional kernel's LDS (rows, the order and a park in LDS) can
// allow fewer.
int64_t resident_wgs(const ScanPlan* p, int io_dtype, int64_t T) {
    (void)io_dtype;
    int64_t r = 3;
    if (!p->uni) {
        const bool lds_park = T * kWave * static_cast<int64_t>(sizeof(float)) <= kLdsParkMaxBytes;
        const int64_t bytes = (4 * T * kN + T + (lds_park ? p->subs * T * kWave : 0)) * sizeof(float);
        if (kLdsPerCu / bytes < r) r = kLdsPerCu / bytes;
    }
    return r;
}

// Issue efficiency of the VALU-bound token loop with a waves per SIMD (a lone wave leaves about
// half the issue slots empty), and the cost in token steps of a round of a workgroups on a CU.
double round_cost(int64_t a) {
    static const double eff[5] = {0.531, 0.841, 0.95, 0.97, 0.98};
    return static_cast<double>(a) / eff[a < 5 ? a - 1 : 4];
}

// Cost of per_cu workgroups on the busiest CU, r at a time.
double rounds(int64_t per_cu, int64_t r) {
    const int64_t n = per_cu / r, rest = per_cu % r;
    return static_cast<double>(n) * round_cost(r) + (rest ? round_cost(rest) : 0.0);
}

// Chunk count of the forward-only scan: a single pass from 1024 waves (channel blocks x
// sequences) on, else first enough chunks for 3072 waves (at least 32 tokens per chunk) and,
// when that leaves only a few rounds of workgroups per CU, the count of least modelled scan time
// up to twice as many chunks and down to 16 tokens per chunk: T + 8 token steps per workgroup in
// rounds of resident_wgs, at an issue efficiency of 0.5, 0.9, 0.92, 0.95 with 1, 2, 3, 4 waves
// per SIMD. (Measured on the forward-only shapes of the forced-chunk sweep, this plan is within
// 4% of the best chunk count where the bidirectional model below misses by up to 13%.)
int64_t uni_chunks(const ScanPlan* p, int io_dtype) {
    const int64_t lanes = p->nseq * p->ncb;
    const int64_t kmin = (p->Lp + kMaxChunk - 1) / kMaxChunk;
    if (p->Lp <= kMaxChunk && lanes >= 1024) return 1;
    const int64_t wpc = (p->ncb + p->subs - 1) / p->subs;
    int64_t K = std::min(std::max((3072 + lanes - 1) / lanes, kmin), std::max(kmin, (p->Lp + 31) / 32));
    auto cost = [&](int64_t k) {
        static const double eff[4] = {0.5, 0.9, 0.92, 0.95};
        const int64_t T = (p->Lp + k - 1) / k;
        const int64_t per_cu = (p->nseq * k * wpc + kCus - 1) / kCus;
        const int64_t r = resident_wgs(p, io_dtype, T);
        auto rc = [&](int64_t a) { return static_cast<double>(a) / eff[a < 4 ? a - 1 : 3]; };
        return static_cast<double>(T + 8) * (static_cast<double>(per_cu / r) * rc(r) + (per_cu % r ? rc(per_cu % r) : 0.0));
    };
    if (p->nseq * K * wpc <= 4 * kCus * resident_wgs(p, io_dtype, (p->Lp + K - 1) / K)) {
        const int64_t khi = std::max(kmin, std::min((p->Lp + 15) / 16, 2 * K));
        double best = -1.0;
        for (int64_t k = kmin; k <= khi; ++k) {
            const double c = cost(k);
            if (best < 0.0 || c < best) best = c, K = k;
        }
    }
    return K;
}

// Modelled time of a whole call with chunks of about Lp / K tokens, in units of one token step of
// a round of workgroups (about 0.17 us on this chip). Terms, fitted to a sweep of forced chunk
// counts over ten bidirectional shapes of the Vim family (the forced-chunk sweep of bench.py;
// points within 1.6x of each shape's best):
//  * the scan: T token steps per workgroup, in rounds of resident_wgs;
//  * with 2..kFoldMaxChunks chunks, the one-pass kernel's own aggregate walk (no readout, walked
//    against the scan order) at 0.296 of a scan step per token plus 62.9 for its staging, stores
//    and hand-over, in the same rounds, and 2.4 per chunk of the sequence per round for the wait
//    on the other chunks and the fold of their aggregates (the fits gave 2.7-2.8, with the tiny
//    case's 6 and 9 chunks 4% apart; 2.4 picks the measured best chunk count of all ten shapes in
//    two sweeps);
//  * past kFoldMaxChunks, the separate aggregate pass: 0.139 of a scan step per token plus 109.6,
//    at up to 5 workgroups per CU; the combine kernel: 3.86 + 14.0 per 16 chunks; 32.2 for each of
//    the two kernels after the first (launch and drain).
double plan_cost(const ScanPlan* p, int io_dtype, int64_t K) {
    const int64_t T = (p->Lp + K - 1) / K;
    const int64_t wpc = (p->ncb + p->subs - 1) / p->subs;
    const int64_t per_cu = (p->nseq * K * wpc + kCus - 1) / kCus;
    const int64_t r = resident_wgs(p, io_dtype, T);
    const int64_t nr = (per_cu + r - 1) / r;
    const double rs = rounds(per_cu, r);
    const double t = static_cast<double>(T);
    double c = t * rs;
    if (K > 1 && K <= kFoldMaxChunks) {
        c += 0.296 * (t + 62.9) * rs + 2.4 * static_cast<double>(K * nr);
    } else if (K > kFoldMaxChunks) {
        c += 0.139 * (t + 109.6) * rounds(per_cu, std::min<int64_t>(5, kLdsPerCu / (T * kN * 8 + 1)));
        c += 3.86 + 14.0 * static_cast<double>((K + 15) / 16) + 2 * 32.2;
    }
    return c;
}

const char* const kStatusText[] = {
    "ok",
    "a required pointer is NULL",
    "bad shape: a size < 0, batch*seqlen*d_inner >= 2^31, d_inner >= 2^22, or d_state / d_inner not accepted by "
    "the entry point (16 for the scans; 16, 32 or 64 with d_inner % 16 == 0 for NC-SSD)",
    "bad seg_len: must be 0 or a positive divisor of seqlen",
    "bad io_dtype: must be VIMSCAN_F32 or VIMSCAN_BF16",
    "misaligned pointer",
    "y overlaps an input",
    "workspace missing or too small",
    "HIP kernel launch failed",
    "bad chunk_len: must be >= 0",
    "unknown flag bits",
    "bad convolution: k must be 1..4",
    "the call needs more scratch than the allocation-free entry point's static array holds (96 MiB)",
};

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && a0 < b0 + nb && b0 < a0 + na;
}


}  // namespace

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_scan_shape(const vimscan_launch* l, int64_t seg_len) {
    if (!l) return VIMSCAN_ERR_NULL;
    if (l->batch < 0 || l->seqlen < 0 || l->d_inner < 0 || l->d_state != kN) return VIMSCAN_ERR_SHAPE;
    // a chunk's rows (up to kMaxChunk tokens of d_inner fp32 values) must fit a 32-bit buffer range
    if (l->d_inner >= (int64_t(1) << 22)) return VIMSCAN_ERR_SHAPE;
    const int64_t lim = int64_t(1) << 31;
    if (l->batch > 0 && l->seqlen > 0 && l->d_inner > 0) {
        if (l->seqlen > lim / l->batch) return VIMSCAN_ERR_SHAPE;
        const int64_t bl = l->batch * l->seqlen;
        if (l->d_inner >= lim / bl + 1 || bl * l->d_inner >= lim) return VIMSCAN_ERR_SHAPE;
    }
    if (l->io_dtype != VIMSCAN_F32 && l->io_dtype != VIMSCAN_BF16) return VIMSCAN_ERR_DTYPE;
    if (seg_len < 0) return VIMSCAN_ERR_SEGLEN;
    if (seg_len > 0 && l->seqlen % seg_len != 0) return VIMSCAN_ERR_SEGLEN;
    if (l->chunk_len < 0) return VIMSCAN_ERR_CHUNK;
    if (l->flags & ~(VIMSCAN_FLAG_GENERAL_DECAY | VIMSCAN_FLAG_AUX_SWAP | VIMSCAN_FLAG_FORWARD_ONLY))
        return VIMSCAN_ERR_FLAGS;

    return VIMSCAN_OK;
}

int make_scan_plan(const vimscan_launch* l, int64_t seg_len, ScanPlan* p) {
    const int rc = check_scan_shape(l, seg_len);
    if (rc != VIMSCAN_OK) return rc;
    std::memset(p, 0, sizeof(*p));
    if (l->batch == 0 || l->seqlen == 0 || l->d_inner == 0) return VIMSCAN_OK;
    p->Lp = seg_len > 0 ? seg_len : l->seqlen;
    p->nseq = seg_len > 0 ? l->batch * (l->seqlen / seg_len) : l->batch;
    p->ncb = (l->d_inner + kWave - 1) / kWave;
    p->uni = (l->flags & VIMSCAN_FLAG_FORWARD_ONLY) != 0;
    p->swap = (l->flags & VIMSCAN_FLAG_AUX_SWAP) != 0;
    // Four waves per workgroup (two channel blocks x two directions, or four channel blocks
    // forward only) when there are enough channel blocks: the hardware spreads a 4-wave
    // workgroup over the CU's four SIMDs, where 2-wave workgroups can leave some SIMDs with twice
    // the waves of others.
    if (p->uni) p->subs = p->ncb >= 4 ? 4 : p->ncb;
    else p->subs = p->ncb >= 2 ? 2 : 1;
    // Bidirectional: the chunk count of least modelled time (plan_cost), from the fewest chunks of
    // at most kMaxChunk tokens (a single pass when the sequence fits one) to chunks of 8 tokens.
    // Forward only: uni_chunks. Sequences of up to 32 tokens are never chunked.
    int64_t T;
    if (l->chunk_len > 0) {
        T = l->chunk_len;
    } else if (p->Lp <= 32) {
        T = p->Lp;
    } else if (p->uni) {
        const int64_t K = uni_chunks(p, l->io_dtype);
        T = (p->Lp + K - 1) / K;
    } else {
        const int64_t kmin = (p->Lp + kMaxChunk - 1) / kMaxChunk;
        const int64_t kmax = std::max(kmin, (p->Lp + 7) / 8);
        int64_t K = kmin;
        double best = -1.0;
        for (int64_t k = kmin; k <= kmax; ++k) {
            const int64_t t = (p->Lp + k - 1) / k;
            if ((p->Lp + t - 1) / t != k) continue;  // k chunks of t tokens: fewer chunks cover the sequence
            const double c = plan_cost(p, l->io_dtype, k);
            if (best < 0.0 || c < best) best = c, K = k;
        }
        T = (p->Lp + K - 1) / K;
    }
    if (T > p->Lp) T = p->Lp;
    if (T > kMaxChunk) T = kMaxChunk;
    p->T = T;
    p->K = (p->Lp + T - 1) / T;
    p->wgs = p->nseq * p->K * ((p->ncb + p->subs - 1) / p->subs);
    // With few chunks every scan workgroup folds the aggregates before its chunk itself: no
    // combine kernel, and the carries are written once and read, not rewritten.
    p->fold = p->K > 1 && p->K <= kFoldMaxChunks;
    // Those plans run as one kernel: every workgroup computes its own chunk's aggregates,
    // publishes them and folds those of the chunks before it (k_bidir_chain, k_fwd_chain).
    p->chain = p->fold;
    p->kernels = (p->K > 1 && !p->chain ? 3 : 1) + (p->swap ? 1 : 0);
    p->park_global = !p->uni && p->T * kWave * static_cast<int64_t>(sizeof(float)) > kLdsParkMaxBytes;
    const size_t f = sizeof(float);
    const size_t ndir = p->uni ? 1 : 2;
    const size_t carry = p->K > 1 ? static_cast<size_t>(ndir * p->nseq * p->K) * kN * l->d_inner * f : 0;
    const size_t dsum = p->K > 1 ? static_cast<size_t>(ndir * p->nseq * p->K) * l->d_inner * f : 0;
    const size_t park = p->park_global ? static_cast<size_t>(p->wgs) * p->subs * p->T * kWave * f : 0;
    const size_t tags = p->chain ? static_cast<size_t>(ndir * p->nseq * p->K * p->ncb) * sizeof(uint64_t) : 0;
    p->off_dsum = round_up(carry, 256);
    p->off_park = round_up(p->off_dsum + dsum, 256);
    p->off_tags = round_up(p->off_park + park, 256);
    p->ws = (carry + dsum + park + tags) > 0 ? p->off_tags + tags : 0;
    return VIMSCAN_OK;
}


int check_scan_call(const void* x, const void* dt, const void* z, const void* B_f, const void* C_f, const void* B_b,
                    const void* C_b, const float* A_f, const float* A_b, const float* D_f, const float* D_b,
                    const float* dt_bias_f, const float* dt_bias_b, const vimscan_conv* conv, const int32_t* order,
                    void* y, const vimscan_launch* launch, const ScanPlan& p, bool use_scratch) {
    if (!x || !dt || !z || !B_f || !C_f || !B_b || !C_b || !A_f || !A_b || !D_f || !D_b || !dt_bias_f ||
        !dt_bias_b || !y)
        return VIMSCAN_ERR_NULL;
    if (conv && (!conv->w_f || !conv->bias_f || !conv->w_b || !conv->bias_b)) return VIMSCAN_ERR_NULL;
    const size_t e = launch->io_dtype == VIMSCAN_F32 ? 4 : 2;
    // in a given order a walk's buffers span a whole sequence, addressed with 32-bit offsets
    if (order && static_cast<uint64_t>(p.Lp) * static_cast<uint64_t>(launch->d_inner) * e >= (uint64_t(1) << 32))
        return VIMSCAN_ERR_SHAPE;
    const void* io[] = {x, dt, z, y};
    for (const void* q : io)
        if (!aligned(q, e)) return VIMSCAN_ERR_ALIGN;
    const void* w4[] = {B_f, C_f, B_b, C_b, A_f, A_b, D_f, D_b, dt_bias_f, dt_bias_b};
    for (const void* q : w4)
        if (!aligned(q, 4)) return VIMSCAN_ERR_ALIGN;
    const size_t S = static_cast<size_t>(launch->batch) * launch->seqlen * launch->d_inner;
    const size_t nbc = static_cast<size_t>(launch->batch) * launch->seqlen * kN;
    const size_t na = static_cast<size_t>(launch->d_inner) * kN * 4, nd = static_cast<size_t>(launch->d_inner) * 4;
    const struct {
        const void* p;
        size_t n;
    } ins[] = {{x, S * e},     {dt, S * e},  {z, S * e},  {B_f, nbc * e}, {C_f, nbc * e}, {B_b, nbc * e},
               {C_b, nbc * e}, {A_f, na},    {A_b, na},   {D_f, nd},      {D_b, nd},      {dt_bias_f, nd},
               {dt_bias_b, nd}};
    for (const auto& in : ins)
        if (overlaps(y, S * e, in.p, in.n)) return VIMSCAN_ERR_ALIAS;
    const size_t nw = conv ? static_cast<size_t>(launch->d_inner) * static_cast<size_t>(conv->k) * 4 : 0;
    const size_t nord = order ? static_cast<size_t>(launch->batch) * launch->seqlen * 4 : 0;
    const struct {
        const void* p;
        size_t n;
    } cins[] = {{conv ? conv->w_f : nullptr, nw},
                {conv ? conv->bias_f : nullptr, nw ? nd : 0},
                {conv ? conv->w_b : nullptr, nw},
                {conv ? conv->bias_b : nullptr, nw ? nd : 0},
                {order, nord}};
    for (const auto& in : cins) {
        if (in.n && !aligned(in.p, 4)) return VIMSCAN_ERR_ALIGN;
        if (overlaps(y, S * e, in.p, in.n)) return VIMSCAN_ERR_ALIAS;
    }
    if (use_scratch && p.ws > VIMSCAN_NOALLOC_SCRATCH_BYTES) return VIMSCAN_ERR_SCRATCH;
    if (p.ws > 0 && !use_scratch) {
        if (!launch->workspace || launch->workspace_bytes < p.ws) return VIMSCAN_ERR_WORKSPACE;
        if (!aligned(launch->workspace, 16)) return VIMSCAN_ERR_ALIGN;
        if (overlaps(y, S * e, launch->workspace, p.ws)) return VIMSCAN_ERR_ALIAS;
        for (const auto& in : ins)
            if (overlaps(launch->workspace, p.ws, in.p, in.n)) return VIMSCAN_ERR_ALIAS;
        for (const auto& in : cins)
            if (overlaps(launch->workspace, p.ws, in.p, in.n)) return VIMSCAN_ERR_ALIAS;
    }

    return VIMSCAN_OK;
}


int make_nc_plan(const vimscan_launch* l, int64_t seg_len, NcPlan* p) {
    if (!l) return VIMSCAN_ERR_NULL;
    if (l->batch < 0 || l->seqlen < 0 || l->d_inner < 0) return VIMSCAN_ERR_SHAPE;
    if (l->d_state != 16 && l->d_state != 32 && l->d_state != 64) return VIMSCAN_ERR_SHAPE;
    if (l->d_inner % 16 != 0 || l->d_inner >= (int64_t(1) << 22)) return VIMSCAN_ERR_SHAPE;
    const int64_t lim = int64_t(1) << 31;
    if (l->batch > 0 && l->seqlen > 0 && l->d_inner > 0) {
        if (l->seqlen > lim / l->batch) return VIMSCAN_ERR_SHAPE;
        const int64_t bl = l->batch * l->seqlen;
        if (l->d_inner >= lim / bl + 1 || bl * l->d_inner >= lim) return VIMSCAN_ERR_SHAPE;
    }
    if (l->io_dtype != VIMSCAN_F32 && l->io_dtype != VIMSCAN_BF16) return VIMSCAN_ERR_DTYPE;
    if (seg_len < 0 || (seg_len > 0 && l->seqlen % seg_len != 0)) return VIMSCAN_ERR_SEGLEN;
    if (l->chunk_len < 0) return VIMSCAN_ERR_CHUNK;
    if (l->flags != 0) return VIMSCAN_ERR_FLAGS;
    std::memset(p, 0, sizeof(*p));
    p->N = l->d_state;
    if (l->batch == 0 || l->seqlen == 0 || l->d_inner == 0) return VIMSCAN_OK;
    p->T = seg_len > 0 ? seg_len : l->seqlen;
    p->nseq = l->batch * (l->seqlen / p->T);
    p->ncb = (l->d_inner + kNcBlock - 1) / kNcBlock;
    const int64_t quantum = kNcTile * kNcWaves;  // one tile per wave
    int64_t span;
    if (l->chunk_len > 0) {
        span = (l->chunk_len + kNcTile - 1) / kNcTile * kNcTile;
    } else {
        // Split long sequences until the pass has about kNcTargetWgs workgroups, keeping at least
        // two tiles per wave.
        const int64_t wgs = p->nseq * p->ncb;
        int64_t k = wgs >= kNcTargetWgs ? 1 : (kNcTargetWgs + wgs - 1) / wgs;
        const int64_t kmax = (p->T + 2 * quantum - 1) / (2 * quantum);
        if (k > kmax) k = kmax;
        if (k < 1) k = 1;
        span = (p->T + k - 1) / k;
        span = (span + quantum - 1) / quantum * quantum;
    }
    if (span >= p->T) span = (p->T + kNcTile - 1) / kNcTile * kNcTile;
    p->span = span;
    p->splits = (p->T + span - 1) / span;
    p->groups = (p->T + kNcOutTokens - 1) / kNcOutTokens;
    if (p->splits > 1) {  // split partial states, then H
        const size_t hsz = static_cast<size_t>(p->nseq) * p->N * l->d_inner * sizeof(float);
        p->off_H = (hsz * static_cast<size_t>(p->splits) + 255) / 256 * 256;
        p->ws = p->off_H + hsz;
    }
    return VIMSCAN_OK;
}


int check_ncssd_call(const void* x, const void* B, const void* C, const float* m, void* y,
                     const vimscan_launch* launch, const NcPlan& p) {
    if (!x || !B || !C || !m || !y) return VIMSCAN_ERR_NULL;
    const bool bf = launch->io_dtype == VIMSCAN_BF16;
    const size_t e = bf ? 2 : 4;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(B, e) || !aligned(C, bf ? 8 : 16) || !aligned(m, 4))
        return VIMSCAN_ERR_ALIGN;
    const size_t tokens = static_cast<size_t>(launch->batch) * launch->seqlen;
    const size_t ny = tokens * launch->d_inner * e;
    const struct {
        const void* p;
        size_t n;
    } ins[] = {{x, ny}, {B, tokens * p.N * e}, {C, tokens * p.N * e}, {m, tokens * 4}};
    for (const auto& in : ins)
        if (overlaps(y, ny, in.p, in.n)) return VIMSCAN_ERR_ALIAS;
    if (p.ws > 0) {
        if (!launch->workspace || launch->workspace_bytes < p.ws) return VIMSCAN_ERR_WORKSPACE;
        if (!aligned(launch->workspace, 16)) return VIMSCAN_ERR_ALIGN;
        if (overlaps(y, ny, launch->workspace, p.ws)) return VIMSCAN_ERR_ALIAS;
        for (const auto& in : ins)
            if (overlaps(launch->workspace, p.ws, in.p, in.n)) return VIMSCAN_ERR_ALIAS;
    }

    return VIMSCAN_OK;
}

}  // namespace vimscan_host

using namespace vimscan_host;

extern "C" {

int vimscan_plan_launch(const vimscan_launch* launch, int64_t seg_len, vimscan_plan* plan) {
    if (!plan) return VIMSCAN_ERR_NULL;
    ScanPlan p;
    const int rc = make_scan_plan(launch, seg_len, &p);
    if (rc != VIMSCAN_OK) return rc;
    plan->sequences = p.nseq;
    plan->seq_tokens = p.Lp;
    plan->chunk_len = p.T;
    plan->chunks = p.K;
    plan->workgroups = p.wgs;
    plan->kernels = p.kernels;
    plan->park_in_workspace = p.park_global ? 1 : 0;
    plan->workspace_bytes = p.ws;
    return VIMSCAN_OK;
}

int vimscan_workspace_bytes(const vimscan_launch* launch, int64_t seg_len, size_t* bytes) {
    if (!bytes) return VIMSCAN_ERR_NULL;
    ScanPlan p;
    const int rc = make_scan_plan(launch, seg_len, &p);
    if (rc != VIMSCAN_OK) return rc;
    *bytes = p.ws;
    return VIMSCAN_OK;
}

const char* vimscan_status_string(int status) {
    const int i = -status;
    if (i < 0 || i >= static_cast<int>(sizeof(kStatusText) / sizeof(kStatusText[0]))) return "unknown status";
    return kStatusText[i];
}

const char* vimscan_version(void) { return "vimscan 0.3.0 gfx950"; }

int vimscan_ncssd_plan(const vimscan_launch* launch, int64_t seg_len, vimscan_plan* plan) {
    if (!plan) return VIMSCAN_ERR_NULL;
    NcPlan p;
    const int rc = make_nc_plan(launch, seg_len, &p);
    if (rc != VIMSCAN_OK) return rc;
    plan->sequences = p.nseq;
    plan->seq_tokens = p.T;
    plan->chunk_len = p.span;
    plan->chunks = p.splits;
    plan->workgroups = p.nseq * p.ncb * p.splits;
    plan->kernels = p.nseq == 0 ? 0 : (p.splits > 1 ? 3 : 1);
    plan->park_in_workspace = 0;
    plan->workspace_bytes = p.ws;
    return VIMSCAN_OK;
}

}  // extern "C"
