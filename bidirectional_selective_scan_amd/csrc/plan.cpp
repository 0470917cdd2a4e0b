// Host side of libvimscan (see plan.h): execution plans and argument checks of the scan and NC-SSD
// entry points, and the host-only entry points of include/vimscan.h (plans, workspace size, status
// text, version).

#include "plan.h"

#include <algorithm>
#include <cstring>

namespace vimscan_host {
namespace {



// Forward only: a single pass needs at least this many waves (channel blocks x sequences), and a
// chunked plan aims at this many.
constexpr int64_t kUniSinglePass = 1024;
constexpr int64_t kUniTarget = 3072;

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

// Modelled time of a chunked pass with chunks of T tokens. The busiest CU runs ceil(wgs / 256)
// workgroups, in rounds of at most resident_wgs; a round of a workgroups on a CU costs a / e(a)
// per token, e(a) being the issue efficiency of the VALU-bound token loop with a waves per SIMD
// (about 0.5 for a lone wave, 0.9 and more from two on, as measured on this kernel), and each
// chunk adds about 8 tokens' worth of fixed work (staging, carries).
double chunk_cost(const ScanPlan* p, int io_dtype, int64_t T) {
    static const double eff[4] = {0.5, 0.9, 0.92, 0.95};
    const int64_t K = (p->Lp + T - 1) / T;
    const int64_t wgs = p->nseq * K * ((p->ncb + p->subs - 1) / p->subs);
    const int64_t per_cu = (wgs + kCus - 1) / kCus;
    const int64_t r = resident_wgs(p, io_dtype, T);
    auto round_cost = [&](int64_t a) { return a / eff[a < 4 ? a - 1 : 3]; };
    const int64_t rounds = per_cu / r, rest = per_cu % r;
    return static_cast<double>(T + 8) * (rounds * round_cost(r) + (rest ? round_cost(rest) : 0.0));
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
    // Units of parallel work of a single pass: wave pairs (forward + backward), or single waves
    // forward only; a chunked plan aims at 1536 of them (3 waves per SIMD bidirectional).
    const int64_t lanes = p->nseq * p->ncb;
    const int64_t target = p->uni ? kUniTarget : 1536;
    // Four waves per workgroup (two channel blocks x two directions, or four channel blocks
    // forward only) when there are enough channel blocks: the hardware spreads a 4-wave
    // workgroup over the CU's four SIMDs, where 2-wave workgroups can leave some SIMDs with twice
    // the waves of others.
    if (p->uni) p->subs = p->ncb >= 4 ? 4 : p->ncb;
    else p->subs = p->ncb >= 2 ? 2 : 1;
    const int64_t wpc = (p->ncb + p->subs - 1) / p->subs;  // workgroups per sequence and chunk
    // A bidirectional single pass with at most one workgroup per CU gives each SIMD a lone wave
    // (Vim-Ti: 192 workgroups on 256 CUs): from 64 tokens on, chunking to the wave-pair target
    // pays for the aggregate pass (Vim-Ti: 4 chunks of 50, 72.9 -> 66.0 us per call).
    const bool single = (p->Lp <= kMaxChunk && lanes >= (p->uni ? kUniSinglePass : 256)) || p->Lp <= 32;
    const bool sparse = single && !p->uni && p->Lp >= 64 && p->nseq * wpc <= kCus;
    int64_t T;
    if (l->chunk_len > 0) {
        T = l->chunk_len;
    } else if (single && !sparse) {
        T = p->Lp;  // single pass: enough workgroups, or too short to be worth chunking
    } else {
        // Chunk for parallelism: first enough chunks for `target` waves, with at least 32 tokens
        // per chunk.
        int64_t K = (target + lanes - 1) / lanes;
        const int64_t kmin = (p->Lp + kMaxChunk - 1) / kMaxChunk;
        const int64_t kmax = (p->Lp + 31) / 32;
        if (K < kmin) K = kmin;
        if (K > kmax) K = kmax;
        // When that leaves only a few rounds of workgroups per CU, a round that is partly empty
        // costs as much as a full one: take instead the chunk count of least modelled time, up
        // to twice as many chunks and down to 16 tokens per chunk.
        if (!sparse && p->nseq * K * wpc <= 4 * kCus * resident_wgs(p, l->io_dtype, (p->Lp + K - 1) / K)) {
            const int64_t khi = std::min((p->Lp + 15) / 16, 2 * K);
            double best = -1.0;
            for (int64_t k = kmin; k <= khi; ++k) {
                const double c = chunk_cost(p, l->io_dtype, (p->Lp + k - 1) / k);
                if (best < 0.0 || c < best) best = c, K = k;
            }
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
    p->kernels = (p->K > 1 ? (p->fold ? 2 : 3) : 1) + (p->swap ? 1 : 0);
    p->park_global = !p->uni && p->T * kWave * static_cast<int64_t>(sizeof(float)) > kLdsParkMaxBytes;
    const size_t f = sizeof(float);
    const size_t ndir = p->uni ? 1 : 2;
    const size_t carry = p->K > 1 ? static_cast<size_t>(ndir * p->nseq * p->K) * kN * l->d_inner * f : 0;
    const size_t dsum = p->K > 1 ? static_cast<size_t>(ndir * p->nseq * p->K) * l->d_inner * f : 0;
    const size_t park = p->park_global ? static_cast<size_t>(p->wgs) * p->subs * p->T * kWave * f : 0;
    p->off_dsum = round_up(carry, 256);
    p->off_park = round_up(p->off_dsum + dsum, 256);
    p->ws = (carry + dsum + park) > 0 ? p->off_park + park : 0;
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
