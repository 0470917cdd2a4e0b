// Host side of libvimscan: the execution plans of the scan and NC-SSD calls and every argument check
// an entry point makes before its first HIP call. Plain C++ (no HIP, no device code), so it also
// builds on its own, with the address and undefined-behaviour sanitizers, for the host tests.
// The launchers (vimscan.hip, ncssd.hip) call make_scan_plan / check_scan_call and make_nc_plan /
// check_ncssd_call, then queue their kernels.
#ifndef VIMSCAN_PLAN_H
#define VIMSCAN_PLAN_H

#include <cstddef>
#include <cstdint>

#include "vimscan.h"

namespace vimscan_host {

// What the scan kernels are built for.
constexpr int kN = 16;              // state width
constexpr int kWave = 64;           // wavefront width on gfx950
constexpr int kMaxChunk = 256;      // tokens per chunk
constexpr int kMaxTaps = 4;         // taps of the directional convolution
// Plans of up to kFoldMaxChunks chunks run as one kernel: each workgroup computes its chunk's
// aggregates, hands them to the later chunks and folds the aggregates before its chunk itself.
constexpr int kFoldMaxChunks = 16;
// A park larger than this goes to global scratch: in LDS it would cap a CU at fewer than 8
// workgroups, and the VALU needs several waves per SIMD to issue at full rate.
constexpr int64_t kLdsParkMaxBytes = 20 * 1024;

// NC-SSD tiling.
constexpr int kNcTile = 16;          // tokens per MFMA tile
constexpr int kNcBlock = 64;         // channels per workgroup
constexpr int kNcWaves = 4;          // waves per workgroup
constexpr int kNcOutTokens = 128;    // tokens per pass-2 workgroup
constexpr int64_t kNcTargetWgs = 1024;

// p is a multiple of a (a power of two).
bool aligned(const void* p, uintptr_t a);

// Plan of a scan call (every bidirectional entry point and vimscan_fwd).
struct ScanPlan {
    int64_t nseq, Lp, T, K, ncb, subs, wgs;
    int kernels;
    bool park_global, uni, swap, fold;
    bool chain;                                // 2..kFoldMaxChunks chunks: one kernel
    size_t ws;                                 // total scratch bytes
    size_t off_dsum, off_park, off_tags;      // byte offsets of the regions after the carries
};

// Shape, dtype, seg_len, chunk_len and flag checks of a scan launch.
int check_scan_shape(const vimscan_launch* l, int64_t seg_len);
// Checks the launch and fills *p (all zero for an empty call).
int make_scan_plan(const vimscan_launch* l, int64_t seg_len, ScanPlan* p);
// The checks of a non-empty scan call after its plan: NULL pointers, the ordered walk's 32-bit
// range, alignment, y overlapping an input, and the workspace (or, with use_scratch, the static
// scratch limit of vimscan_bidir_fwd_noalloc). conv and order may be NULL.
int check_scan_call(const void* x, const void* dt, const void* z, const void* B_f, const void* C_f, const void* B_b,
                    const void* C_b, const float* A_f, const float* A_b, const float* D_f, const float* D_b,
                    const float* dt_bias_f, const float* dt_bias_b, const vimscan_conv* conv, const int32_t* order,
                    void* y, const vimscan_launch* launch, const ScanPlan& p, bool use_scratch);

// Plan of an NC-SSD call.
struct NcPlan {
    int64_t nseq, T, splits, span, ncb, groups, N;
    size_t off_H, ws;
};

int make_nc_plan(const vimscan_launch* l, int64_t seg_len, NcPlan* p);
// The checks of a non-empty NC-SSD call after its plan.
int check_ncssd_call(const void* x, const void* B, const void* C, const float* m, void* y,
                     const vimscan_launch* launch, const NcPlan& p);

}  // namespace vimscan_host

#endif  // VIMSCAN_PLAN_H
