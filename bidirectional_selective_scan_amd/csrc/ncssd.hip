// NC-SSD, the non-causal global-state form of state-space duality, for AMD MI355X (gfx950): HIP
// kernels and the vimscan_ncssd_fwd / vimscan_ncssd_plan entry points of include/vimscan.h.
//
// What is computed (VSSD page, sections 4.2.3 to 4.2.5): per sequence of T tokens, with token
// weights m_j (the reciprocal of the token's scalar transition),
//     H = B^T (X . m)   [N x Di]   one hidden state shared by every token of the sequence
//     Y = C H           [T x Di]   every token reads it out with its own C row
// where X . m scales token j's row of X by m_j. Both are dense contractions (the first reduces
// over the tokens into N states, the second over the N states), so they run on the matrix cores;
// with N = 16 they move 16 flops per byte, far below the matrix cores' ridge point, so HBM bounds
// the call and the design aims at reading x once and writing y once.
//
// Execution design (gfx950, wave64, MFMA 16x16 tiles):
//  * A workgroup owns one sequence and 64 channels (k_ncssd_fused): its four waves take the
//    sequence's 16-token tiles round-robin for the state, add their partial states through LDS
//    in wave order, and read the state out for the same tiles: x is read once, y written
//    once, H never leaves the chip. Long sequences with too few workgroups for the chip are
//    split instead: pass 1 (k_ncssd_state) stores one partial state per token range, a small
//    kernel (k_ncssd_reduce) adds them in range order into H in the workspace, and pass 2
//    (k_ncssd_out) reads it out for groups of kOutTokens tokens. Results never depend on timing.
//  * The state contraction of a wave, per 16-token tile: H += B'^T X with B' = B . m as the MFMA
//    A operand (rows = states, K = tokens) and X as the B operand (K = tokens, columns =
//    channels). Each lane reads its four consecutive channels of four consecutive tokens as
//    plain 8-byte (bf16) or 16-byte (fp32) row loads, so X needs no transposition through LDS:
//    the four MFMA column sets of a wave are the channels d0 + 4c + q, q = 0..3, and the lane
//    regroups its loads into one operand per q.
//  * The readout computes Y^T = H^T C^T: rows = channels, K = states, columns = 16 tokens.
//    MFMA q's row m is channel d0 + 4 m + q, the column mapping of the state contraction, so a
//    lane's state accumulators are already its A operand (the four waves' partial states are
//    added lane by lane through LDS), and the four accumulators a lane ends with hold 16
//    consecutive channels of one token; a per-wave LDS tile regroups them so every store
//    instruction writes whole rows. The C rows of a wave's first readout tiles are loaded
//    before the state pass.
//  * bf16 io: X and C are exact bf16 MFMA operands. B . m and H are fp32 values; each is split
//    into a bf16 high part and a bf16 remainder and both are multiplied (two MFMAs), so the
//    contraction keeps about 16 significant bits on those operands and accumulates in fp32.
//    fp32 io uses the fp32 MFMA (16x16x4) directly.
//  * Sequences are split only when sequences x channel blocks is below about a thousand
//    workgroups, so the chip has several thousand waves either way.
//  * Every load is unconditional at a row clamped into range (a token past a range is zeroed by a
//    select where it would enter a sum), so a tile's loads are all in flight together; workgroup
//    ids are remapped so the channel blocks of one sequence share an XCD's L2 (B, C and m are
//    fetched from memory once).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <type_traits>

#include "plan.h"
#include "vimscan.h"

namespace {

using vimscan_host::NcPlan;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTile = vimscan_host::kNcTile;          // tokens per MFMA tile
constexpr int kBlock = vimscan_host::kNcBlock;        // channels per workgroup
constexpr int kWaves = vimscan_host::kNcWaves;        // waves per workgroup
constexpr int kOutTokens = vimscan_host::kNcOutTokens;  // tokens per pass-2 workgroup
constexpr int kStageRow = 36;   // words per token row of a wave's bf16 output tile in LDS (32 + 4 pad)
constexpr int kStageRowF = 68;  // the same for fp32 (64 + 4 pad)
template <typename IO> constexpr int kStageWords = kTile * (sizeof(IO) == 2 ? kStageRow : kStageRowF);  // per wave

struct NcArgs {
    const void* x;   // [nseq * T][Di]
    const void* B;   // [nseq * T][N]
    const void* C;   // [nseq * T][N]
    const float* m;  // [nseq * T]
    void* y;         // [nseq * T][Di]
    float* part;     // pass 1 output: [nseq][splits][N][Di] (the state itself when splits == 1)
    float* H;        // [nseq][N][Di]
    int T;           // tokens per sequence
    int Di;
    int splits;      // token ranges per sequence in pass 1
    int span;        // tokens per range (a multiple of kTile)
    int ncb;         // channel blocks of 64
    int groups;      // token groups of kOutTokens per sequence in pass 2
};

__device__ __forceinline__ uint16_t to_bf16(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // round to nearest even
}
__device__ __forceinline__ float from_bf16(uint32_t b) { return __uint_as_float(b << 16); }

// v = hi + lo + O(2^-16 |v|), hi and lo bf16.
struct HiLo {
    short hi, lo;
};
__device__ __forceinline__ HiLo split_bf16(float v) {
    const uint16_t h = to_bf16(v);
    return {static_cast<short>(h), static_cast<short>(to_bf16(v - from_bf16(h)))};
}

// Logical workgroup id for hardware id i of n: the hardware deals workgroups to the 8 XCDs
// round-robin; this gives each XCD one contiguous range of logical ids, so the channel blocks of
// one sequence (consecutive logical ids) share an L2 and fetch that sequence's B, C and m rows
// from memory once.
__device__ __forceinline__ int xcd_remap(int i, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = i & 7, k = i >> 3;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + k;
}

template <typename IO> struct Io;
template <> struct Io<float> { using elem = float; };
template <> struct Io<uint16_t> { using elem = uint16_t; };

__device__ __forceinline__ float ld_val(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_val(const uint16_t* p, int64_t i) { return from_bf16(p[i]); }

// ---------------------------------------------------------------------------------------------
// The state contraction of one wave: acc[q][nb] += B'^T X over the 16-token tiles t0 = tb +
// 16 wave, tb + 16 (wave + 4), ... below te, for the 64 channels d0..d0+63. On return acc[q][nb][r]
// is the state at n = 16 nb + 4 grp + r, channel d0 + 4 col + q (lane = 16 grp + col).
// Tiles are taken kGroup<NB> at a time: every load of a group is issued before any of its
// arithmetic, so a wave waits for memory once per group rather than once per tile.

template <int NB> constexpr int kGroup = NB >= 4 ? 2 : 1;

template <typename IO, int NB>
__device__ __forceinline__ void state_tiles(const NcArgs& a, int64_t row0, int d0, int tb, int te, int wave,
                                            int lane, v4f (&acc)[4][NB]) {
    constexpr int N = 16 * NB;
    constexpr int G = kGroup<NB>;
    using E = typename Io<IO>::elem;
    const E* x = static_cast<const E*>(a.x);
    const E* Bm = static_cast<const E*>(a.B);
    const int col = lane & 15, grp = lane >> 4;
    // This lane's channels dl..dl+3. A lane past d_inner (Di % 16 == 0: all four or none) reads
    // the last four channels instead: its MFMA column feeds only outputs of its own (invalid)
    // channels, which are never stored. Every load below is unconditional and in bounds, so the
    // loads of a group are all in flight together; a token past the range is read at the range's
    // last token and its x and B' are zeroed by a select, which keeps it out of the sums even when
    // that token holds NaN or Inf.
    const int dl = min(d0 + 4 * col, a.Di - 4);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[q][nb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    for (int g0 = tb + wave * kTile; g0 < te; g0 += G * kWaves * kTile) {
        // the lane's token of slot (gi, e): bf16 t0 + 4 grp + e (K = 16), fp32 t0 + 4 e + grp
        // (four K = 4 steps), t0 = g0 + 64 gi
        auto token = [&](int gi, int e) {
            return g0 + gi * kWaves * kTile + (sizeof(E) == 2 ? 4 * grp + e : 4 * e + grp);
        };
        using XRaw = typename std::conditional<sizeof(E) == 2, uint2, float4>::type;
        XRaw xr[G][4];
        float mv[G][4];
        E braw[G][NB][4];
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = row0 + min(token(gi, e), te - 1);
                xr[gi][e] = *reinterpret_cast<const XRaw*>(x + row * a.Di + dl);
                mv[gi][e] = a.m[row];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) braw[gi][nb][e] = Bm[row * N + nb * 16 + col];
            }
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (token(gi, e) >= te) {   // a select: both values are already loaded
                    xr[gi][e] = XRaw{};
                    mv[gi][e] = 0.0f;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) braw[gi][nb][e] = E{};
                }
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            if constexpr (sizeof(E) == 2) {
                v4s bx[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bx[0][e] = static_cast<short>(xr[gi][e].x & 0xffffu);
                    bx[1][e] = static_cast<short>(xr[gi][e].x >> 16);
                    bx[2][e] = static_cast<short>(xr[gi][e].y & 0xffffu);
                    bx[3][e] = static_cast<short>(xr[gi][e].y >> 16);
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    v4s ah, al;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const HiLo hl = split_bf16(from_bf16(braw[gi][nb][e]) * mv[gi][e]);
                        ah[e] = hl.hi;
                        al[e] = hl.lo;
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[q][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bx[q], acc[q][nb], 0, 0, 0);
                        acc[q][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bx[q], acc[q][nb], 0, 0, 0);
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const float bv = braw[gi][nb][e] * mv[gi][e];
                        acc[0][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv, xr[gi][e].x, acc[0][nb], 0, 0, 0);
                        acc[1][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv, xr[gi][e].y, acc[1][nb], 0, 0, 0);
                        acc[2][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv, xr[gi][e].z, acc[2][nb], 0, 0, 0);
                        acc[3][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv, xr[gi][e].w, acc[3][nb], 0, 0, 0);
                    }
            }
        }
    }
}

// The four waves' partial states added in wave order through LDS: every wave ends with the
// workgroup's state in its own accumulator layout, h[q][nb][r] = state n = 16 nb + 4 grp + r of
// channel d0 + 4 col + q. red holds one float4 per (wave, q, nb, lane).
template <int NB>
__device__ __forceinline__ void sum_waves(float4 (*red)[4 * NB][64], int wave, int lane, const v4f (&acc)[4][NB],
                                          v4f (&h)[4][NB]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            red[wave][q * NB + nb][lane] = make_float4(acc[q][nb][0], acc[q][nb][1], acc[q][nb][2], acc[q][nb][3]);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float4 v = red[0][q * NB + nb][lane];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                const float4 o = red[w][q * NB + nb][lane];
                v.x += o.x;
                v.y += o.y;
                v.z += o.z;
                v.w += o.w;
            }
            h[q][nb] = v4f{v.x, v.y, v.z, v.w};
        }
}

// C rows of the readout, kOutGroup<NB> tiles at a time, as the B operands of this lane: the four
// states 16 nb + 4 grp + 0..3 of token t0 + col (t0 = g0 + 64 gi), bf16 packed in a uint2 or
// fp32 in a float4. The readout's first group is loaded before the state contraction, so its
// latency is hidden behind that pass.
template <int NB> constexpr int kOutGroup = NB >= 4 ? 2 : 4;
template <typename IO, int NB> struct CRows;
template <int NB> struct CRows<uint16_t, NB> { uint2 v[kOutGroup<NB>][NB]; };
template <int NB> struct CRows<float, NB> { float4 v[kOutGroup<NB>][NB]; };

template <typename IO, int NB>
__device__ __forceinline__ void load_c(const NcArgs& a, int64_t row0, int g0, int ge, int lane, CRows<IO, NB>& c) {
    constexpr int N = 16 * NB;
    using E = typename Io<IO>::elem;
    using V = typename std::conditional<sizeof(E) == 2, uint2, float4>::type;
    const E* Cm = static_cast<const E*>(a.C);
    const int col = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int gi = 0; gi < kOutGroup<NB>; ++gi) {
        // a token past the group reads the group's last row (only its own output column, never
        // stored, depends on it): the loads are unconditional and in bounds
        const int64_t row = row0 + min(g0 + gi * kWaves * kTile + col, ge - 1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) c.v[gi][nb] = *reinterpret_cast<const V*>(Cm + row * N + nb * 16 + 4 * grp);
    }
}

// The readout of one wave: y = C H for the 16-token tiles i0 = gb + 16 wave, gb + 16 (wave + 4),
// ... below ge and the 64 channels d0..d0+63. MFMA q's row m is channel d0 + 4 m + q, the
// column mapping of the state contraction, so h (in that pass's accumulator layout) is already
// this lane's A operand: row col, states 16 nb + 4 grp + e. The K index e of a 16x16x16 bf16
// step, or the step s of the four 16x16x4 fp32 steps, is state 16 nb + 4 grp + e (or + s), and
// the C operand follows the same order. The output lane holds rows 4 grp + r, i.e. channels
// d0 + 16 grp + 4 r + q of token i0 + col: 16 consecutive channels, regrouped into whole rows
// through the wave's LDS area stage before they are stored. cr holds the C rows of the wave's
// first group of tiles.
template <typename IO, int NB>
__device__ __forceinline__ void out_tiles(const NcArgs& a, int64_t row0, int d0, int gb, int ge, int wave, int lane,
                                          const v4f (&h)[4][NB], uint32_t* stage, CRows<IO, NB> cr) {
    constexpr int G = kOutGroup<NB>;
    using E = typename Io<IO>::elem;
    E* y = static_cast<E*>(a.y);
    const int col = lane & 15, grp = lane >> 4;
    const int first = gb + wave * kTile;

    if constexpr (sizeof(E) == 2) {
        v4s ah[4][NB], al[4][NB];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const HiLo hl = split_bf16(h[q][nb][e]);
                    ah[q][nb][e] = hl.hi;
                    al[q][nb][e] = hl.lo;
                }
        for (int g0 = first; g0 < ge; g0 += G * kWaves * kTile) {
            if (g0 != first) load_c<IO, NB>(a, row0, g0, ge, lane, cr);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                if (g0 + gi * kWaves * kTile >= ge) break;
                v4f acc[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    v4s bc;
                    bc[0] = static_cast<short>(cr.v[gi][nb].x & 0xffffu);
                    bc[1] = static_cast<short>(cr.v[gi][nb].x >> 16);
                    bc[2] = static_cast<short>(cr.v[gi][nb].y & 0xffffu);
                    bc[3] = static_cast<short>(cr.v[gi][nb].y >> 16);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah[q][nb], bc, acc[q], 0, 0, 0);
                        acc[q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al[q][nb], bc, acc[q], 0, 0, 0);
                    }
                }
                // channel 16 grp + 4 r + q is acc[q][r]; pairs (q = 0, 1) and (2, 3) share a word
                uint32_t w[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    w[2 * r] = static_cast<uint32_t>(to_bf16(acc[0][r])) | (static_cast<uint32_t>(to_bf16(acc[1][r])) << 16);
                    w[2 * r + 1] =
                        static_cast<uint32_t>(to_bf16(acc[2][r])) | (static_cast<uint32_t>(to_bf16(acc[3][r])) << 16);
                }
                // through the wave's LDS tile [16 tokens][64 channels] (rows padded to 36 words) so
                // that each store instruction writes eight whole 128-byte rows
                uint4* srow = reinterpret_cast<uint4*>(stage + col * kStageRow + 8 * grp);
                srow[0] = make_uint4(w[0], w[1], w[2], w[3]);
                srow[1] = make_uint4(w[4], w[5], w[6], w[7]);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int r = 8 * hh + (lane >> 3), c8 = lane & 7;  // row of the tile, 8-channel piece
                    const uint4 v = *reinterpret_cast<const uint4*>(stage + r * kStageRow + 4 * c8);
                    const int t = g0 + gi * kWaves * kTile + r;
                    if (t < ge && d0 + 8 * c8 < a.Di)
                        *reinterpret_cast<uint4*>(y + (row0 + t) * a.Di + d0 + 8 * c8) = v;
                }
            }
        }
    } else {
        for (int g0 = first; g0 < ge; g0 += G * kWaves * kTile) {
            if (g0 != first) load_c<IO, NB>(a, row0, g0, ge, lane, cr);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                if (g0 + gi * kWaves * kTile >= ge) break;
                v4f acc[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float cs[4] = {cr.v[gi][nb].x, cr.v[gi][nb].y, cr.v[gi][nb].z, cr.v[gi][nb].w};
#pragma unroll
                    for (int st = 0; st < 4; ++st)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(h[q][nb][st], cs[st], acc[q], 0, 0, 0);
                }
                // through the wave's LDS tile [16 tokens][64 channels] (rows padded to 68 words):
                // each store instruction writes four whole 256-byte rows
                float4* srow = reinterpret_cast<float4*>(stage + col * kStageRowF + 16 * grp);
#pragma unroll
                for (int r = 0; r < 4; ++r) srow[r] = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
#pragma unroll
                for (int hh = 0; hh < 4; ++hh) {
                    const int r = 4 * hh + (lane >> 4), c4 = lane & 15;  // row of the tile, 4-channel piece
                    const float4 v = *reinterpret_cast<const float4*>(stage + r * kStageRowF + 4 * c4);
                    const int t = g0 + gi * kWaves * kTile + r;
                    if (t < ge && d0 + 4 * c4 < a.Di)
                        *reinterpret_cast<float4*>(y + (row0 + t) * a.Di + d0 + 4 * c4) = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Whole sequence in one workgroup (the sequence is not split): the state is summed in LDS and
// read out at once; it never goes to memory. One workgroup per (channel block, sequence), channel
// block fastest.

// bf16 with N = 16 (the Vim shapes) is asked for 6 waves per SIMD: left alone the compiler used
// 84 VGPRs, which allocate as 88 and fit 5, so a grid of 6 waves per SIMD ran as one full and one
// partial generation; at 70 VGPRs (no spills) it is a single generation.
template <typename IO, int NB>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(sizeof(typename Io<IO>::elem) == 2 && NB == 1 ? 6 : 1)))
void k_ncssd_fused(NcArgs a) {
    __shared__ float4 red[kWaves][4 * NB][64];
    __shared__ __attribute__((aligned(16))) uint32_t stage[kWaves][kStageWords<IO>];
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int wave = static_cast<int>(threadIdx.x) >> 6;
    const int lid = xcd_remap(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
    const int d0 = (lid % a.ncb) * kBlock;
    const int64_t row0 = static_cast<int64_t>(lid / a.ncb) * a.T;
    CRows<IO, NB> cr;
    load_c<IO, NB>(a, row0, wave * kTile, a.T, lane, cr);  // in flight during the state pass
    v4f acc[4][NB], h[4][NB];
    state_tiles<IO, NB>(a, row0, d0, 0, a.T, wave, lane, acc);
    sum_waves<NB>(red, wave, lane, acc, h);
    out_tiles<IO, NB>(a, row0, d0, 0, a.T, wave, lane, h, stage[wave], cr);
}

// Pass 1 of a split sequence: the partial state of one token range. One workgroup per (channel
// block, range, sequence), in that order of speed.
template <typename IO, int NB>
__global__ __launch_bounds__(256) void k_ncssd_state(NcArgs a) {
    constexpr int N = 16 * NB;
    __shared__ float4 red[kWaves][4 * NB][64];
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int wave = static_cast<int>(threadIdx.x) >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int lid = xcd_remap(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
    const int d0 = (lid % a.ncb) * kBlock;
    const int split = (lid / a.ncb) % a.splits;
    const int s = lid / a.ncb / a.splits;
    const int tb = split * a.span;
    const int te = min(tb + a.span, a.T);
    v4f acc[4][NB], h[4][NB];
    state_tiles<IO, NB>(a, static_cast<int64_t>(s) * a.T, d0, tb, te, wave, lane, acc);
    sum_waves<NB>(red, wave, lane, acc, h);
    // wave 0 stores the block: state n = 16 nb + 4 grp + r, channels d0 + 4 col + 0..3
    if (wave == 0 && d0 + 4 * col < a.Di) {
        float* dst = a.part + (static_cast<int64_t>(s) * a.splits + split) * N * a.Di + d0 + 4 * col;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<float4*>(dst + static_cast<int64_t>(nb * 16 + 4 * grp + r) * a.Di) =
                    make_float4(h[0][nb][r], h[1][nb][r], h[2][nb][r], h[3][nb][r]);
    }
}

// Sum of the split partial states, in split order. One thread per 4 values of H.
__global__ __launch_bounds__(256) void k_ncssd_reduce(NcArgs a, int64_t quads, int nd) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= quads) return;
    const int64_t s = i / (nd / 4), r = i % (nd / 4);  // nd = N * Di values per sequence
    const float4* src = reinterpret_cast<const float4*>(a.part + s * a.splits * nd) + r;
    float4 v = src[0];
    for (int k = 1; k < a.splits; ++k) {
        const float4 o = src[static_cast<int64_t>(k) * (nd / 4)];
        v.x += o.x;
        v.y += o.y;
        v.z += o.z;
        v.w += o.w;
    }
    reinterpret_cast<float4*>(a.H + s * nd)[r] = v;
}

// Pass 2 of a split sequence: y = C H for kOutTokens tokens x 64 channels, H from memory. One
// workgroup per (channel block, token group, sequence), in that order of speed.
template <typename IO, int NB>
__global__ __launch_bounds__(256) void k_ncssd_out(NcArgs a) {
    constexpr int N = 16 * NB;
    __shared__ __attribute__((aligned(16))) uint32_t stage[kWaves][kStageWords<IO>];
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int wave = static_cast<int>(threadIdx.x) >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int lid = xcd_remap(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
    const int d0 = (lid % a.ncb) * kBlock;
    const int gb = ((lid / a.ncb) % a.groups) * kOutTokens;
    const int s = lid / a.ncb / a.groups;
    const int ge = min(gb + kOutTokens, a.T);
    const int64_t row0 = static_cast<int64_t>(s) * a.T;
    CRows<IO, NB> cr;
    load_c<IO, NB>(a, row0, gb + wave * kTile, ge, lane, cr);
    // this lane's state values in the accumulator layout; a lane past d_inner reads the last four
    // channels (only its own output rows, never stored, depend on them)
    const float* Hs = a.H + static_cast<int64_t>(s) * N * a.Di + min(d0 + 4 * col, a.Di - 4);
    v4f h[4][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 v = *reinterpret_cast<const float4*>(Hs + static_cast<int64_t>(nb * 16 + 4 * grp + r) * a.Di);
            h[0][nb][r] = v.x;
            h[1][nb][r] = v.y;
            h[2][nb][r] = v.z;
            h[3][nb][r] = v.w;
        }
    out_tiles<IO, NB>(a, row0, d0, gb, ge, wave, lane, h, stage[wave], cr);
}

// ---------------------------------------------------------------------------------------------
// Host side

template <typename IO, int NB>
int nc_launch(const NcArgs& a, const NcPlan& p, hipStream_t s) {
    const dim3 block(kBlock * kWaves);
    if (p.splits == 1) {
        hipLaunchKernelGGL((k_ncssd_fused<IO, NB>), dim3(static_cast<unsigned>(p.ncb * p.nseq)), block, 0, s, a);
        return hipGetLastError() == hipSuccess ? VIMSCAN_OK : VIMSCAN_ERR_HIP;
    }
    hipLaunchKernelGGL((k_ncssd_state<IO, NB>), dim3(static_cast<unsigned>(p.ncb * p.splits * p.nseq)), block, 0, s, a);
    const int nd = static_cast<int>(p.N * a.Di);
    const int64_t quads = p.nseq * nd / 4;
    hipLaunchKernelGGL(k_ncssd_reduce, dim3(static_cast<unsigned>((quads + 255) / 256)), dim3(256), 0, s, a, quads, nd);
    hipLaunchKernelGGL((k_ncssd_out<IO, NB>), dim3(static_cast<unsigned>(p.ncb * p.groups * p.nseq)), block, 0, s, a);
    return hipGetLastError() == hipSuccess ? VIMSCAN_OK : VIMSCAN_ERR_HIP;
}

template <typename IO>
int nc_dispatch(const NcArgs& a, const NcPlan& p, hipStream_t s) {
    switch (p.N) {
        case 16: return nc_launch<IO, 1>(a, p, s);
        case 32: return nc_launch<IO, 2>(a, p, s);
        default: return nc_launch<IO, 4>(a, p, s);
    }
}

}  // namespace

extern "C" {

int vimscan_ncssd_fwd(const void* x, const void* B, const void* C, const float* m, int64_t seg_len, void* y,
                      const vimscan_launch* launch) {
    if (!launch) return VIMSCAN_ERR_NULL;
    NcPlan p;
    int rc = vimscan_host::make_nc_plan(launch, seg_len, &p);
    if (rc != VIMSCAN_OK) return rc;
    if (launch->batch == 0 || launch->seqlen == 0 || launch->d_inner == 0) return VIMSCAN_OK;
    rc = vimscan_host::check_ncssd_call(x, B, C, m, y, launch, p);
    if (rc != VIMSCAN_OK) return rc;
    const bool bf = launch->io_dtype == VIMSCAN_BF16;

    NcArgs a;
    a.x = x;
    a.B = B;
    a.C = C;
    a.m = m;
    a.y = y;
    char* ws = static_cast<char*>(launch->workspace);
    a.H = p.splits > 1 ? reinterpret_cast<float*>(ws + p.off_H) : nullptr;
    a.part = p.splits > 1 ? reinterpret_cast<float*>(ws) : nullptr;
    a.T = static_cast<int>(p.T);
    a.Di = static_cast<int>(launch->d_inner);
    a.splits = static_cast<int>(p.splits);
    a.span = static_cast<int>(p.span);
    a.ncb = static_cast<int>(p.ncb);
    a.groups = static_cast<int>(p.groups);
    hipStream_t s = static_cast<hipStream_t>(launch->stream);
    hipEvent_t ev0 = static_cast<hipEvent_t>(launch->scan_events[0]);
    hipEvent_t ev1 = static_cast<hipEvent_t>(launch->scan_events[1]);
    const bool timed = ev0 && ev1;
    if (timed && hipEventRecord(ev0, s) != hipSuccess) return VIMSCAN_ERR_HIP;
    const int lr = bf ? nc_dispatch<uint16_t>(a, p, s) : nc_dispatch<float>(a, p, s);
    if (lr != VIMSCAN_OK) return lr;
    if (timed && hipEventRecord(ev1, s) != hipSuccess) return VIMSCAN_ERR_HIP;
    return VIMSCAN_OK;
}

}  // extern "C"
