/*
 * vimscan.h -- C ABI of the bidirectional selective scan on AMD MI355X (gfx950), with its
 * variants (directional convolution in front, forward only with the auxiliary swap, a given token
 * order) and the NC-SSD global-state form (declared further down).
 *
 * The operation (Vision Mamba page, section 2.2 "bidirectional state-space modelling": a
 * forward path over the tokens in raster order and a backward path over them in reverse, the
 * two fused; the fusion here is the sum gated by SiLU(z)). For every batch row b, channel d:
 *
 *   delta_t   = softplus(dt[b,t,d] + dt_bias[d])                       (selective step size)
 *   Abar_t[n] = exp(delta_t * A[d,n]),  Bbar_t[n] = delta_t * B[b,t,n]
 *                 (discretisation: VSSD notes page, section 4.1.2, first-order form for B)
 *   forward:  h_t = Abar_t * h_{t-1} + Bbar_t * x[b,t,d],  t = 0..L-1,  h_{-1} = 0
 *   backward: g_t = Abar'_t * g_{t+1} + Bbar'_t * x[b,t,d], t = L-1..0,  g_L = 0
 *                 (linear SSD form: VSSD notes page, section 4.2.1.3)
 *   yf_t = C_f[b,t,:] . h_t + D_f[d] x[b,t,d];   yb_t = C_b[b,t,:] . g_t + D_b[d] x[b,t,d]
 *                 (readout with skip term: Mamba2D page, "standard Mamba 1D formula")
 *   y[b,t,d]  = silu(z[b,t,d]) * (yf_t + yb_t),   silu(v) = v / (1 + exp(-v))
 *
 * with the forward quantities taken from (A_f, B_f, C_f, D_f, dt_bias_f) and the backward ones
 * from (A_b, B_b, C_b, D_b, dt_bias_b). The backward path reads the same buffers at descending
 * t; nothing is flipped or copied. State (N = 16 floats per channel and direction) is fp32 and
 * never leaves the chip except as chunk carries in the workspace.
 *
 * Periodic reset (SF-Mamba page, "Batch folding and periodic state reset"): with seg_len > 0
 * the state is cleared before the update at the first token of every segment the scan enters
 * (forward: t % seg_len == 0; backward: (t + 1) % seg_len == 0), so B short sequences of
 * length T folded into one stream of length B*T give the same outputs as the unfolded batch.
 *
 * Layouts (row-major, last index fastest, all dense):
 *   x, dt, z, y           [batch][seqlen][d_inner]   io dtype (fp32 or bf16)
 *   B_f, C_f, B_b, C_b    [batch][seqlen][d_state]   io dtype
 *   A_f, A_b              [d_inner][d_state]         fp32
 *   D_f, D_b, dt_bias_*   [d_inner]                  fp32
 * dt is the step before the bias is added. bf16 outputs are rounded to nearest even.
 *
 * Ownership and execution: every pointer is device memory owned by the caller; the library
 * allocates and frees nothing and keeps no state between calls. Work is queued on the given
 * stream and the call returns without synchronising. Inputs are read only; y must not overlap
 * any input. All argument checks run on the host before any HIP call, so every error other
 * than VIMSCAN_ERR_HIP leaves the device untouched.
 */
#ifndef VIMSCAN_H
#define VIMSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum vimscan_status {
    VIMSCAN_OK = 0,
    VIMSCAN_ERR_NULL = -1,      /* a required pointer is NULL (launch, an input, or y) */
    VIMSCAN_ERR_SHAPE = -2,     /* batch, seqlen or d_inner < 0; d_inner >= 2^22;
                                   batch*seqlen*d_inner >= 2^31; d_state != 16 for the scans;
                                   for NC-SSD d_state not 16, 32 or 64 or d_inner % 16 != 0 */
    VIMSCAN_ERR_SEGLEN = -3,    /* seg_len < 0, or seg_len > 0 and seqlen % seg_len != 0 */
    VIMSCAN_ERR_DTYPE = -4,     /* io_dtype is not VIMSCAN_F32 or VIMSCAN_BF16 */
    VIMSCAN_ERR_ALIGN = -5,     /* a pointer is not aligned: x, dt, z, y to the io element
                                   size; B_*, C_* and the fp32 parameters to 4 bytes */
    VIMSCAN_ERR_ALIAS = -6,     /* y overlaps an input */
    VIMSCAN_ERR_WORKSPACE = -7, /* workspace NULL or smaller than vimscan_workspace_bytes */
    VIMSCAN_ERR_HIP = -8,       /* a kernel launch failed (hipGetLastError after launching) */
    VIMSCAN_ERR_CHUNK = -9,     /* chunk_len < 0 */
    VIMSCAN_ERR_FLAGS = -10,    /* unknown bits in flags */
    VIMSCAN_ERR_CONV = -11,     /* vimscan_conv.k outside 1..4 */
    VIMSCAN_ERR_SCRATCH = -12   /* vimscan_bidir_fwd_noalloc: the call needs more scratch than
                                   VIMSCAN_NOALLOC_SCRATCH_BYTES */
};

/* dtype of x, dt, z, B_*, C_* and y. */
enum vimscan_io_dtype { VIMSCAN_F32 = 0, VIMSCAN_BF16 = 1 };

/* flags */
/* Evaluate exp(delta*A[d,n]) once per (token, channel, state) even when a channel's A row is
   an arithmetic progression in n that is non-positive and non-increasing (A[d,0] <= 0 and
   A[d,1] - A[d,0] <= 0), for which the library otherwise forms the transitions as
   exp(delta*A[d,0]) * exp(delta*(A[d,1]-A[d,0]))^n. Both give the defined result. Other rows
   always take one exponential per state. */
#define VIMSCAN_FLAG_GENERAL_DECAY 1
/* Auxiliary-token swap (SF-Mamba page, "auxiliary patch swapping"): after the scan, exchange
   the outputs of the first and the last token of every sequence (every segment when
   seg_len > 0), i.e. the page's exchange of the head and tail auxiliary tokens between layers
   (one more small kernel on the stream). For every entry point. */
#define VIMSCAN_FLAG_AUX_SWAP 2
/* The launch describes a forward-only call (vimscan_fwd). vimscan_fwd implies it; the planning
   functions need it to size the forward-only plan; vimscan_bidir_fwd, vimscan_bidir_conv_fwd and
   vimscan_bidir_order_fwd reject it (VIMSCAN_ERR_FLAGS). */
#define VIMSCAN_FLAG_FORWARD_ONLY 4

/* Shape and launch description, passed by pointer to every entry point. */
typedef struct vimscan_launch {
    int64_t batch;          /* B >= 0 */
    int64_t seqlen;         /* L >= 0 (the folded stream length when seg_len > 0) */
    int64_t d_inner;        /* Di >= 0 */
    int64_t d_state;        /* N; 16 for the scans; 16, 32 or 64 for vimscan_ncssd_fwd */
    int32_t io_dtype;       /* enum vimscan_io_dtype */
    int32_t flags;          /* VIMSCAN_FLAG_* bits */
    int64_t chunk_len;      /* 0: the library picks; > 0: tokens per chunk of the chunked scan,
                               capped at 256 (a value >= the sequence length gives a single
                               pass for sequences of up to 256 tokens) */
    void* workspace;        /* device scratch of at least vimscan_workspace_bytes() bytes;
                               may be NULL when that size is 0. Its contents on entry do not
                               matter (no clearing needed); calls that can overlap in time must
                               not share one */
    size_t workspace_bytes; /* size of workspace */
    void* stream;           /* hipStream_t to queue the work on; NULL = the null stream */
    void* scan_events[2];   /* optional pair of hipEvent_t created by the caller: when both are
                               non-NULL, the call records scan_events[0] on the stream just
                               before the main scan kernel and scan_events[1] just after it, so
                               the caller can time that kernel alone; NULL: nothing recorded.
                               A failed record returns VIMSCAN_ERR_HIP. */
} vimscan_launch;

/*
 * The directional depthwise convolution in front of the scan (vimscan_bidir_conv_fwd): each
 * direction passes x through its own 1D depthwise convolution of k taps plus a bias, then SiLU,
 * and scans the result u in place of x (in delta*B*u and in the skip term D*u). The forward
 * convolution is causal and the backward one anti-causal, each in its own walking order
 * (Vim page, section 2.3: the forward and backward paths use 1D convolutions of opposite
 * directions; SF-Mamba page, "MambaVision Mixer": SSM(SiLU(Conv(.)))):
 *   u_f[t] = silu(bias_f[d] + sum_{j=0}^{k-1} w_f[d][k-1-j] * x[t-j])
 *   u_b[t] = silu(bias_b[d] + sum_{j=0}^{k-1} w_b[d][k-1-j] * x[t+j])
 * so w[d][k-1] weights the current token, as in a PyTorch conv1d weight [d][0][k] with k-1
 * zeros of padding on the side the direction comes from. Tokens outside the current sequence
 * (the current segment when seg_len > 0) count as zero: the convolution never crosses a fold
 * boundary (SF-Mamba page, "1D depthwise separable convolution adaptation").
 */
typedef struct vimscan_conv {
    const float* w_f;       /* [d_inner][k] fp32 forward taps, device memory */
    const float* bias_f;    /* [d_inner] fp32 */
    const float* w_b;       /* [d_inner][k] fp32 backward taps */
    const float* bias_b;    /* [d_inner] fp32 */
    int64_t k;              /* taps, 1..4 (VIMSCAN_ERR_CONV otherwise) */
} vimscan_conv;

/* How a call with this launch is executed (for reporting and tests). */
typedef struct vimscan_plan {
    int64_t sequences;      /* independent sequences: batch, or batch*seqlen/seg_len */
    int64_t seq_tokens;     /* tokens per independent sequence */
    int64_t chunk_len;      /* tokens per chunk */
    int64_t chunks;         /* chunks per sequence; 1 = single pass (no chunk carries) */
    int64_t workgroups;     /* workgroups of the main scan kernel */
    int32_t kernels;        /* kernels launched per call: 1 for a single pass and for 2..16
                               chunks per sequence (one kernel computes each chunk's aggregate,
                               hands it to the later chunks through the workspace and folds
                               those it receives), bidirectional and forward only alike; past
                               16 chunks 3 (chunk aggregates, carry combine, scan); plus 1 with
                               VIMSCAN_FLAG_AUX_SWAP */
    int32_t park_in_workspace; /* 1: the two directions exchange their outputs through the
                               workspace (long chunks); 0: through LDS */
    size_t workspace_bytes; /* scratch this call needs: chunk carries and delta sums when
                               chunks > 1, chunk_len*64*4 bytes per wave pair when
                               park_in_workspace, and 8 bytes per (direction, sequence, chunk,
                               64-channel block) of hand-over tags for the one-kernel chunked
                               scan (0: no workspace needed) */
} vimscan_plan;

/*
 * y = silu(z) * (forward scan + backward scan), as defined above, queued on launch->stream.
 * x, dt, z, B_f, C_f, B_b, C_b and y are io-dtype device arrays; A_*, D_*, dt_bias_* are fp32
 * device arrays. seg_len: 0 for no reset, else the reset period (must divide seqlen).
 * Returns VIMSCAN_OK or a negative vimscan_status. Empty shapes (batch, seqlen or d_inner 0)
 * are checked for shape, dtype, seg_len and flags and then return VIMSCAN_OK without launching;
 * their pointers may be NULL.
 */
int vimscan_bidir_fwd(const void* x, const void* dt, const void* z, const void* B_f,
                      const void* C_f, const void* B_b, const void* C_b, const float* A_f,
                      const float* A_b, const float* D_f, const float* D_b,
                      const float* dt_bias_f, const float* dt_bias_b, int64_t seg_len, void* y,
                      const vimscan_launch* launch);

/*
 * The same as vimscan_bidir_fwd with the directional convolution of *conv in front of each
 * direction (see vimscan_conv). x is the convolution's input; conv and the arrays it points to
 * are read only (host struct, device arrays 4-byte aligned) and must not overlap y or the
 * workspace. Plan and workspace are those of vimscan_bidir_fwd for the same launch.
 * Returns VIMSCAN_OK or a negative vimscan_status (VIMSCAN_ERR_NULL for a NULL conv or conv
 * array, VIMSCAN_ERR_CONV for k outside 1..4, checked before the shape).
 */
int vimscan_bidir_conv_fwd(const void* x, const vimscan_conv* conv, const void* dt, const void* z,
                           const void* B_f, const void* C_f, const void* B_b, const void* C_b,
                           const float* A_f, const float* A_b, const float* D_f, const float* D_b,
                           const float* dt_bias_f, const float* dt_bias_b, int64_t seg_len, void* y,
                           const vimscan_launch* launch);

/*
 * The bidirectional scan in a given token order (DefMamba page: section 1 compares raster,
 * Hilbert-curve and local-window scan orders; section 2.1 re-ranks the tokens of the sequence by
 * per-token index offsets). order is device memory, int32 [batch * seqlen / T][T] with T =
 * seg_len (or seqlen when seg_len is 0): row s lists the token positions 0..T-1 of sequence
 * (segment) s in the order the forward path visits them; the backward path visits the same
 * tokens from the end of the list. Every step reads its token's x, dt, B and C, and each
 * direction's output lands at the token's own position:
 *   forward:  h at step k uses token order[s][k], k = 0..T-1
 *   backward: g at step k uses token order[s][k], k = T-1..0
 *   y[b,t,d] = silu(z[b,t,d]) * (yf_t + yb_t) with yf_t, yb_t the readouts at token t.
 * The raster order order[s][k] = k gives vimscan_bidir_fwd's result. Rows must be permutations;
 * entries outside 0..T-1 are clamped into the sequence (unspecified outputs, no access outside
 * the arrays). order must be 4-byte aligned (VIMSCAN_ERR_ALIGN) and must not overlap y or the
 * workspace (VIMSCAN_ERR_ALIAS); NULL is VIMSCAN_ERR_NULL unless the call is empty. Everything
 * else -- layouts, reset, dtypes, plan and workspace -- is that of vimscan_bidir_fwd, plus
 * VIMSCAN_ERR_SHAPE when T * d_inner * (io element size) >= 2^32 (a walk addresses a whole
 * sequence with 32-bit offsets).
 */
int vimscan_bidir_order_fwd(const void* x, const void* dt, const void* z, const void* B_f,
                            const void* C_f, const void* B_b, const void* C_b, const float* A_f,
                            const float* A_b, const float* D_f, const float* D_b,
                            const float* dt_bias_f, const float* dt_bias_b, const int32_t* order,
                            int64_t seg_len, void* y, const vimscan_launch* launch);

/*
 * Unidirectional scan (SF-Mamba page: Vim with a one-way scan and auxiliary patch swap): only
 * the forward path of the definition above, gated:
 *   y[b,t,d] = silu(z[b,t,d]) * (C[b,t,:] . h_t + D[d] x[b,t,d])
 * with h_t from (A, B, D, dt_bias) as the forward direction of vimscan_bidir_fwd, the same
 * layouts, reset, dtypes and errors; usually combined with VIMSCAN_FLAG_AUX_SWAP. Plan and
 * workspace are those of a launch with VIMSCAN_FLAG_FORWARD_ONLY (implied here).
 */
int vimscan_fwd(const void* x, const void* dt, const void* z, const void* B, const void* C,
                const float* A, const float* D, const float* dt_bias, int64_t seg_len, void* y,
                const vimscan_launch* launch);

/*
 * NC-SSD, the non-causal global-state form of state-space duality (VSSD page, sections 4.2.3 to
 * 4.2.5): the SSD recurrence divided by each token's scalar transition A_j, summed over both
 * scan directions and without the token's own term, leaves one hidden state per sequence that
 * every token reads out:
 *   H[n][d] = sum_j B[j][n] * m[j] * x[j][d],   y[i][d] = sum_n C[i][n] * H[n][d]
 * i.e. y = C (B^T (x . m)) per sequence, with m[j] = 1 / A_j the weight of token j. With
 * seg_len > 0 every segment of seg_len tokens is its own sequence with its own H (folding).
 *
 * Layouts (row-major, dense): x, y [batch][seqlen][d_inner] io dtype; B, C
 * [batch][seqlen][d_state] io dtype; m [batch][seqlen] fp32. launch->d_state is N (16, 32 or
 * 64); d_inner must be a multiple of 16; flags must be 0 (VIMSCAN_ERR_FLAGS); chunk_len > 0
 * sets the tokens of a sequence that one workgroup of the state pass sums (rounded up to a
 * multiple of 16; 0: the library picks); scan_events, when set, are recorded before the first
 * and after the last kernel. x and y must be 16-byte aligned, B aligned to its element size, C to
 * 8 bytes (bf16) or 16 (fp32), m to 4 (VIMSCAN_ERR_ALIGN). When one workgroup covers a whole
 * sequence, H stays on the chip and no workspace is needed; when long sequences are split
 * (vimscan_ncssd_plan: chunks > 1) the workspace holds the split partial states and H. fp32 io runs the fp32 matrix-core contraction; bf16 io multiplies the
 * exact bf16 x and C by B*m and H each split into two bf16 parts, accumulating in fp32. Same
 * ownership, stream, aliasing and empty-shape rules as vimscan_bidir_fwd; VIMSCAN_ERR_SHAPE also
 * for d_state outside {16, 32, 64} or d_inner % 16 != 0.
 */
int vimscan_ncssd_fwd(const void* x, const void* B, const void* C, const float* m, int64_t seg_len,
                      void* y, const vimscan_launch* launch);

/* Plan of a vimscan_ncssd_fwd call: sequences, seq_tokens; chunk_len = tokens per state-pass
   workgroup, chunks = workgroups per sequence and channel block in that pass; workgroups of the
   state pass; kernels (1 when a sequence is not split: state and readout in one kernel; 3 when
   it is: partial states, their sum, readout); workspace_bytes (0 when not split). Host only. Returns VIMSCAN_OK or the error the call would
   return. */
int vimscan_ncssd_plan(const vimscan_launch* launch, int64_t seg_len, vimscan_plan* plan);

/* Size of the static scratch array behind vimscan_bidir_fwd_noalloc, per GPU: 96 MiB. */
#define VIMSCAN_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): vimscan_bidir_fwd with its scratch (the chunk carries,
 * delta sums and long-chunk park that vimscan_workspace_bytes reports) taken from a static device
 * array of VIMSCAN_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the
 * process ends, instead of from launch->workspace (whose two fields are ignored). Arguments,
 * results, plan and every other error are those of vimscan_bidir_fwd, checked in the same order
 * before any HIP call; a call whose workspace_bytes exceed VIMSCAN_NOALLOC_SCRATCH_BYTES returns
 * VIMSCAN_ERR_SCRATCH without launching (every workload shape of this library fits, Vim-S's
 * 77.5 MB park included). The array belongs to the current HIP device: its address is looked up
 * (hipGetSymbolAddress) on the first call on each device, which must therefore be current; the
 * call allocates nothing (no hipMalloc, hipFree or allocating library routine). The array keeps
 * the last call's contents; the scan uses no scratch value it has not written in the same call
 * (the one-kernel chunked scan reads hand-over tags that earlier calls left only to see that they
 * are not its own). Calls on one GPU share its array: two calls that can overlap in time on the same GPU
 * (different streams without an ordering between them) race on it and give undefined results;
 * calls on one stream are ordered and safe.
 */
int vimscan_bidir_fwd_noalloc(const void* x, const void* dt, const void* z, const void* B_f,
                              const void* C_f, const void* B_b, const void* C_b, const float* A_f,
                              const float* A_b, const float* D_f, const float* D_b,
                              const float* dt_bias_f, const float* dt_bias_b, int64_t seg_len, void* y,
                              const vimscan_launch* launch);

/* Fills *plan for a call with this launch and seg_len (workspace fields of launch are
   ignored). Host only; no HIP call. Returns VIMSCAN_OK or the error the call would return. */
int vimscan_plan_launch(const vimscan_launch* launch, int64_t seg_len, vimscan_plan* plan);

/* Scratch bytes a call with this launch and seg_len needs (0 for an fp32 single pass whose
   park fits in LDS). Host only. */
int vimscan_workspace_bytes(const vimscan_launch* launch, int64_t seg_len, size_t* bytes);

/* Static text for a status code; never NULL. */
const char* vimscan_status_string(int status);

/* Library version string, e.g. "vimscan 0.3.0 gfx950". */
const char* vimscan_version(void);

/*
 * Diagnostics of the one-kernel chunked scans (plans of 2..16 chunks): *count = the number of
 * waves on the current HIP device, since the library was loaded, whose wait for the chunk
 * aggregates of the earlier chunks of their sequence gave up after its bound (about a second);
 * their calls' outputs are unspecified. The hardware starts the workgroups of every XCD in
 * increasing id order, which makes every such wait end (the kernel's own comment gives the
 * argument), so the count stays 0; it exists so that a failure of that premise is visible.
 * Synchronous (a device-to-host copy after the device's queued work). Returns VIMSCAN_OK,
 * VIMSCAN_ERR_NULL or VIMSCAN_ERR_HIP.
 */
int vimscan_wait_timeouts(uint64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* VIMSCAN_H */
