/*
 * Float64 CPU oracle for the bidirectional selective scan.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain definition that the HIP path is
 * checked against. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * build, load or call it. It shares no code, header, table or helper with the HIP library.
 *
 * What it computes, for every batch row b and channel d (all in double precision):
 *
 *   Discretisation (VSSD page, section 4.1.2): the discrete transition is exp(delta * A) and
 *   the discrete input matrix is taken as delta * B (the page's first-order form, not the exact
 *   zero-order-hold one). delta = softplus(dt + dt_bias) is the selective step size: delta, B
 *   and C depend on the token (VSSD page, section 4.1.4).
 *
 *   Recurrence (VSSD page, section 4.2.1.3, the linear form of SSD; A is diagonal per
 *   (channel, state) as in S6):
 *       h_t[n] = exp(delta_t * A[d,n]) * h_{t-1}[n] + delta_t * B_t[n] * x_t,   h before t=0 is 0
 *   Readout with the skip term (Mamba2D page, "standard Mamba 1D formula": y = C h + D x):
 *       y_t = sum_n C_t[n] * h_t[n] + D[d] * x_t
 *
 *   Directions (Vim page, section 2.2): the forward path walks the tokens in raster order
 *   t = 0..L-1 with (A_f, B_f, C_f, D_f, dt_bias_f); the backward path walks them in reverse,
 *   t = L-1..0, with (A_b, B_b, C_b, D_b, dt_bias_b):
 *       g_t[n] = exp(delta^b_t * A_b[d,n]) * g_{t+1}[n] + delta^b_t * B_b_t[n] * x_t,  g after L-1 is 0
 *       yb_t   = sum_n C_b_t[n] * g_t[n] + D_b[d] * x_t
 *   Every tensor is indexed by the natural token index t in both directions, and yb lands at t.
 *
 *   Output: y_t = silu(z_t) * (yf_t + yb_t), silu(v) = v / (1 + exp(-v)).
 *
 *   Periodic reset (SF-Mamba page, "Batch folding and periodic state reset"): with
 *   seg_len > 0 the discrete transition is forced to 0 at the first token of every segment the
 *   scan enters, i.e. the state is set to 0 before the update: forward at t % seg_len == 0,
 *   backward at (t + 1) % seg_len == 0. seg_len == 0 means no reset.
 *
 * Directional convolution in front of the scan (vimscan_oracle_bidir_conv_f64): each direction
 * first passes x through its own depthwise 1D convolution followed by SiLU (Vim page, section
 * 2.3: the forward and backward paths use 1D convolutions of opposite directions; SF-Mamba
 * page, "MambaVision Mixer": SSM(SiLU(Conv(.)))), and that direction's scan then uses the result
 * u in place of x, in delta * B * u and in the skip term D * u. The forward convolution is
 * causal and the backward one anti-causal, each in its own walking order:
 *     u_f[t] = silu(cb_f[d] + sum_{j=0}^{K-1} w_f[d][K-1-j] * x[t - j])
 *     u_b[t] = silu(cb_b[d] + sum_{j=0}^{K-1} w_b[d][K-1-j] * x[t + j])
 * (w[d][K-1] weights the current token, as a padded PyTorch conv1d weight [d][0][k] does.)
 * Tokens outside the current segment count as zero (SF-Mamba page, "1D depthwise separable
 * convolution adaptation": implicit padding at every segment boundary, so the convolution never
 * crosses from one folded sequence into another).
 *
 * Unidirectional scan with auxiliary-token swap (vimscan_oracle_fwd_f64; SF-Mamba page,
 * "auxiliary patch swapping"): only the forward path, y_t = silu(z_t) * yf_t. The caller's
 * sequence already holds the two auxiliary tokens at its first and last position; with swap != 0
 * the outputs of the first and the last token of every sequence (every segment when
 * seg_len > 0) are stored at each other's position, which is the page's exchange
 * x_aux_head(i+1) = y_aux_tail(i), x_aux_tail(i+1) = y_aux_head(i) between layers.
 *
 * Non-causal global-state form, NC-SSD (vimscan_oracle_ncssd_f64; VSSD page, sections 4.2.3 to
 * 4.2.5). Dividing the SSD recurrence by the token's scalar transition A_t and keeping only the
 * relative weights gives h(t) = h(t-1) + (1/A_t) B_t x(t); summing it in both directions and
 * dropping the token's own term leaves one hidden state shared by every token of the sequence,
 *     H = sum_j m_j * B_j (x) x_j,     m_j = 1 / A_j,
 * read out by every token with its own C: y_i = C_i . H. In matrix form, per sequence,
 * Y = C (B^T (X . m)), where X . m scales token j's row of X by m_j. With seg_len > 0 every
 * segment of the stream is its own sequence with its own H. Layouts: x, y [batch][seqlen][d_inner];
 * B, C [batch][seqlen][d_state]; m [batch][seqlen]; H (optional output)
 * [batch * seqlen / T][d_state][d_inner].
 *
 * Scan in a given token order (vimscan_oracle_bidir_order_f64; DefMamba page, section 1, the
 * table of scan orders (raster, Hilbert curve, local windows), and section 2.1, the deformable
 * scan whose index offsets re-rank the tokens of the sequence): per sequence (segment when
 * seg_len > 0) an order lists the T token positions in the sequence the scan visits them in.
 * The forward path visits order[0], order[1], ..., order[T-1]; the backward path visits the same
 * tokens in the opposite order, order[T-1], ..., order[0]. Each step uses that token's x, dt, B
 * and C, and each direction's readout lands at the token's own position, so
 * y[t] = silu(z[t]) * (yf[t] + yb[t]) as before. The raster order order[k] = k is the plain
 * bidirectional scan. The state starts from zero at the first step of every sequence.
 *
 * Layouts (row-major, last index fastest):
 *   x, dt, z, y, yf, yb : [batch][seqlen][d_inner]
 *   B_f, C_f, B_b, C_b  : [batch][seqlen][d_state]
 *   A_f, A_b            : [d_inner][d_state]
 *   D_f, D_b, dt_bias_* : [d_inner]
 *   conv w_f, w_b       : [d_inner][K];  conv cb_f, cb_b : [d_inner]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(v) = log(1 + exp(v)), evaluated without overflow and without a threshold. */
double vimscan_oracle_softplus(double v) {
    if (v > 0.0) return v + log1p(exp(-v));
    return log1p(exp(v));
}

/* silu(v) = v * sigmoid(v) = v / (1 + exp(-v)). */
double vimscan_oracle_silu(double v) { return v / (1.0 + exp(-v)); }

/* One direction over one (b, d) channel. step = +1 (forward) or -1 (backward).
 * x is the direction's input (the shared x, or its convolved u). out[t] receives that
 * direction's readout at the natural index t. */
static void scan_one_direction(const double* x, const double* dt, const double* Bm, const double* Cm,
                               const double* A, double Dd, double dt_bias, int64_t b, int64_t d,
                               int64_t L, int64_t Di, int64_t N, int64_t seg_len, int step,
                               double* h, double* out) {
    for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
    for (int64_t k = 0; k < L; ++k) {
        const int64_t t = (step > 0) ? k : (L - 1 - k);
        if (seg_len > 0) {
            const int64_t entry = (step > 0) ? t : (t + 1);
            if (entry % seg_len == 0) {
                for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
            }
        }
        const double xt = x[(b * L + t) * Di + d];
        const double delta = vimscan_oracle_softplus(dt[(b * L + t) * Di + d] + dt_bias);
        const double* Bt = Bm + (b * L + t) * N;
        const double* Ct = Cm + (b * L + t) * N;
        double y = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double abar = exp(delta * A[d * N + n]);
            h[n] = abar * h[n] + delta * Bt[n] * xt;
            y += Ct[n] * h[n];
        }
        out[t] = y + Dd * xt;
    }
}

/* Returns 0 on success, -1 on a bad argument, -2 on allocation failure.
 * yf and yb may be NULL; when given they receive the two branch outputs. nthreads <= 0 uses
 * the OpenMP default. */
int vimscan_oracle_bidir_f64(const double* x, const double* dt, const double* z,
                             const double* B_f, const double* C_f, const double* B_b,
                             const double* C_b, const double* A_f, const double* A_b,
                             const double* D_f, const double* D_b, const double* dt_bias_f,
                             const double* dt_bias_b, int64_t batch, int64_t seqlen,
                             int64_t d_inner, int64_t d_state, int64_t seg_len, double* y,
                             double* yf, double* yb, int nthreads) {
    if (!x || !dt || !z || !B_f || !C_f || !B_b || !C_b || !A_f || !A_b || !D_f || !D_b ||
        !dt_bias_f || !dt_bias_b || !y)
        return -1;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0 || seg_len < 0) return -1;
    if (seg_len > 0 && seqlen % seg_len != 0) return -1;
    const int64_t B = batch, L = seqlen, Di = d_inner, N = d_state;
    if (B == 0 || L == 0 || Di == 0) return 0;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * (size_t)N);
        double* of = (double*)malloc(sizeof(double) * (size_t)L);
        double* ob = (double*)malloc(sizeof(double) * (size_t)L);
        const int ok = (h && of && ob);
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
        /* every thread reaches the worksharing loop; one without buffers skips its share */
#pragma omp for collapse(2) schedule(static)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t d = 0; d < Di; ++d) {
                if (!ok) continue;
                scan_one_direction(x, dt, B_f, C_f, A_f, D_f[d], dt_bias_f[d], b, d, L, Di, N,
                                   seg_len, +1, h, of);
                scan_one_direction(x, dt, B_b, C_b, A_b, D_b[d], dt_bias_b[d], b, d, L, Di, N,
                                   seg_len, -1, h, ob);
                for (int64_t t = 0; t < L; ++t) {
                    const int64_t i = (b * L + t) * Di + d;
                    y[i] = vimscan_oracle_silu(z[i]) * (of[t] + ob[t]);
                    if (yf) yf[i] = of[t];
                    if (yb) yb[i] = ob[t];
                }
            }
        }
        free(h);
        free(of);
        free(ob);
    }
    return err;
}

/* The directional convolution of one direction for every (b, t, d): u = silu(cb + taps . x),
 * with taps walking back from t (step = +1, forward: x[t], x[t-1], ...) or forward from t
 * (step = -1, backward: x[t], x[t+1], ...), zero outside t's segment. Returns 0 or -1. */
int vimscan_oracle_dirconv_f64(const double* x, const double* w, const double* cb, int64_t k,
                               int step, int64_t batch, int64_t seqlen, int64_t d_inner,
                               int64_t seg_len, double* u) {
    if (!x || !w || !cb || !u || k < 1 || (step != 1 && step != -1)) return -1;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || seg_len < 0) return -1;
    if (seg_len > 0 && seqlen % seg_len != 0) return -1;
    const int64_t L = seqlen, Di = d_inner, T = seg_len > 0 ? seg_len : seqlen;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t t = 0; t < L; ++t) {
            const int64_t seg0 = (t / T) * T; /* first token of t's segment */
            for (int64_t d = 0; d < Di; ++d) {
                double acc = cb[d];
                for (int64_t j = 0; j < k; ++j) {
                    const int64_t s = t - step * j; /* the token j steps behind t in walk order */
                    if (s < seg0 || s >= seg0 + T) continue;
                    acc += w[d * k + (k - 1 - j)] * x[(b * L + s) * Di + d];
                }
                u[(b * L + t) * Di + d] = vimscan_oracle_silu(acc);
            }
        }
    }
    return 0;
}

/* The bidirectional scan with the directional convolution in front of each direction (see the
 * header): y = silu(z) * (scan_f(u_f) + scan_b(u_b)). Returns 0, -1 or -2 as above. */
int vimscan_oracle_bidir_conv_f64(const double* x, const double* w_f, const double* cb_f,
                                  const double* w_b, const double* cb_b, int64_t k,
                                  const double* dt, const double* z, const double* B_f,
                                  const double* C_f, const double* B_b, const double* C_b,
                                  const double* A_f, const double* A_b, const double* D_f,
                                  const double* D_b, const double* dt_bias_f,
                                  const double* dt_bias_b, int64_t batch, int64_t seqlen,
                                  int64_t d_inner, int64_t d_state, int64_t seg_len, double* y,
                                  double* yf, double* yb, int nthreads) {
    if (!x || !w_f || !cb_f || !w_b || !cb_b || !dt || !z || !B_f || !C_f || !B_b || !C_b ||
        !A_f || !A_b || !D_f || !D_b || !dt_bias_f || !dt_bias_b || !y || k < 1)
        return -1;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0 || seg_len < 0) return -1;
    if (seg_len > 0 && seqlen % seg_len != 0) return -1;
    const int64_t B = batch, L = seqlen, Di = d_inner, N = d_state;
    if (B == 0 || L == 0 || Di == 0) return 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const size_t S = (size_t)(B * L * Di);
    double* u_f = (double*)malloc(sizeof(double) * S);
    double* u_b = (double*)malloc(sizeof(double) * S);
    int err = (u_f && u_b) ? 0 : -2;
    if (!err) err = vimscan_oracle_dirconv_f64(x, w_f, cb_f, k, +1, B, L, Di, seg_len, u_f);
    if (!err) err = vimscan_oracle_dirconv_f64(x, w_b, cb_b, k, -1, B, L, Di, seg_len, u_b);
    if (!err) {
#pragma omp parallel
        {
            double* h = (double*)malloc(sizeof(double) * (size_t)N);
            double* of = (double*)malloc(sizeof(double) * (size_t)L);
            double* ob = (double*)malloc(sizeof(double) * (size_t)L);
            const int ok = (h && of && ob);
            if (!ok) {
#pragma omp atomic write
                err = -2;
            }
#pragma omp for collapse(2) schedule(static)
            for (int64_t b = 0; b < B; ++b) {
                for (int64_t d = 0; d < Di; ++d) {
                    if (!ok) continue;
                    scan_one_direction(u_f, dt, B_f, C_f, A_f, D_f[d], dt_bias_f[d], b, d, L, Di,
                                       N, seg_len, +1, h, of);
                    scan_one_direction(u_b, dt, B_b, C_b, A_b, D_b[d], dt_bias_b[d], b, d, L, Di,
                                       N, seg_len, -1, h, ob);
                    for (int64_t t = 0; t < L; ++t) {
                        const int64_t i = (b * L + t) * Di + d;
                        y[i] = vimscan_oracle_silu(z[i]) * (of[t] + ob[t]);
                        if (yf) yf[i] = of[t];
                        if (yb) yb[i] = ob[t];
                    }
                }
            }
            free(h);
            free(of);
            free(ob);
        }
    }
    free(u_f);
    free(u_b);
    return err;
}

/* Unidirectional (forward) scan, gate, and the optional auxiliary swap. Returns 0, -1 or -2. */
int vimscan_oracle_fwd_f64(const double* x, const double* dt, const double* z, const double* Bm,
                           const double* Cm, const double* A, const double* D, const double* dt_bias,
                           int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                           int64_t seg_len, int swap, double* y, int nthreads) {
    if (!x || !dt || !z || !Bm || !Cm || !A || !D || !dt_bias || !y) return -1;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0 || seg_len < 0) return -1;
    if (seg_len > 0 && seqlen % seg_len != 0) return -1;
    const int64_t B = batch, L = seqlen, Di = d_inner, N = d_state;
    const int64_t T = seg_len > 0 ? seg_len : L;
    if (B == 0 || L == 0 || Di == 0) return 0;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * (size_t)N);
        double* of = (double*)malloc(sizeof(double) * (size_t)L);
        const int ok = (h && of);
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for collapse(2) schedule(static)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t d = 0; d < Di; ++d) {
                if (!ok) continue;
                scan_one_direction(x, dt, Bm, Cm, A, D[d], dt_bias[d], b, d, L, Di, N, seg_len, +1,
                                   h, of);
                for (int64_t t = 0; t < L; ++t) {
                    const int64_t first = (t / T) * T, last = first + T - 1;
                    int64_t dst = t;
                    if (swap && t == first) dst = last;
                    else if (swap && t == last) dst = first;
                    const int64_t i = (b * L + t) * Di + d;
                    y[(b * L + dst) * Di + d] = vimscan_oracle_silu(z[i]) * of[t];
                }
            }
        }
        free(h);
        free(of);
    }
    return err;
}

/* NC-SSD: y = C (B^T (X . m)) per sequence (segment). Returns 0, -1 (bad arguments) or -2 (no
   memory). H may be NULL. */
int vimscan_oracle_ncssd_f64(const double* x, const double* Bm, const double* Cm, const double* m,
                             int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                             int64_t seg_len, double* y, double* H, int nthreads) {
    if (!x || !Bm || !Cm || !m || !y) return -1;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0 || seg_len < 0) return -1;
    if (seg_len > 0 && seqlen % seg_len != 0) return -1;
    const int64_t Di = d_inner, N = d_state;
    const int64_t T = seg_len > 0 ? seg_len : seqlen;
    if (batch == 0 || seqlen == 0 || Di == 0) return 0;
    const int64_t S = batch * seqlen / T; /* sequences: token t of sequence s is stream row s*T+t */
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* xm = (double*)malloc(sizeof(double) * (size_t)T);
        double* h = (double*)malloc(sizeof(double) * (size_t)N);
        const int ok = (xm && h);
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for collapse(2) schedule(static)
        for (int64_t s = 0; s < S; ++s) {
            for (int64_t d = 0; d < Di; ++d) {
                if (!ok) continue;
                /* X . m: every token's input weighted by m_j */
                for (int64_t j = 0; j < T; ++j) xm[j] = x[(s * T + j) * Di + d] * m[s * T + j];
                /* H = B^T (X . m): the global state, one column (channel d) of it */
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < T; ++j) acc += Bm[(s * T + j) * N + n] * xm[j];
                    h[n] = acc;
                    if (H) H[(s * N + n) * Di + d] = acc;
                }
                /* Y = C H: every token reads the same state out with its own C row */
                for (int64_t i = 0; i < T; ++i) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) acc += Cm[(s * T + i) * N + n] * h[n];
                    y[(s * T + i) * Di + d] = acc;
                }
            }
        }
        free(xm);
        free(h);
    }
    return err;
}

/* Bidirectional scan in the token order of `order` ([batch * seqlen / T][T], every row a
   permutation of 0..T-1). Returns 0, -1 (bad arguments, including an order entry outside
   0..T-1) or -2 (no memory). */
int vimscan_oracle_bidir_order_f64(const double* x, const double* dt, const double* z,
                                   const double* B_f, const double* C_f, const double* B_b,
                                   const double* C_b, const double* A_f, const double* A_b,
                                   const double* D_f, const double* D_b, const double* dt_bias_f,
                                   const double* dt_bias_b, const int32_t* order, int64_t batch,
                                   int64_t seqlen, int64_t d_inner, int64_t d_state,
                                   int64_t seg_len, double* y, int nthreads) {
    if (!x || !dt || !z || !B_f || !C_f || !B_b || !C_b || !A_f || !A_b || !D_f || !D_b ||
        !dt_bias_f || !dt_bias_b || !order || !y)
        return -1;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0 || seg_len < 0) return -1;
    if (seg_len > 0 && seqlen % seg_len != 0) return -1;
    const int64_t Di = d_inner, N = d_state;
    const int64_t T = seg_len > 0 ? seg_len : seqlen;
    if (batch == 0 || seqlen == 0 || Di == 0) return 0;
    const int64_t S = batch * seqlen / T;
    for (int64_t i = 0; i < S * T; ++i)
        if (order[i] < 0 || order[i] >= T) return -1;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * (size_t)N);
        double* of = (double*)malloc(sizeof(double) * (size_t)T);
        double* ob = (double*)malloc(sizeof(double) * (size_t)T);
        const int ok = (h && of && ob);
        if (!ok) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for collapse(2) schedule(static)
        for (int64_t s = 0; s < S; ++s) {
            for (int64_t d = 0; d < Di; ++d) {
                if (!ok) continue;
                const int32_t* ord = order + s * T;
                for (int dir = 0; dir < 2; ++dir) {
                    const double* Bm = dir == 0 ? B_f : B_b;
                    const double* Cm = dir == 0 ? C_f : C_b;
                    const double* A = dir == 0 ? A_f : A_b;
                    const double Dd = dir == 0 ? D_f[d] : D_b[d];
                    const double bias = dir == 0 ? dt_bias_f[d] : dt_bias_b[d];
                    double* out = dir == 0 ? of : ob;
                    for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
                    for (int64_t k = 0; k < T; ++k) {
                        /* forward: the order's k-th token; backward: the same list from its end */
                        const int64_t t = ord[dir == 0 ? k : T - 1 - k];
                        const int64_t row = s * T + t;
                        const double xt = x[row * Di + d];
                        const double delta = vimscan_oracle_softplus(dt[row * Di + d] + bias);
                        double acc = 0.0;
                        for (int64_t n = 0; n < N; ++n) {
                            h[n] = exp(delta * A[d * N + n]) * h[n] + delta * Bm[row * N + n] * xt;
                            acc += Cm[row * N + n] * h[n];
                        }
                        out[t] = acc + Dd * xt;
                    }
                }
                for (int64_t t = 0; t < T; ++t) {
                    const int64_t i = (s * T + t) * Di + d;
                    y[i] = vimscan_oracle_silu(z[i]) * (of[t] + ob[t]);
                }
            }
        }
        free(h);
        free(of);
        free(ob);
    }
    return err;
}

/* Number of threads an OpenMP parallel region would use right now (for reporting). */
int vimscan_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
