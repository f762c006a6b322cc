/*
 * kda_oracle.c -- plain, slow, fp64 CPU oracle of the KDA token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library: it is written from the pages' definitions alone.
 *
 * Sources (cited by page title and panel; see the oracle's package docstring
 * for the full list):
 *   [CONV]  "Inside Kimi K3" (lei.chat), KDA short-convolution diagram
 *           (one channel c at token t, causal window of width 4).
 *   [KDA]   "Inside Kimi K3" (lei.chat), Kimi Delta Attention one-head
 *           diagram (projections, Swish + L2 norm, alpha/beta, recurrent
 *           state, read, head RMSNorm, sigmoid gate).
 *   [MEM]   "Animated Kimi K3 architecture diagram" (github.io), local-memory
 *           panel (fixed dk x dv state; probe, correct, decay, write).
 *
 * Every array is dense row-major fp64 and owned by the caller.  No function
 * allocates except the layer drivers, which use per-thread scratch.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_VERSION 1

int oracle_version(void) { return KDA_ORACLE_VERSION; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel loops that follow (timing runs on one core). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------------------
 * [CONV] Causal depthwise convolution of width 4 followed by SiLU.
 *
 * For one channel c the pre-activation at token t is the weighted sum of the
 * four most recent inputs x_{t-3}, x_{t-2}, x_{t-1}, x_t with weights
 * w0, w1, w2, w3 in that order; the output is SiLU(pre) = pre * sigmoid(pre).
 * Channels never mix; the sequence length is preserved by left padding.  The
 * padding is the caller's rolling state (the 3 previous raw inputs, oldest
 * first) or zeros when none is given.  state_out receives the last 3 raw
 * inputs of the window, which is what the next call (or decode step) needs.
 *
 *   x         [T][C]
 *   w         [C][4]      tap 0 multiplies x_{t-3}, tap 3 multiplies x_t
 *   state_in  [C][3] or NULL (zeros)
 *   y         [T][C]
 *   state_out [C][3] or NULL
 * ------------------------------------------------------------------------- */
static double padded_input(const double* x, int64_t C, const double* state_in,
                           int64_t tau, int64_t c) {
    if (tau >= 0) return x[tau * C + c];
    if (state_in == NULL) return 0.0;
    return state_in[c * 3 + (tau + 3)]; /* tau in {-3,-2,-1} -> slots 0,1,2 */
}

static double silu(double u) { return u / (1.0 + exp(-u)); }

void oracle_short_conv_silu(const double* x, int64_t T, int64_t C, const double* w,
                            const double* state_in, double* y, double* state_out) {
    for (int64_t c = 0; c < C; ++c) {
        for (int64_t t = 0; t < T; ++t) {
            double pre = 0.0;
            for (int64_t i = 0; i < 4; ++i)
                pre += w[c * 4 + i] * padded_input(x, C, state_in, t - 3 + i, c);
            y[t * C + c] = silu(pre);
        }
        if (state_out != NULL)
            for (int64_t j = 0; j < 3; ++j)
                state_out[c * 3 + j] = padded_input(x, C, state_in, T - 3 + j, c);
    }
}

/* ---------------------------------------------------------------------------
 * [KDA] L2 normalisation of q and k over the 128-d head vector:
 *   u <- u / sqrt(sum_d u_d^2 + eps)
 * u is [rows][D], normalised in place, one row per (token, head).
 * ------------------------------------------------------------------------- */
void oracle_l2norm_rows(double* u, int64_t rows, int64_t D, double eps) {
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int64_t d = 0; d < D; ++d) ss += u[r * D + d] * u[r * D + d];
        const double inv = 1.0 / sqrt(ss + eps);
        for (int64_t d = 0; d < D; ++d) u[r * D + d] *= inv;
    }
}

/* ---------------------------------------------------------------------------
 * [KDA][MEM] Gated delta rule for one head, token by token.
 *
 * State S is dk x dv (fixed shape).  For each token t:
 *   alpha_t = exp(clamp(g_t, -5, 0))        channel-wise retention; the pages
 *                                           bound the log-decay below by -5
 *   Sbar    = Diag(alpha_t) S_{t-1}          decay scales the key rows
 *   e_t     = v_t - Sbar^T k_t               probe the decayed memory, correct
 *   S_t     = Sbar + beta_t k_t e_t^T        write with strength beta_t
 *   o_t     = S_t^T q_t                      read after the write
 *
 *   q, k, g [T][DK]; v [T][DV]; beta [T]; S0 [DK][DV] or NULL (zeros)
 *   o [T][DV]; S [DK][DV] receives the final state
 *   snap_t[n_snap]: prefix lengths T' (1..T) at which a copy of S_{T'} is
 *   written to snaps[i][DK][DV]; pass n_snap = 0 for none.
 * Scratch: e[DV] allocated here (small).
 * ------------------------------------------------------------------------- */
void oracle_gated_delta_rule(const double* q, const double* k, const double* v,
                             const double* g, const double* beta, int64_t T,
                             int64_t DK, int64_t DV, const double* S0, double* o,
                             double* S, int64_t n_snap, const int64_t* snap_t,
                             double* snaps) {
    double* e = (double*)malloc(sizeof(double) * (size_t)DV);
    double* alpha = (double*)malloc(sizeof(double) * (size_t)DK);
    for (int64_t i = 0; i < DK * DV; ++i) S[i] = (S0 != NULL) ? S0[i] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
        const double* qt = q + t * DK;
        const double* kt = k + t * DK;
        const double* gt = g + t * DK;
        const double* vt = v + t * DV;
        for (int64_t i = 0; i < DK; ++i) {
            double gi = gt[i];
            if (gi < -5.0) gi = -5.0;
            if (gi > 0.0) gi = 0.0;
            alpha[i] = exp(gi);
        }
        /* decay */
        for (int64_t i = 0; i < DK; ++i)
            for (int64_t j = 0; j < DV; ++j) S[i * DV + j] *= alpha[i];
        /* probe + correct: e = v - Sbar^T k */
        for (int64_t j = 0; j < DV; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < DK; ++i) acc += S[i * DV + j] * kt[i];
            e[j] = vt[j] - acc;
        }
        /* write: S = Sbar + beta k e^T */
        for (int64_t i = 0; i < DK; ++i)
            for (int64_t j = 0; j < DV; ++j) S[i * DV + j] += beta[t] * kt[i] * e[j];
        /* read: o = S^T q */
        for (int64_t j = 0; j < DV; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < DK; ++i) acc += S[i * DV + j] * qt[i];
            o[t * DV + j] = acc;
        }
        for (int64_t s = 0; s < n_snap; ++s)
            if (snap_t[s] == t + 1)
                memcpy(snaps + s * DK * DV, S, sizeof(double) * (size_t)(DK * DV));
    }
    free(alpha);
    free(e);
}

/* ---------------------------------------------------------------------------
 * [KDA] Head RMSNorm times a full-rank sigmoid output gate:
 *   y_d = o_d / sqrt(mean_d o_d^2 + eps) * w_d * sigmoid(z_d)
 * o, z, y [rows][D]; w [D] shared by all heads.
 * ------------------------------------------------------------------------- */
void oracle_gated_rmsnorm(const double* o, const double* z, const double* w, int64_t rows,
                          int64_t D, double eps, double* y) {
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int64_t d = 0; d < D; ++d) ss += o[r * D + d] * o[r * D + d];
        const double inv = 1.0 / sqrt(ss / (double)D + eps);
        for (int64_t d = 0; d < D; ++d) {
            const double gate = 1.0 / (1.0 + exp(-z[r * D + d]));
            y[r * D + d] = o[r * D + d] * inv * w[d] * gate;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Layer driver: one KDA token mixer over packed sequences.
 *
 * Layout (token-major, as the pages draw the projected tensors [B,T,H,D]):
 *   x      [N][3*H*D]   projected q|k|v before the convolution; channel index
 *                        part*H*D + h*D + d with part 0=q, 1=k, 2=v
 *   w      [3*H*D][4]   conv filter banks (q bank, k bank, v bank)
 *   g      [N][H][D]    log-decay; beta [N][H]; gate [N][H][D]; norm_w [D]
 *   cu     [S+1]        sequence offsets into the N tokens (cu[0]=0)
 *   conv_state_in  [S][3*H*D][3] or NULL; conv_state_out same or NULL
 *   S0     [S][H][D][D] or NULL; S_final [S][H][D][D]
 * Outputs:
 *   y_qkv  [N][3*H*D]   conv + SiLU, then q and k L2-normalised per head
 *   o      [N][H][D]    recurrent read
 *   y      [N][H][D]    gated RMSNorm of o
 * n_snap/snap_t/snaps: per-sequence snapshots of S at prefix lengths,
 *   snaps[s][i][h][D][D]; pass n_snap = 0 for none.
 * Parallel over (sequence, channel) for the conv and over (sequence, head)
 * for the recurrence; each task is the plain sequential definition.
 * ------------------------------------------------------------------------- */
void oracle_kda_prefill(const double* x, const double* w, const double* g, const double* beta,
                        const double* gate, const double* norm_w, const int64_t* cu,
                        int64_t S, int64_t H, int64_t D, const double* conv_state_in,
                        double* conv_state_out, const double* S0, double* S_final,
                        double l2_eps, double rms_eps, double* y_qkv, double* o, double* y,
                        int64_t n_snap, const int64_t* snap_t, double* snaps) {
    const int64_t P = 3 * H * D;
    /* 1. conv + SiLU per (sequence, channel) */
#pragma omp parallel for collapse(2) schedule(dynamic, 64)
    for (int64_t s = 0; s < S; ++s) {
        for (int64_t c = 0; c < P; ++c) {
            const int64_t t0 = cu[s], T = cu[s + 1] - cu[s];
            double* xc = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
            double* yc = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
            for (int64_t t = 0; t < T; ++t) xc[t] = x[(t0 + t) * P + c];
            double st_in[3], st_out[3];
            const double* sin = NULL;
            if (conv_state_in != NULL) {
                for (int j = 0; j < 3; ++j) st_in[j] = conv_state_in[(s * P + c) * 3 + j];
                sin = st_in;
            }
            oracle_short_conv_silu(xc, T, 1, w + c * 4, sin, yc, st_out);
            for (int64_t t = 0; t < T; ++t) y_qkv[(t0 + t) * P + c] = yc[t];
            if (conv_state_out != NULL)
                for (int j = 0; j < 3; ++j) conv_state_out[(s * P + c) * 3 + j] = st_out[j];
            free(xc);
            free(yc);
        }
    }
    /* 2..4. per (sequence, head): L2(q,k), recurrence, gated norm */
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t s = 0; s < S; ++s) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t t0 = cu[s], T = cu[s + 1] - cu[s];
            const size_t n = (size_t)(T > 0 ? T : 1) * (size_t)D;
            double* qh = (double*)malloc(sizeof(double) * n);
            double* kh = (double*)malloc(sizeof(double) * n);
            double* vh = (double*)malloc(sizeof(double) * n);
            double* gh = (double*)malloc(sizeof(double) * n);
            double* bh = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
            double* oh = (double*)malloc(sizeof(double) * n);
            double* zh = (double*)malloc(sizeof(double) * n);
            double* yh = (double*)malloc(sizeof(double) * n);
            double* Sh = (double*)malloc(sizeof(double) * (size_t)(D * D));
            double* snap_h = n_snap > 0 ? (double*)malloc(sizeof(double) * (size_t)(n_snap * D * D)) : NULL;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t row = (t0 + t) * P;
                for (int64_t d = 0; d < D; ++d) {
                    qh[t * D + d] = y_qkv[row + 0 * H * D + h * D + d];
                    kh[t * D + d] = y_qkv[row + 1 * H * D + h * D + d];
                    vh[t * D + d] = y_qkv[row + 2 * H * D + h * D + d];
                    gh[t * D + d] = g[((t0 + t) * H + h) * D + d];
                    zh[t * D + d] = gate[((t0 + t) * H + h) * D + d];
                }
                bh[t] = beta[(t0 + t) * H + h];
            }
            oracle_l2norm_rows(qh, T, D, l2_eps);
            oracle_l2norm_rows(kh, T, D, l2_eps);
            /* write the normalised q, k back into y_qkv (the conv stage output) */
            for (int64_t t = 0; t < T; ++t) {
                const int64_t row = (t0 + t) * P;
                for (int64_t d = 0; d < D; ++d) {
                    y_qkv[row + 0 * H * D + h * D + d] = qh[t * D + d];
                    y_qkv[row + 1 * H * D + h * D + d] = kh[t * D + d];
                }
            }
            const double* S0h = S0 != NULL ? S0 + (s * H + h) * D * D : NULL;
            oracle_gated_delta_rule(qh, kh, vh, gh, bh, T, D, D, S0h, oh, Sh, n_snap, snap_t,
                                    snap_h);
            oracle_gated_rmsnorm(oh, zh, norm_w, T, D, rms_eps, yh);
            for (int64_t t = 0; t < T; ++t)
                for (int64_t d = 0; d < D; ++d) {
                    o[((t0 + t) * H + h) * D + d] = oh[t * D + d];
                    y[((t0 + t) * H + h) * D + d] = yh[t * D + d];
                }
            memcpy(S_final + (s * H + h) * D * D, Sh, sizeof(double) * (size_t)(D * D));
            for (int64_t i = 0; i < n_snap; ++i)
                memcpy(snaps + ((s * n_snap + i) * H + h) * D * D, snap_h + i * D * D,
                       sizeof(double) * (size_t)(D * D));
            free(qh); free(kh); free(vh); free(gh); free(bh);
            free(oh); free(zh); free(yh); free(Sh); free(snap_h);
        }
    }
}

/* ---------------------------------------------------------------------------
 * [CONV][KDA][MEM] One decode step for B sequences (one new token each).
 *
 * The conv window for channel c is [conv_state (3, oldest first), x_t]; after
 * the step the state holds the 3 most recent raw inputs [x_{t-2}, x_{t-1}, x_t].
 * Then SiLU, L2(q, k) per head, and one gated-delta-rule step on S (in place).
 *   x [B][3*H*D]; w [3*H*D][4]; conv_state [B][3*H*D][3] (in place)
 *   g [B][H][D]; beta [B][H]; state [B][H][D][D] (in place); o [B][H][D]
 * ------------------------------------------------------------------------- */
void oracle_kda_decode_step(const double* x, const double* w, double* conv_state,
                            const double* g, const double* beta, double* state, double* o,
                            int64_t B, int64_t H, int64_t D, double l2_eps) {
    const int64_t P = 3 * H * D;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            double* u = (double*)malloc(sizeof(double) * (size_t)(3 * D));
            for (int64_t part = 0; part < 3; ++part) {
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t c = part * H * D + h * D + d;
                    double* st = conv_state + (b * P + c) * 3;
                    double xt = x[b * P + c];
                    double y1;
                    /* the window is a length-1 sequence with the rolling state
                       as its left padding */
                    double st_out[3];
                    oracle_short_conv_silu(&xt, 1, 1, w + c * 4, st, &y1, st_out);
                    for (int j = 0; j < 3; ++j) st[j] = st_out[j];
                    u[part * D + d] = y1;
                }
            }
            oracle_l2norm_rows(u + 0 * D, 1, D, l2_eps);
            oracle_l2norm_rows(u + 1 * D, 1, D, l2_eps);
            double* Sb = state + (b * H + h) * D * D;
            double* Snew = (double*)malloc(sizeof(double) * (size_t)(D * D));
            oracle_gated_delta_rule(u + 0 * D, u + 1 * D, u + 2 * D, g + (b * H + h) * D,
                                    beta + b * H + h, 1, D, D, Sb, o + (b * H + h) * D, Snew,
                                    0, NULL, NULL);
            memcpy(Sb, Snew, sizeof(double) * (size_t)(D * D));
            free(Snew);
            free(u);
        }
    }
}
