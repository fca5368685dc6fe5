/*
 * gdn_oracle.c -- plain fp64 CPU oracle of the Gated DeltaNet layer core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP product path
 * never links, loads or calls it, and it shares no code with that path: only
 * the seeded input arrays are common to both.
 *
 * Everything is computed in double precision with plain loops, in the order
 * the definitions state, so a reader can check each step by eye.
 *
 * Sources (page titles as cited throughout):
 *   [GDN]   Gated DeltaNet, as named by the method statement of this project:
 *           width-4 depthwise causal conv with SiLU over q/k/v, L2-normalised
 *           q/k, decay g = -exp(A_log) * softplus(a + dt_bias), beta =
 *           sigmoid(b), the gated delta rule and its chunked WY/UT form.
 *   [R924]  "r9700-stack v0.2.4: one GDN state page per request", section
 *           "What it does" (replay of accepted candidate rows from a one-page
 *           record, bit-identical to per-candidate slot pages).
 *   [R923]  "r9700-stack v0.2.3: first token in half the time", section
 *           "1. Time to first token: the GDN prefill core" (token-by-token
 *           core, fp64 token-by-token reference, chunked form).
 *
 * Readings where the sources leave a step open (each also listed in the
 * design notes of the repository):
 *   - state S is d_k x d_v; the step is S_t = e^{g_t} (I - b_t k_t k_t^T) S_{t-1}
 *     + b_t k_t v_t^T and o_t = scale * S_t^T q_t (the transposed form of the
 *     published d_v x d_k recurrence; the same linear map);
 *   - L2 norm x / sqrt(sum x^2 + eps);
 *   - v-head h reads key head h / (H_v / H_k);
 *   - conv tap w[c][W-1] multiplies the newest row, no bias, SiLU on every
 *     q/k/v channel; window rows are stored oldest first;
 *   - a speculative acceptance a counts accepted drafts, so 1 + a candidate
 *     rows are committed;
 *   - a bf16 state is rounded (nearest-even) once per verify step, when the
 *     committed state is stored;
 *   - a verify page's flag word holds the live record slot (bit 0), the
 *     parity of the step that wrote it (bit 1) and a done counter (bits
 *     8..31, zero between steps); the conv buffer holds W-1 + n_spec rows and
 *     a step's window is rows a..a+W-2, a the replayed acceptance
 *     (ora_book_step).
 *
 * Parity pins (tests/test_oracle.py): every function below is pinned by
 * closed forms, special cases and brute-force cross-checks; none is pinned
 * only against itself.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t h_k, h_v, d_k, d_v, conv_w;
    double scale, l2_eps;
} ora_dims;

static int64_t c_conv(const ora_dims* d) {
    return 2 * (int64_t)d->h_k * d->d_k + (int64_t)d->h_v * d->d_v;
}

/* ---------------------------------------------------------------- scalars */

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z})                        [GDN] (a) */
double ora_silu(double z) { return z / (1.0 + exp(-z)); }

/* softplus(u) = log(1 + e^u), written so neither branch overflows     [GDN] (b) */
double ora_softplus(double u) {
    if (u > 0.0) return u + log1p(exp(-u));
    return log1p(exp(u));
}

/* sigmoid(b) = 1 / (1 + e^{-b})                                        [GDN] (b) */
double ora_sigmoid(double b) { return 1.0 / (1.0 + exp(-b)); }

/* decay g = -exp(A_log) * softplus(a + dt_bias)                         [GDN] (b) */
double ora_decay(double a, double a_log, double dt_bias) {
    return -exp(a_log) * ora_softplus(a + dt_bias);
}

/* Round to the nearest bf16 value (8 significant bits), ties to even.
 * Used only for the bf16 state variant of speculative verify.             */
double ora_round_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    double ax = fabs(x);
    if (ax < ldexp(1.0, -126)) {               /* bf16 subnormal range: step 2^-133 */
        return nearbyint(ldexp(x, 133)) * ldexp(1.0, -133);
    }
    int e;
    double m = frexp(x, &e);                   /* x = m * 2^e, 0.5 <= |m| < 1 */
    return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

void ora_round_bf16_array(double* x, int64_t n) {
    for (int64_t i = 0; i < n; ++i) x[i] = ora_round_bf16(x[i]);
}

/* ------------------------------------------------------------------- conv */

/*
 * Depthwise causal conv of one sequence, every channel independent   [GDN] (a):
 *   z_t[c] = sum_{j=0}^{W-1} w[c][j] * X_{t-(W-1)+j}[c],   y = SiLU(z) if act
 * where X_r = x[r] for r >= 0 and X_r = window row (W-1)+r for r < 0
 * (window rows oldest first; a NULL window means zeros).
 * win_out receives the last W-1 rows of (window ++ x), the rolling window.
 */
void ora_conv_seq(int32_t T, int32_t C, int32_t W, const double* x, const double* w,
                  const double* win_in, int32_t act, double* y, double* win_out) {
    for (int32_t c = 0; c < C; ++c) {
        for (int32_t t = 0; t < T; ++t) {
            double z = 0.0;
            for (int32_t j = 0; j < W; ++j) {
                int32_t r = t - (W - 1) + j;
                double xr;
                if (r >= 0) xr = x[(int64_t)r * C + c];
                else xr = win_in ? win_in[(int64_t)((W - 1) + r) * C + c] : 0.0;
                z += w[(int64_t)c * W + j] * xr;
            }
            y[(int64_t)t * C + c] = act ? ora_silu(z) : z;
        }
        if (win_out) {
            for (int32_t j = 0; j < W - 1; ++j) {
                int32_t r = T - (W - 1) + j;
                double xr;
                if (r >= 0) xr = x[(int64_t)r * C + c];
                else xr = win_in ? win_in[(int64_t)((W - 1) + r) * C + c] : 0.0;
                win_out[(int64_t)j * C + c] = xr;
            }
        }
    }
}

/*
 * fp32 operation-order model of the conv without activation: acc starts at
 * 0 and takes one fused multiply-add per tap, oldest tap first.  This fixes
 * the exact bits a single-precision conv with that order must produce; it is
 * pinned against ora_conv_seq within fp32 rounding.
 */
void ora_conv_f32_model(int32_t T, int32_t C, int32_t W, const float* x, const float* w,
                        const float* win_in, float* y) {
    for (int32_t c = 0; c < C; ++c) {
        for (int32_t t = 0; t < T; ++t) {
            float acc = 0.0f;
            for (int32_t j = 0; j < W; ++j) {
                int32_t r = t - (W - 1) + j;
                float xr;
                if (r >= 0) xr = x[(int64_t)r * C + c];
                else xr = win_in ? win_in[(int64_t)((W - 1) + r) * C + c] : 0.0f;
                acc = fmaf(w[(int64_t)c * W + j], xr, acc);
            }
            y[(int64_t)t * C + c] = acc;
        }
    }
}

/* ----------------------------------------------------------------- gating */

/*
 * Post-conv gating of one token row y (C_conv channels, [q | k | v]) [GDN] (b):
 *   q_i <- q_i / sqrt(|q_i|^2 + eps), k_i likewise, per key head i;
 *   g_h = -exp(A_log[h]) softplus(a_h + dt_bias[h]);  beta_h = sigmoid(b_h).
 * Outputs qn, kn [H_k][d_k], v [H_v][d_v], g, beta [H_v].
 */
void ora_gate_row(const ora_dims* d, const double* y, const double* a, const double* b,
                  const double* a_log, const double* dt_bias, double* qn, double* kn,
                  double* v, double* g, double* beta) {
    const int64_t qk = (int64_t)d->h_k * d->d_k;
    for (int32_t i = 0; i < d->h_k; ++i) {
        const double* q = y + (int64_t)i * d->d_k;
        const double* k = y + qk + (int64_t)i * d->d_k;
        double sq = 0.0, sk = 0.0;
        for (int32_t e = 0; e < d->d_k; ++e) { sq += q[e] * q[e]; sk += k[e] * k[e]; }
        double nq = sqrt(sq + d->l2_eps), nk = sqrt(sk + d->l2_eps);
        for (int32_t e = 0; e < d->d_k; ++e) {
            qn[(int64_t)i * d->d_k + e] = q[e] / nq;
            kn[(int64_t)i * d->d_k + e] = k[e] / nk;
        }
    }
    memcpy(v, y + 2 * qk, sizeof(double) * (size_t)d->h_v * d->d_v);
    for (int32_t h = 0; h < d->h_v; ++h) {
        g[h] = ora_decay(a[h], a_log[h], dt_bias[h]);
        beta[h] = ora_sigmoid(b[h]);
    }
}

/* ------------------------------------------------------- the delta rule */

/*
 * Gated delta rule, token by token, for one value head               [GDN] (c):
 *   S_t = e^{g_t} (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *   o_t = scale * S_t^T q_t
 * S is d_k x d_v row-major and is updated in place.  q, k are T x dk with row
 * stride qk_stride, v and o are T x dv with row strides v_stride / o_stride.
 * The step is written as the matrix product it is: P = k^T S, then
 * S <- e^g (S - beta k P) + beta k v^T.
 */
void ora_delta_rule(int32_t T, int32_t dk, int32_t dv, double scale, const double* q,
                    const double* k, int64_t qk_stride, const double* v, int64_t v_stride,
                    const double* g, const double* beta, double* S, double* o,
                    int64_t o_stride) {
    double* P = (double*)malloc(sizeof(double) * (size_t)dv);
    for (int32_t t = 0; t < T; ++t) {
        const double* kt = k + (int64_t)t * qk_stride;
        const double* qt = q + (int64_t)t * qk_stride;
        const double* vt = v + (int64_t)t * v_stride;
        double eg = exp(g[t]), bt = beta[t];
        for (int32_t j = 0; j < dv; ++j) {
            double p = 0.0;
            for (int32_t i = 0; i < dk; ++i) p += kt[i] * S[(int64_t)i * dv + j];
            P[j] = p;
        }
        for (int32_t i = 0; i < dk; ++i)
            for (int32_t j = 0; j < dv; ++j)
                S[(int64_t)i * dv + j] =
                    eg * (S[(int64_t)i * dv + j] - bt * kt[i] * P[j]) + bt * kt[i] * vt[j];
        if (o) {
            for (int32_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int32_t i = 0; i < dk; ++i) acc += S[(int64_t)i * dv + j] * qt[i];
                o[(int64_t)t * o_stride + j] = scale * acc;
            }
        }
    }
    free(P);
}

/*
 * Chunked WY/UT form of the same recurrence for one value head       [GDN] (c),
 * chunk length C (the last chunk may be shorter).  Within a chunk of n rows,
 * with chunk-local cumulative decay G_i = sum_{j<=i} g_j and start state S0:
 *   1. A_ij = beta_i e^{G_i - G_j} (k_i . k_j) for i > j, else 0 (masked
 *      before the exponential, so only non-positive exponents occur);
 *   2. T = (I + A)^{-1} by forward substitution (unit lower triangular);
 *   3. W = T diag(beta e^{G}) K,  U = T diag(beta) V;
 *   4. D = U - W S0;
 *   5. O = scale [ diag(e^{G}) Q S0 + (tril(Q K^T) o e^{G_i - G_j}) D ];
 *   6. S_next = e^{G_{n-1}} S0 + (diag(e^{G_{n-1} - G}) K)^T D.
 * Used only to pin the equivalence of the two forms of the method.
 */
void ora_chunked_rule(int32_t T, int32_t dk, int32_t dv, int32_t C, double scale,
                      const double* q, const double* k, int64_t qk_stride, const double* v,
                      int64_t v_stride, const double* g, const double* beta, double* S,
                      double* o, int64_t o_stride) {
    double* G = (double*)malloc(sizeof(double) * (size_t)C);
    double* A = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* Tm = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* Wm = (double*)malloc(sizeof(double) * (size_t)C * dk);
    double* Um = (double*)malloc(sizeof(double) * (size_t)C * dv);
    double* D = (double*)malloc(sizeof(double) * (size_t)C * dv);
    double* Sn = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    for (int32_t c0 = 0; c0 < T; c0 += C) {
        const int32_t n = (T - c0 < C) ? (T - c0) : C;
        const double* K = k + (int64_t)c0 * qk_stride;
        const double* Q = q + (int64_t)c0 * qk_stride;
        const double* V = v + (int64_t)c0 * v_stride;
        const double* gc = g + c0;
        const double* bc = beta + c0;
        double run = 0.0;
        for (int32_t i = 0; i < n; ++i) { run += gc[i]; G[i] = run; }
        /* 1. A */
        for (int32_t i = 0; i < n; ++i)
            for (int32_t j = 0; j < n; ++j) {
                double aij = 0.0;
                if (i > j) {
                    double kk = 0.0;
                    for (int32_t e = 0; e < dk; ++e)
                        kk += K[(int64_t)i * qk_stride + e] * K[(int64_t)j * qk_stride + e];
                    aij = bc[i] * exp(G[i] - G[j]) * kk;
                }
                A[(int64_t)i * n + j] = aij;
            }
        /* 2. T = (I + A)^{-1}: solve (I + A) T = I row by row */
        for (int32_t i = 0; i < n; ++i)
            for (int32_t j = 0; j < n; ++j) {
                double t = (i == j) ? 1.0 : 0.0;
                for (int32_t m = 0; m < i; ++m) t -= A[(int64_t)i * n + m] * Tm[(int64_t)m * n + j];
                Tm[(int64_t)i * n + j] = t;
            }
        /* 3. W, U */
        for (int32_t i = 0; i < n; ++i) {
            for (int32_t e = 0; e < dk; ++e) {
                double acc = 0.0;
                for (int32_t m = 0; m < n; ++m)
                    acc += Tm[(int64_t)i * n + m] * bc[m] * exp(G[m]) * K[(int64_t)m * qk_stride + e];
                Wm[(int64_t)i * dk + e] = acc;
            }
            for (int32_t e = 0; e < dv; ++e) {
                double acc = 0.0;
                for (int32_t m = 0; m < n; ++m)
                    acc += Tm[(int64_t)i * n + m] * bc[m] * V[(int64_t)m * v_stride + e];
                Um[(int64_t)i * dv + e] = acc;
            }
        }
        /* 4. D = U - W S0 */
        for (int32_t i = 0; i < n; ++i)
            for (int32_t e = 0; e < dv; ++e) {
                double ws = 0.0;
                for (int32_t m = 0; m < dk; ++m) ws += Wm[(int64_t)i * dk + m] * S[(int64_t)m * dv + e];
                D[(int64_t)i * dv + e] = Um[(int64_t)i * dv + e] - ws;
            }
        /* 5. O */
        if (o) {
            for (int32_t i = 0; i < n; ++i)
                for (int32_t e = 0; e < dv; ++e) {
                    double qs = 0.0;
                    for (int32_t m = 0; m < dk; ++m) qs += Q[(int64_t)i * qk_stride + m] * S[(int64_t)m * dv + e];
                    double acc = exp(G[i]) * qs;
                    for (int32_t j = 0; j <= i; ++j) {
                        double qkij = 0.0;
                        for (int32_t m = 0; m < dk; ++m)
                            qkij += Q[(int64_t)i * qk_stride + m] * K[(int64_t)j * qk_stride + m];
                        acc += qkij * exp(G[i] - G[j]) * D[(int64_t)j * dv + e];
                    }
                    o[(int64_t)(c0 + i) * o_stride + e] = scale * acc;
                }
        }
        /* 6. state at the end of the chunk */
        for (int32_t m = 0; m < dk; ++m)
            for (int32_t e = 0; e < dv; ++e) {
                double acc = exp(G[n - 1]) * S[(int64_t)m * dv + e];
                for (int32_t j = 0; j < n; ++j)
                    acc += exp(G[n - 1] - G[j]) * K[(int64_t)j * qk_stride + m] * D[(int64_t)j * dv + e];
                Sn[(int64_t)m * dv + e] = acc;
            }
        memcpy(S, Sn, sizeof(double) * (size_t)dk * dv);
    }
    free(G); free(A); free(Tm); free(Wm); free(Um); free(D); free(Sn);
}

/* ----------------------------------------------- one sequence, all heads */

/* Per-token gated quantities of one sequence: conv, then gating of each row. */
typedef struct {
    double *qn, *kn, *v, *g, *beta;  /* [T][H_k d_k], [T][H_k d_k], [T][H_v d_v], [T][H_v] x2 */
} gated_seq;

static void gate_sequence(const ora_dims* d, int32_t T, const double* conv_w,
                          const double* a_log, const double* dt_bias, const double* x,
                          const double* a, const double* b, const double* win_in,
                          double* win_out, gated_seq* gs) {
    const int64_t C = c_conv(d);
    const int64_t qk = (int64_t)d->h_k * d->d_k, vv = (int64_t)d->h_v * d->d_v;
    double* y = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * C);
    ora_conv_seq(T, (int32_t)C, d->conv_w, x, conv_w, win_in, 1, y, win_out);
    gs->qn = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * qk);
    gs->kn = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * qk);
    gs->v = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * vv);
    gs->g = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * d->h_v);
    gs->beta = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * d->h_v);
    for (int32_t t = 0; t < T; ++t)
        ora_gate_row(d, y + (int64_t)t * C, a + (int64_t)t * d->h_v, b + (int64_t)t * d->h_v,
                     a_log, dt_bias, gs->qn + t * qk, gs->kn + t * qk, gs->v + t * vv,
                     gs->g + (int64_t)t * d->h_v, gs->beta + (int64_t)t * d->h_v);
    free(y);
}

static void free_gated(gated_seq* gs) {
    free(gs->qn); free(gs->kn); free(gs->v); free(gs->g); free(gs->beta);
}

/* Run value head h of one gated sequence, token by token (chunk == 0) or in
 * the chunked WY/UT form (chunk > 0). */
static void run_head(const ora_dims* d, int32_t T, const gated_seq* gs, int32_t h, int32_t chunk,
                     double* S, double* o, int64_t o_stride) {
    const int32_t r = d->h_v / d->h_k;
    const int32_t i = h / r;
    const int64_t qk = (int64_t)d->h_k * d->d_k, vv = (int64_t)d->h_v * d->d_v;
    double* gh = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double* bh = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int32_t t = 0; t < T; ++t) {
        gh[t] = gs->g[(int64_t)t * d->h_v + h];
        bh[t] = gs->beta[(int64_t)t * d->h_v + h];
    }
    const double* q = gs->qn + (int64_t)i * d->d_k;
    const double* k = gs->kn + (int64_t)i * d->d_k;
    const double* v = gs->v + (int64_t)h * d->d_v;
    if (chunk > 0)
        ora_chunked_rule(T, d->d_k, d->d_v, chunk, d->scale, q, k, qk, v, vv, gh, bh, S, o, o_stride);
    else
        ora_delta_rule(T, d->d_k, d->d_v, d->scale, q, k, qk, v, vv, gh, bh, S, o, o_stride);
    free(gh); free(bh);
}

/*
 * The whole layer core over a ragged batch (token by token when chunk == 0,
 * chunked WY/UT form otherwise).
 *   x      [N][C_conv]  pre-conv rows, sequences packed by cu_seqlens
 *   a, b   [N][H_v]
 *   win    [n_seqs][W-1][C_conv]    initial window in, rolled window out
 *   S      [n_seqs][H_v][d_k][d_v]  initial state in, final state out
 *   o      [N][H_v][d_v]
 *   has_init[s] == 0 means the sequence starts from a zero window and state.
 *   head_sel (optional, [n_seqs][H_v]): heads with 0 are skipped (their S and
 *   o are left untouched), for spot checks of large workloads.
 */
int ora_layer(const ora_dims* d, const double* conv_w, const double* a_log,
              const double* dt_bias, const double* x, const double* a, const double* b,
              const int32_t* cu_seqlens, int32_t n_seqs, const uint8_t* has_init,
              double* win, double* S, double* o, int32_t chunk, const uint8_t* head_sel) {
    if (d->h_v % d->h_k != 0) return 1;
    const int64_t C = c_conv(d);
    const int64_t hs = (int64_t)d->d_k * d->d_v;
    const int64_t ws = (int64_t)(d->conv_w - 1) * C;
    for (int32_t s = 0; s < n_seqs; ++s) {
        const int32_t r0 = cu_seqlens[s], T = cu_seqlens[s + 1] - cu_seqlens[s];
        const int init = has_init ? has_init[s] : 1;
        if (!init) {
            memset(win + s * ws, 0, sizeof(double) * (size_t)ws);
            memset(S + s * (int64_t)d->h_v * hs, 0, sizeof(double) * (size_t)(d->h_v * hs));
        }
        double* wprev = (double*)malloc(sizeof(double) * (size_t)ws);
        memcpy(wprev, win + s * ws, sizeof(double) * (size_t)ws);
        gated_seq gs;
        gate_sequence(d, T, conv_w, a_log, dt_bias, x + (int64_t)r0 * C, a + (int64_t)r0 * d->h_v,
                      b + (int64_t)r0 * d->h_v, wprev, win + s * ws, &gs);
        free(wprev);
#pragma omp parallel for schedule(dynamic, 1)
        for (int32_t h = 0; h < d->h_v; ++h) {
            if (head_sel && !head_sel[(int64_t)s * d->h_v + h]) continue;
            run_head(d, T, &gs, h, chunk, S + ((int64_t)s * d->h_v + h) * hs,
                     o + (int64_t)r0 * d->h_v * d->d_v + (int64_t)h * d->d_v,
                     (int64_t)d->h_v * d->d_v);
        }
        free_gated(&gs);
    }
    return 0;
}

/* Conv update on its own over a ragged batch (activation optional).
 * win [n_seqs][W-1][C] in/out, y [N][C]. */
int ora_conv_update(int32_t C, int32_t W, const double* conv_w, const double* x,
                    const int32_t* cu_seqlens, int32_t n_seqs, const uint8_t* has_init,
                    double* win, int32_t act, double* y) {
    const int64_t ws = (int64_t)(W - 1) * C;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t s = 0; s < n_seqs; ++s) {
        const int32_t r0 = cu_seqlens[s], T = cu_seqlens[s + 1] - cu_seqlens[s];
        const int init = has_init ? has_init[s] : 1;
        double* wprev = (double*)calloc((size_t)ws, sizeof(double));
        if (init) memcpy(wprev, win + s * ws, sizeof(double) * (size_t)ws);
        ora_conv_seq(T, C, W, x + (int64_t)r0 * C, conv_w, wprev, act, y + (int64_t)r0 * C,
                     win + s * ws);
        free(wprev);
    }
    return 0;
}

/* --------------------------------------------------- speculative verify */

/*
 * Semantics of speculative verify, independent of how pages are laid out
 * [R924, "What it does"].  For each request and step s, the candidates
 * c_0 .. c_{n-1} continue the committed stream in order; o^{(s)}_i is the
 * layer output at c_i on (committed stream ++ c_0 .. c_i).  Afterwards
 * 1 + accepted[s][r] rows are committed: the committed state and window
 * become those after candidate accepted[s][r].  With state_bf16, the
 * committed state is rounded to bf16 each time it is committed.
 *   x [n_steps][n_req][n_cand][C], a, b [n_steps][n_req][n_cand][H_v]
 *   win [n_req][W-1][C], S [n_req][H_v][d_k][d_v] (in: start; out: committed)
 *   o [n_steps][n_req][n_cand][H_v][d_v]
 */
int ora_verify(const ora_dims* d, const double* conv_w, const double* a_log,
               const double* dt_bias, int32_t n_req, int32_t n_steps, int32_t n_cand,
               const double* x, const double* a, const double* b, const int32_t* accepted,
               int32_t state_bf16, double* win, double* S, double* o) {
    if (d->h_v % d->h_k != 0) return 1;
    const int64_t C = c_conv(d);
    const int64_t hs = (int64_t)d->d_k * d->d_v, Sreq = (int64_t)d->h_v * hs;
    const int64_t ws = (int64_t)(d->conv_w - 1) * C;
    const int64_t ov = (int64_t)d->h_v * d->d_v;
    for (int64_t i = 0; i < (int64_t)n_steps * n_req; ++i)
        if (accepted[i] < 0 || accepted[i] >= n_cand) return 2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < n_req; ++r) {
        double* Srun = (double*)malloc(sizeof(double) * (size_t)Sreq);
        double* Sacc = (double*)malloc(sizeof(double) * (size_t)Sreq);
        double* wnext = (double*)malloc(sizeof(double) * (size_t)ws);
        for (int32_t s = 0; s < n_steps; ++s) {
            const int64_t row0 = ((int64_t)s * n_req + r) * n_cand;
            const int32_t acc = accepted[(int64_t)s * n_req + r];
            double* wr = win + r * ws;
            /* conv + gating of the candidate block continuing the committed window */
            gated_seq gs;
            gate_sequence(d, n_cand, conv_w, a_log, dt_bias, x + row0 * C, a + row0 * d->h_v,
                          b + row0 * d->h_v, wr, NULL, &gs);
            /* committed window after candidate acc: last W-1 rows of (window ++ c_0..c_acc) */
            {
                double* tmp = (double*)malloc(sizeof(double) * (size_t)(C * (acc + 1)));
                double* ydummy = (double*)malloc(sizeof(double) * (size_t)(C * (acc + 1)));
                memcpy(tmp, x + row0 * C, sizeof(double) * (size_t)(C * (acc + 1)));
                ora_conv_seq(acc + 1, (int32_t)C, d->conv_w, tmp, conv_w, wr, 0, ydummy, wnext);
                free(tmp); free(ydummy);
            }
            memcpy(Srun, S + r * Sreq, sizeof(double) * (size_t)Sreq);
            /* run candidates one at a time so the state after c_acc can be kept */
            for (int32_t i = 0; i < n_cand; ++i) {
                gated_seq gi;
                const int64_t qk = (int64_t)d->h_k * d->d_k;
                gi.qn = gs.qn + i * qk; gi.kn = gs.kn + i * qk; gi.v = gs.v + i * ov;
                gi.g = gs.g + (int64_t)i * d->h_v; gi.beta = gs.beta + (int64_t)i * d->h_v;
                for (int32_t h = 0; h < d->h_v; ++h)
                    run_head(d, 1, &gi, h, 0, Srun + h * hs,
                             o + (row0 + i) * ov + (int64_t)h * d->d_v, ov);
                if (i == acc) memcpy(Sacc, Srun, sizeof(double) * (size_t)Sreq);
            }
            if (state_bf16) ora_round_bf16_array(Sacc, Sreq);
            memcpy(S + r * Sreq, Sacc, sizeof(double) * (size_t)Sreq);
            memcpy(wr, wnext, sizeof(double) * (size_t)ws);
            free_gated(&gs);
        }
        free(Srun); free(Sacc); free(wnext);
    }
    return 0;
}

/* ------------------------------------------- page bookkeeping of verify */

/*
 * Bookkeeping of one speculative verify step for one request's page
 * [R924, "What it does": the two record slots and the flag word's three
 * fields; "A defect found and fixed before the tag": the conv buffer rolls
 * by the rows the record holds, not by a tensor's width].  Integers and data
 * movement only: nothing of the method's arithmetic happens here.
 *
 *   hdr[4]  = {flag, n_rows[0], n_rows[1], accepted}.  flag bit 0 is the
 *             live record slot L, bit 1 the parity P of the step that wrote
 *             the page, bits 8..31 a done counter that is 0 between steps.
 *             An all-zero header is a fresh page: slot 0 live, no rows.
 *   cbuf    = the request's conv buffer, `rows` rows of C channels, oldest
 *             first (values only moved, carried as doubles).
 *   x       = the step's n_cand pre-conv candidate rows [n_cand][C].
 *
 * The step is refused and nothing changes when its parity equals P (the
 * step was applied already: ORA_BOOK_PARITY), or when the live slot holds
 * rows and num_accepted is not one of them or the slot holds more than
 * n_spec + 1 rows (ORA_BOOK_ACCEPTED).  Otherwise, with a = num_accepted
 * when the live slot holds rows and a = 0 when it holds none:
 *   - the step replays rows 0..a of slot L (none when it holds no rows);
 *   - its conv window is cbuf rows a .. a+W-2;
 *   - cbuf becomes [rows a+1 .. a+W-2, x_0 .. x_{n_cand-1}] when n_cand > 0,
 *     [rows a .. a+W-2] when n_cand == 0; rows past those keep their values;
 *   - the candidates go to slot 1-L, and the header becomes
 *     {(1-L) | parity << 1, n_rows[1-L] = n_cand, n_rows[L] as it was,
 *     accepted = a}.
 * out (4 ints, optional): a, the number of replayed rows, the replayed slot
 * and the written slot.
 */
#define ORA_BOOK_ACCEPTED 1
#define ORA_BOOK_PARITY 2
#define ORA_BOOK_ARG 16

int ora_book_step(int32_t W, int32_t n_spec, int32_t C, int32_t rows, int32_t n_cand,
                  int32_t num_accepted, int32_t parity, uint32_t* hdr, double* cbuf,
                  const double* x, int32_t* out) {
    if (W < 2 || n_spec < 0 || C < 0 || rows < W - 1 + n_spec || n_cand < 0 || n_cand > n_spec + 1 ||
        (parity != 0 && parity != 1))
        return ORA_BOOK_ARG;
    const uint32_t flag = hdr[0];
    const int32_t L = (int32_t)(flag & 1u);
    const int32_t P = (int32_t)((flag >> 1) & 1u);
    const int32_t held = (int32_t)hdr[1 + L];
    if (parity == P) return ORA_BOOK_PARITY;
    int32_t a = 0;
    if (held > 0) {
        if (num_accepted < 0 || num_accepted >= held || held > n_spec + 1) return ORA_BOOK_ACCEPTED;
        a = num_accepted;
    }
    /* the window a .. a+W-2, read before any row is written */
    double* win = (double*)malloc(sizeof(double) * (size_t)(W - 1) * (size_t)(C > 0 ? C : 1));
    for (int32_t j = 0; j < W - 1; ++j)
        memcpy(win + (int64_t)j * C, cbuf + (int64_t)(a + j) * C, sizeof(double) * (size_t)C);
    if (n_cand > 0) {
        for (int32_t j = 0; j < W - 2; ++j)
            memcpy(cbuf + (int64_t)j * C, win + (int64_t)(j + 1) * C, sizeof(double) * (size_t)C);
        memcpy(cbuf + (int64_t)(W - 2) * C, x, sizeof(double) * (size_t)n_cand * (size_t)C);
    } else {
        memcpy(cbuf, win, sizeof(double) * (size_t)(W - 1) * (size_t)C);
    }
    free(win);
    hdr[0] = (uint32_t)(1 - L) | ((uint32_t)parity << 1);
    hdr[1 + (1 - L)] = (uint32_t)n_cand;
    hdr[3] = (uint32_t)a;
    if (out) {
        out[0] = a;
        out[1] = held > 0 ? a + 1 : 0;
        out[2] = L;
        out[3] = 1 - L;
    }
    return 0;
}
