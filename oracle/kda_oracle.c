/*
 * kda_oracle.c -- fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header or constant
 * with the HIP kernels of the package; it is plain C99 with OpenMP over the
 * independent (sequence, head) units.
 *
 * What it computes (the plain definition, token by token, in double):
 *   per (sequence n, head h) the state S is a dk x dv matrix, and for every
 *   token t of the sequence, in order:
 *     a   = exp(g_t)                      per-key-channel decay
 *     S   = diag(a) S                     decay the rows (key channels)
 *     p   = S^T k_t                       the state's prediction for k_t
 *     u   = beta_t (v_t - p)              delta-rule correction
 *     S   = S + k_t u^T                   write
 *     y_t = sigmoid(z_t) * (scale S^T q_t)  read after the write, then gate
 *
 * Sources (pages, cited by title and section):
 *   - "Kimi K3 second-pass study ledger" (llm-atlas research/K3_RESEARCH.md),
 *     section 1, question ledger: row Q04 (fixed-shape recurrent state,
 *     channel-wise decay, delta-rule write), row Q05 (before writing a new
 *     value, subtract what the state already predicts for the current key),
 *     row Q07 (decode is an O(1) state update), row Q08 (input-dependent,
 *     full-rank output gate on the readout).
 *   - "Kimi K3 plain-language guide", section 5.1 (a fixed-size recurrent
 *     state replaces a growing KV cache; the update is serial).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   decay before the prediction; decay on the key channels (rows of S);
 *   read after the write; the gate is sigmoid of a logit z with no
 *   normalisation in between; beta and g arrive as values (beta in [0,1],
 *   g a natural-log decay, g = -inf allowed and gives a = 0).
 *
 * Parity unpinned: the report's own equation for KDA is cited by the ledger
 * but not printed on the pages, so the readings above cannot be checked
 * against it.  Everything else is pinned by the tests (exact brute force,
 * closed forms, invariants).
 *
 * Layouts (row-major, all contiguous):
 *   q, k, g    [T_total, H, dk]      v, z, out  [T_total, H, dv]
 *   beta       [T_total, H]          state      [N, H, dk, dv]
 *   cu_seqlens [N + 1], int64, cu[0] = 0, non-decreasing, cu[N] = T_total.
 * Inputs are double (in_type = 0), float (1) or bfloat16 bit patterns (2,
 * uint16); float and bfloat16 inputs are widened exactly to double on read.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Element i of an input: in_type 0 = double, 1 = float, 2 = bfloat16 (the
 * upper 16 bits of an IEEE single, widened exactly). */
static double rd(const void *p, int in_type, int64_t i)
{
    if (in_type == 1)
        return (double)((const float *)p)[i];
    if (in_type == 2) {
        uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double *)p)[i];
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* One token of the recurrence on the state S (dk x dv, row-major).
 * qo, ko, vo, bo: element offsets of this token-head in the inputs.
 * a, p, u: scratch of length dk, dv, dv.  Writes dv outputs to y. */
static void kda_token(const void *q, const void *k, const void *v, const void *g,
                      const void *beta, const void *z, int in_type,
                      int64_t qo, int64_t vo, int64_t bo, int64_t dk, int64_t dv,
                      double scale, double *S, double *a, double *p, double *u,
                      double *y)
{
    int64_t i, j;
    for (i = 0; i < dk; ++i)
        a[i] = exp(rd(g, in_type, qo + i));
    /* decay: every row i (key channel) scales by a[i] */
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            S[i * dv + j] *= a[i];
    /* prediction of the decayed state for the current key */
    for (j = 0; j < dv; ++j)
        p[j] = 0.0;
    for (i = 0; i < dk; ++i) {
        double ki = rd(k, in_type, qo + i);
        for (j = 0; j < dv; ++j)
            p[j] += S[i * dv + j] * ki;
    }
    /* delta-rule correction */
    double b = rd(beta, in_type, bo);
    for (j = 0; j < dv; ++j)
        u[j] = b * (rd(v, in_type, vo + j) - p[j]);
    /* write */
    for (i = 0; i < dk; ++i) {
        double ki = rd(k, in_type, qo + i);
        for (j = 0; j < dv; ++j)
            S[i * dv + j] += ki * u[j];
    }
    /* read by the query after the write, then the output gate */
    for (j = 0; j < dv; ++j)
        p[j] = 0.0;
    for (i = 0; i < dk; ++i) {
        double qi = rd(q, in_type, qo + i);
        for (j = 0; j < dv; ++j)
            p[j] += S[i * dv + j] * qi;
    }
    for (j = 0; j < dv; ++j)
        y[j] = sigmoid(rd(z, in_type, vo + j)) * (scale * p[j]);
}

/* Whole-sequence forward.  init_state may be NULL (zeros); final_state may
 * be NULL (not written); out may be NULL (not written).
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int kda_oracle_forward(const void *q, const void *k, const void *v, const void *g,
                       const void *beta, const void *z, int in_type,
                       const double *init_state, double *out, double *final_state,
                       const int64_t *cu_seqlens, int64_t n_seq, int64_t H,
                       int64_t dk, int64_t dv, double scale, int n_threads)
{
    if (!q || !k || !v || !g || !beta || !z || !cu_seqlens)
        return -1;
    if (n_seq < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    for (int64_t n = 0; n < n_seq; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n] || cu_seqlens[0] != 0)
            return -1;
    int64_t units = n_seq * H;
    int failed = 0;
    if (n_threads <= 0)
        n_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int64_t unit = 0; unit < units; ++unit) {
        int64_t n = unit / H, h = unit % H;
        double *S = (double *)malloc(sizeof(double) * dk * dv);
        double *a = (double *)malloc(sizeof(double) * dk);
        double *p = (double *)malloc(sizeof(double) * dv);
        double *u = (double *)malloc(sizeof(double) * dv);
        double *y = (double *)malloc(sizeof(double) * dv);
        if (!S || !a || !p || !u || !y) {
#pragma omp atomic write
            failed = 1;
        } else {
            const double *S0 = init_state ? init_state + unit * dk * dv : NULL;
            for (int64_t e = 0; e < dk * dv; ++e)
                S[e] = S0 ? S0[e] : 0.0;
            for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
                int64_t qo = (t * H + h) * dk, vo = (t * H + h) * dv, bo = t * H + h;
                kda_token(q, k, v, g, beta, z, in_type, qo, vo, bo, dk, dv, scale,
                          S, a, p, u, y);
                if (out)
                    memcpy(out + vo, y, sizeof(double) * dv);
            }
            if (final_state)
                memcpy(final_state + unit * dk * dv, S, sizeof(double) * dk * dv);
        }
        free(S);
        free(a);
        free(p);
        free(u);
        free(y);
    }
    return failed ? -2 : 0;
}

/* The same forward as kda_oracle_forward, compared on the fly with an output
 * x computed elsewhere (x_type 1 = float, 2 = bfloat16 bits, layout of out),
 * so that long inputs need no double-precision output array.  For every
 * (sequence, head) unit: err[unit] = max |x - y| and ref[unit] = max |y| over
 * the unit's tokens and value channels, y the recurrence's output (0 for an
 * empty sequence).  final_state as in kda_oracle_forward (may be NULL). */
int kda_oracle_forward_compare(const void *q, const void *k, const void *v, const void *g,
                               const void *beta, const void *z, int in_type,
                               const double *init_state, const void *x, int x_type,
                               const int64_t *cu_seqlens, int64_t n_seq, int64_t H,
                               int64_t dk, int64_t dv, double scale, int n_threads,
                               double *err, double *ref, double *final_state)
{
    if (!q || !k || !v || !g || !beta || !z || !cu_seqlens || !x || !err || !ref)
        return -1;
    if (n_seq < 0 || H <= 0 || dk <= 0 || dv <= 0 || (x_type != 1 && x_type != 2))
        return -1;
    for (int64_t n = 0; n < n_seq; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n] || cu_seqlens[0] != 0)
            return -1;
    int64_t units = n_seq * H;
    int failed = 0;
    if (n_threads <= 0)
        n_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int64_t unit = 0; unit < units; ++unit) {
        int64_t n = unit / H, h = unit % H;
        double *S = (double *)malloc(sizeof(double) * dk * dv);
        double *a = (double *)malloc(sizeof(double) * dk);
        double *p = (double *)malloc(sizeof(double) * dv);
        double *u = (double *)malloc(sizeof(double) * dv);
        double *y = (double *)malloc(sizeof(double) * dv);
        double e_max = 0.0, r_max = 0.0;
        if (!S || !a || !p || !u || !y) {
#pragma omp atomic write
            failed = 1;
        } else {
            const double *S0 = init_state ? init_state + unit * dk * dv : NULL;
            for (int64_t e = 0; e < dk * dv; ++e)
                S[e] = S0 ? S0[e] : 0.0;
            for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
                int64_t qo = (t * H + h) * dk, vo = (t * H + h) * dv, bo = t * H + h;
                kda_token(q, k, v, g, beta, z, in_type, qo, vo, bo, dk, dv, scale,
                          S, a, p, u, y);
                for (int64_t j = 0; j < dv; ++j) {
                    double d = fabs(rd(x, x_type, vo + j) - y[j]);
                    if (!(d <= e_max))          /* NaN in x counts as infinite error */
                        e_max = d == d ? d : INFINITY;
                    if (fabs(y[j]) > r_max)
                        r_max = fabs(y[j]);
                }
            }
            if (final_state)
                memcpy(final_state + unit * dk * dv, S, sizeof(double) * dk * dv);
        }
        err[unit] = e_max;
        ref[unit] = r_max;
        free(S);
        free(a);
        free(p);
        free(u);
        free(y);
    }
    return failed ? -2 : 0;
}

/* One decode step for N independent sequences: the body of the recurrence
 * applied once to state [N, H, dk, dv] in place.  q, k, g [N, H, dk];
 * v, z, out [N, H, dv]; beta [N, H]. */
int kda_oracle_decode_step(const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const void *z, int in_type, double *state,
                           double *out, int64_t N, int64_t H, int64_t dk, int64_t dv,
                           double scale, int n_threads)
{
    if (!q || !k || !v || !g || !beta || !z || !state || !out)
        return -1;
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    int failed = 0;
    if (n_threads <= 0)
        n_threads = 1;
#pragma omp parallel for schedule(dynamic, 16) num_threads(n_threads)
    for (int64_t unit = 0; unit < N * H; ++unit) {
        double *a = (double *)malloc(sizeof(double) * dk);
        double *p = (double *)malloc(sizeof(double) * dv);
        double *u = (double *)malloc(sizeof(double) * dv);
        if (!a || !p || !u) {
#pragma omp atomic write
            failed = 1;
        } else {
            kda_token(q, k, v, g, beta, z, in_type, unit * dk, unit * dv, unit, dk, dv,
                      scale, state + unit * dk * dv, a, p, u, out + unit * dv);
        }
        free(a);
        free(p);
        free(u);
    }
    return failed ? -2 : 0;
}

/* Backward of the whole-sequence forward (reverse-mode, token by token, in
 * double).  For the loss sum(dout * out) + sum(dfinal * final_state) it
 * returns the gradients with respect to every input:
 *   dq, dk, dg [T_total, H, dk], dv, dz [T_total, H, dv], dbeta [T_total, H],
 *   dinit [N, H, dk, dv] (may be NULL).
 * dfinal may be NULL (zero).  Each token's forward step is reversed in the
 * opposite order of its operations; with S~ = diag(a) S_prev the decayed
 * state and S_new the state after the write:
 *   o  = scale S_new^T q,  y = sigmoid(z) o:
 *        dz = dy o sigmoid'(z),  do = dy sigmoid(z),
 *        dS_new += scale q do^T,  dq = scale S_new do
 *   S_new = S~ + k u^T:   du = dS_new^T k,  dk += dS_new u,  dS~ = dS_new
 *   u = beta (v - p):     dbeta = du . (v - p),  dv = beta du,  dp = -beta du
 *   p = S~^T k:           dS~ += k dp^T,  dk += S~ dp
 *   S~ = diag(a) S_prev:  dS_prev = diag(a) dS~,  dg = a * rowsum(dS~ * S_prev)
 * States are recomputed from checkpoints taken every 32 tokens. */
#define KDA_ORACLE_SEG 32
int kda_oracle_backward(const void *q, const void *k, const void *v, const void *g,
                        const void *beta, const void *z, int in_type,
                        const double *init_state, const double *dout, const double *dfinal,
                        const int64_t *cu_seqlens, int64_t n_seq, int64_t H, int64_t dk,
                        int64_t dv, double scale, int n_threads, double *dq, double *dk_out,
                        double *dv_out, double *dg, double *dbeta, double *dz, double *dinit)
{
    if (!q || !k || !v || !g || !beta || !z || !cu_seqlens || !dout)
        return -1;
    if (!dq || !dk_out || !dv_out || !dg || !dbeta || !dz)
        return -1;
    if (n_seq < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    for (int64_t n = 0; n < n_seq; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n] || cu_seqlens[0] != 0)
            return -1;
    const int64_t units = n_seq * H, sd = dk * dv;
    int failed = 0;
    if (n_threads <= 0)
        n_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t n = unit / H, h = unit % H;
        const int64_t t0 = cu_seqlens[n], len = cu_seqlens[n + 1] - cu_seqlens[n];
        const int64_t nseg = (len + KDA_ORACLE_SEG - 1) / KDA_ORACLE_SEG;
        double *ck = (double *)malloc(sizeof(double) * sd * (nseg > 0 ? nseg : 1));
        double *sb = (double *)malloc(sizeof(double) * sd * (KDA_ORACLE_SEG + 1));
        double *dS = (double *)malloc(sizeof(double) * sd);
        double *Sd = (double *)malloc(sizeof(double) * sd);
        double *a = (double *)malloc(sizeof(double) * dk);
        double *p = (double *)malloc(sizeof(double) * dv);
        double *u = (double *)malloc(sizeof(double) * dv);
        double *y = (double *)malloc(sizeof(double) * dv);
        double *dov = (double *)malloc(sizeof(double) * dv);
        double *du = (double *)malloc(sizeof(double) * dv);
        double *dp = (double *)malloc(sizeof(double) * dv);
        if (!ck || !sb || !dS || !Sd || !a || !p || !u || !y || !dov || !du || !dp) {
#pragma omp atomic write
            failed = 1;
        } else {
            const double *S0 = init_state ? init_state + unit * sd : NULL;
            /* forward, keeping the state on entry to every segment */
            double *S = sb;
            for (int64_t e = 0; e < sd; ++e)
                S[e] = S0 ? S0[e] : 0.0;
            for (int64_t i = 0; i < len; ++i) {
                if (i % KDA_ORACLE_SEG == 0)
                    memcpy(ck + (i / KDA_ORACLE_SEG) * sd, S, sizeof(double) * sd);
                const int64_t t = t0 + i;
                kda_token(q, k, v, g, beta, z, in_type, (t * H + h) * dk, (t * H + h) * dv,
                          t * H + h, dk, dv, scale, S, a, p, u, y);
            }
            for (int64_t e = 0; e < sd; ++e)
                dS[e] = dfinal ? dfinal[unit * sd + e] : 0.0;
            for (int64_t c = nseg - 1; c >= 0; --c) {
                const int64_t i0 = c * KDA_ORACLE_SEG;
                const int64_t nl = (len - i0) < KDA_ORACLE_SEG ? (len - i0) : KDA_ORACLE_SEG;
                /* states of the segment: sb[i] = state before token i0 + i */
                memcpy(sb, ck + c * sd, sizeof(double) * sd);
                for (int64_t i = 0; i < nl; ++i) {
                    memcpy(sb + (i + 1) * sd, sb + i * sd, sizeof(double) * sd);
                    const int64_t t = t0 + i0 + i;
                    kda_token(q, k, v, g, beta, z, in_type, (t * H + h) * dk, (t * H + h) * dv,
                              t * H + h, dk, dv, scale, sb + (i + 1) * sd, a, p, u, y);
                }
                for (int64_t i = nl - 1; i >= 0; --i) {
                    const int64_t t = t0 + i0 + i;
                    const int64_t qo = (t * H + h) * dk, vo = (t * H + h) * dv, bo = t * H + h;
                    const double *Sp = sb + i * sd, *Sn = sb + (i + 1) * sd;
                    const double b = rd(beta, in_type, bo);
                    int64_t r, j;
                    /* recompute a, S~, p, u of this token */
                    for (r = 0; r < dk; ++r)
                        a[r] = exp(rd(g, in_type, qo + r));
                    for (r = 0; r < dk; ++r)
                        for (j = 0; j < dv; ++j)
                            Sd[r * dv + j] = a[r] * Sp[r * dv + j];
                    for (j = 0; j < dv; ++j)
                        p[j] = 0.0;
                    for (r = 0; r < dk; ++r) {
                        const double kr = rd(k, in_type, qo + r);
                        for (j = 0; j < dv; ++j)
                            p[j] += Sd[r * dv + j] * kr;
                    }
                    for (j = 0; j < dv; ++j)
                        u[j] = (rd(v, in_type, vo + j) - p[j]) * b;
                    /* read and gate */
                    for (j = 0; j < dv; ++j)
                        y[j] = 0.0;                        /* y = S_new^T q (unscaled) */
                    for (r = 0; r < dk; ++r) {
                        const double qr = rd(q, in_type, qo + r);
                        for (j = 0; j < dv; ++j)
                            y[j] += Sn[r * dv + j] * qr;
                    }
                    for (j = 0; j < dv; ++j) {
                        const double sg = sigmoid(rd(z, in_type, vo + j));
                        const double o = scale * y[j];
                        dz[vo + j] = dout[vo + j] * o * sg * (1.0 - sg);
                        dov[j] = dout[vo + j] * sg;
                    }
                    for (r = 0; r < dk; ++r) {
                        const double qr = rd(q, in_type, qo + r);
                        double acc = 0.0;
                        for (j = 0; j < dv; ++j) {
                            acc += Sn[r * dv + j] * dov[j];
                            dS[r * dv + j] += scale * qr * dov[j];
                        }
                        dq[qo + r] = scale * acc;
                    }
                    /* write: S_new = S~ + k u^T */
                    for (j = 0; j < dv; ++j)
                        du[j] = 0.0;
                    for (r = 0; r < dk; ++r) {
                        const double kr = rd(k, in_type, qo + r);
                        double acc = 0.0;
                        for (j = 0; j < dv; ++j) {
                            du[j] += dS[r * dv + j] * kr;
                            acc += dS[r * dv + j] * u[j];
                        }
                        dk_out[qo + r] = acc;
                    }
                    /* correction: u = beta (v - p) */
                    double db = 0.0;
                    for (j = 0; j < dv; ++j) {
                        const double vj = rd(v, in_type, vo + j);
                        db += du[j] * (vj - p[j]);
                        dv_out[vo + j] = b * du[j];
                        dp[j] = -b * du[j];
                    }
                    dbeta[bo] = db;
                    /* prediction: p = S~^T k; then the decay S~ = diag(a) S_prev */
                    for (r = 0; r < dk; ++r) {
                        const double kr = rd(k, in_type, qo + r);
                        double acc = 0.0, da = 0.0;
                        for (j = 0; j < dv; ++j) {
                            acc += Sd[r * dv + j] * dp[j];
                            const double dsd = dS[r * dv + j] + kr * dp[j];   /* dS~ */
                            da += dsd * Sp[r * dv + j];
                            dS[r * dv + j] = a[r] * dsd;                      /* dS_prev */
                        }
                        dk_out[qo + r] += acc;
                        dg[qo + r] = a[r] * da;
                    }
                }
            }
            if (dinit)
                memcpy(dinit + unit * sd, dS, sizeof(double) * sd);
        }
        free(ck);
        free(sb);
        free(dS);
        free(Sd);
        free(a);
        free(p);
        free(u);
        free(y);
        free(dov);
        free(du);
        free(dp);
    }
    return failed ? -2 : 0;
}

/* Threads OpenMP would use by default (for reporting the CPU baseline). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
