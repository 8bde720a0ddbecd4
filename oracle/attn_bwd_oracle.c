/*
 * attn_bwd_oracle.c -- plain, slow, scalar fp64 CPU oracle for the gradient
 * of segment-masked, non-causal softmax self-attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file or the library built from it; only the tests, the
 * package smoke check and the benchmark's CPU-baseline leg do.  It shares no
 * code, header, helper or constant with the HIP path.
 *
 * What it computes.  The forward is out_i = sum_j P_ij v_j with
 * P_ij = exp(s_ij) / sum_{j' in J_i} exp(s_ij'), s_ij = scale * q_i . k_j over
 * the valid keys J_i of row i (segment rule of the forward oracle; a row with
 * no valid key has out_i = 0).  Given dout, this returns the exact gradients
 * of sum_i dout_i . out_i (vidax paper, arXiv:2609.18077: section 5 lists
 * training and fine-tuning as future work; the forward's log-sum-exp output
 * is what a backward pass reuses):
 *   dv_j = sum_i P_ij dout_i
 *   dP_ij = dout_i . v_j,  delta_i = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - delta_i)
 *   dq_i = scale * sum_j dS_ij k_j,  dk_j = scale * sum_i dS_ij q_i
 * P, delta and everything else are recomputed here from q, k, v in fp64; the
 * oracle takes no forward output.  Rows with no valid key contribute nothing
 * and get dq_i = 0.  Inputs are bf16 bit patterns [B, S, H, D]; outputs fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_EXPORT __attribute__((visibility("default")))

static double b2d(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v, *dout;
    const int32_t *seg_q, *seg_kv;
    int64_t B, S, H, D;
    double scale;
    double *dq, *dk, *dv;
    double *tq, *tk, *tv; /* optional rounding-sensitivity sums (NULL: skip) */
    int64_t next;
    pthread_mutex_t mu;
} bjob_t;

static int64_t at(const bjob_t *J, int64_t b, int64_t s, int64_t h) {
    return ((b * J->S + s) * J->H + h) * J->D;
}

static int valid(const bjob_t *J, int64_t b, int64_t i, int64_t j) {
    if (!J->seg_q) return 1;
    const int32_t c = J->seg_q[b * J->S + i];
    return c != 0 && J->seg_kv[b * J->S + j] == c;
}

/* One (b, h): dense S x S probabilities and score gradients in fp64. */
static int one_head(const bjob_t *J, int64_t b, int64_t h) {
    const int64_t S = J->S, D = J->D;
    double *P = (double *)malloc(sizeof(double) * (size_t)(S * S));
    double *dS = (double *)malloc(sizeof(double) * (size_t)(S * S));
    double *E = J->tq ? (double *)malloc(sizeof(double) * (size_t)S) : NULL;
    double *acc = (double *)malloc(sizeof(double) * (size_t)(4 * D));
    if (!P || !dS || (J->tq && !E) || !acc) {
        free(P);
        free(dS);
        free(E);
        free(acc);
        return 1;
    }
    double *accv = acc + D, *tacc = acc + 2 * D, *taccv = acc + 3 * D;
    for (int64_t i = 0; i < S; ++i) {
        double m = -INFINITY;
        for (int64_t j = 0; j < S; ++j) {
            if (!valid(J, b, i, j)) {
                P[i * S + j] = -INFINITY;
                continue;
            }
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d)
                dot += b2d(J->q[at(J, b, i, h) + d]) * b2d(J->k[at(J, b, j, h) + d]);
            P[i * S + j] = J->scale * dot;
            if (P[i * S + j] > m) m = P[i * S + j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < S; ++j) {
            const double w = (m == -INFINITY || P[i * S + j] == -INFINITY) ? 0.0 : exp(P[i * S + j] - m);
            P[i * S + j] = w;
            l += w;
        }
        for (int64_t j = 0; j < S; ++j) P[i * S + j] = (l > 0.0) ? P[i * S + j] / l : 0.0;
        /* dP_ij = dout_i . v_j over valid pairs, delta_i = sum_j P_ij dP_ij */
        double delta = 0.0;
        for (int64_t j = 0; j < S; ++j) {
            double dp = 0.0;
            if (valid(J, b, i, j))
                for (int64_t d = 0; d < D; ++d)
                    dp += b2d(J->dout[at(J, b, i, h) + d]) * b2d(J->v[at(J, b, j, h) + d]);
            dS[i * S + j] = dp;
            delta += P[i * S + j] * dp;
        }
        for (int64_t j = 0; j < S; ++j) dS[i * S + j] = P[i * S + j] * (dS[i * S + j] - delta);
        if (E) {
            /* E_i = sum_j P_ij sum_d |dout_id| |v_jd|: bounds how far delta_i
             * moves per unit relative error in out_i's terms */
            double e = 0.0;
            for (int64_t j = 0; j < S; ++j) {
                if (P[i * S + j] == 0.0) continue;
                double a = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    a += fabs(b2d(J->dout[at(J, b, i, h) + d])) * fabs(b2d(J->v[at(J, b, j, h) + d]));
                e += P[i * S + j] * a;
            }
            E[i] = e;
        }
    }
    /* The sums below run the index being summed over in ascending order for
     * each output element; the loops nest with that index outside the head
     * dimension so P, dS and the operand rows are walked contiguously. */
    for (int64_t i = 0; i < S; ++i) {
        for (int64_t d = 0; d < D; ++d) acc[d] = tacc[d] = 0.0;
        for (int64_t j = 0; j < S; ++j) {
            const double ds = dS[i * S + j];
            const uint16_t *kj = J->k + at(J, b, j, h);
            for (int64_t d = 0; d < D; ++d) acc[d] += ds * b2d(kj[d]);
            if (E) {
                const double w = fabs(ds) + P[i * S + j] * E[i];
                for (int64_t d = 0; d < D; ++d) tacc[d] += w * fabs(b2d(kj[d]));
            }
        }
        for (int64_t d = 0; d < D; ++d) {
            J->dq[at(J, b, i, h) + d] = J->scale * acc[d];
            if (E) J->tq[at(J, b, i, h) + d] = J->scale * tacc[d];
        }
    }
    /* dk and dv sum over the queries i: transpose P and dS so that key j's
     * column is contiguous. */
    for (int64_t i = 0; i < S; ++i)
        for (int64_t j = 0; j < i; ++j) {
            const double p = P[i * S + j], g = dS[i * S + j];
            P[i * S + j] = P[j * S + i];
            dS[i * S + j] = dS[j * S + i];
            P[j * S + i] = p;
            dS[j * S + i] = g;
        }
    /* P and dS now hold P^T and dS^T: P[j * S + i] = P_ij */
    for (int64_t j = 0; j < S; ++j) {
        for (int64_t d = 0; d < D; ++d) acc[d] = accv[d] = tacc[d] = taccv[d] = 0.0;
        for (int64_t i = 0; i < S; ++i) {
            const double ds = dS[j * S + i], p = P[j * S + i];
            const uint16_t *qi = J->q + at(J, b, i, h), *oi = J->dout + at(J, b, i, h);
            for (int64_t d = 0; d < D; ++d) {
                acc[d] += ds * b2d(qi[d]);
                accv[d] += p * b2d(oi[d]);
            }
            if (E) {
                const double w = fabs(ds) + p * E[i];
                for (int64_t d = 0; d < D; ++d) {
                    tacc[d] += w * fabs(b2d(qi[d]));
                    taccv[d] += p * fabs(b2d(oi[d]));
                }
            }
        }
        for (int64_t d = 0; d < D; ++d) {
            J->dk[at(J, b, j, h) + d] = J->scale * acc[d];
            J->dv[at(J, b, j, h) + d] = accv[d];
            if (E) {
                J->tk[at(J, b, j, h) + d] = J->scale * tacc[d];
                J->tv[at(J, b, j, h) + d] = taccv[d];
            }
        }
    }
    free(acc);
    free(P);
    free(dS);
    free(E);
    return 0;
}

static void *b_worker(void *arg) {
    bjob_t *J = (bjob_t *)arg;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t r = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (r >= J->B * J->H) break;
        if (one_head(J, r / J->H, r % J->H)) return (void *)1;
    }
    return NULL;
}

/* dq of listed rows only: the same formulas restricted to one row i, whose
 * probabilities, dP and delta need row i's scores alone (O(S D) per row). */
typedef struct {
    const bjob_t *J;
    const int64_t *rows;
    int64_t n_rows;
    double *dq, *tq;
    int64_t next;
    pthread_mutex_t mu;
} rjob_t;

static int one_row(const bjob_t *J, int64_t b, int64_t h, int64_t i, double *P, double *dP, double *dq,
                   double *tq) {
    const int64_t S = J->S, D = J->D;
    double m = -INFINITY;
    for (int64_t j = 0; j < S; ++j) {
        if (!valid(J, b, i, j)) {
            P[j] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += b2d(J->q[at(J, b, i, h) + d]) * b2d(J->k[at(J, b, j, h) + d]);
        P[j] = J->scale * dot;
        if (P[j] > m) m = P[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < S; ++j) {
        const double w = (m == -INFINITY || P[j] == -INFINITY) ? 0.0 : exp(P[j] - m);
        P[j] = w;
        l += w;
    }
    double delta = 0.0;
    for (int64_t j = 0; j < S; ++j) {
        P[j] = (l > 0.0) ? P[j] / l : 0.0;
        double dp = 0.0;
        if (valid(J, b, i, j))
            for (int64_t d = 0; d < D; ++d)
                dp += b2d(J->dout[at(J, b, i, h) + d]) * b2d(J->v[at(J, b, j, h) + d]);
        dP[j] = dp;
        delta += P[j] * dp;
    }
    for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < S; ++j) acc += P[j] * (dP[j] - delta) * b2d(J->k[at(J, b, j, h) + d]);
        dq[d] = J->scale * acc;
    }
    if (tq) {
        double e = 0.0;
        for (int64_t j = 0; j < S; ++j) {
            if (P[j] == 0.0) continue;
            double a = 0.0;
            for (int64_t d = 0; d < D; ++d)
                a += fabs(b2d(J->dout[at(J, b, i, h) + d])) * fabs(b2d(J->v[at(J, b, j, h) + d]));
            e += P[j] * a;
        }
        for (int64_t d = 0; d < D; ++d) {
            double t = 0.0;
            for (int64_t j = 0; j < S; ++j)
                t += (fabs(P[j] * (dP[j] - delta)) + P[j] * e) * fabs(b2d(J->k[at(J, b, j, h) + d]));
            tq[d] = J->scale * t;
        }
    }
    return 0;
}

static void *r_worker(void *arg) {
    rjob_t *R = (rjob_t *)arg;
    const bjob_t *J = R->J;
    double *P = (double *)malloc(sizeof(double) * (size_t)J->S);
    double *dP = (double *)malloc(sizeof(double) * (size_t)J->S);
    if (!P || !dP) {
        free(P);
        free(dP);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&R->mu);
        const int64_t r = R->next++;
        pthread_mutex_unlock(&R->mu);
        if (r >= R->n_rows) break;
        const int64_t *t = R->rows + 3 * r;
        one_row(J, t[0], t[1], t[2], P, dP, R->dq + r * J->D, R->tq ? R->tq + r * J->D : NULL);
    }
    free(P);
    free(dP);
    return NULL;
}

/*
 * vdx_oracle_attn_bwd_dq_rows
 *   Same inputs as vdx_oracle_attn_bwd; rows = n_rows (b, h, i) triples;
 *   dq = fp64 [n_rows, D], the dq of each listed row; tq = NULL or fp64
 *   [n_rows, D], its rounding-sensitivity sum (as for vdx_oracle_attn_bwd).
 *   No limit on S.
 * Returns 0 on success, 1 on bad arguments, 2 on allocation failure.
 */
ORACLE_EXPORT int vdx_oracle_attn_bwd_dq_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                              const uint16_t *dout, const int32_t *seg_q,
                                              const int32_t *seg_kv, int64_t B, int64_t S, int64_t H,
                                              int64_t D, double scale, const int64_t *rows,
                                              int64_t n_rows, double *dq, double *tq, int n_threads) {
    if (!q || !k || !v || !dout || !dq || !rows) return 1;
    if ((seg_q == NULL) != (seg_kv == NULL)) return 1;
    if (B < 1 || S < 1 || H < 1 || D < 1 || n_rows < 0) return 1;
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t *t = rows + 3 * r;
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= H || t[2] < 0 || t[2] >= S) return 1;
    }
    if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (n_threads < 1) n_threads = 1;
    bjob_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dout = dout;
    J.seg_q = seg_q; J.seg_kv = seg_kv;
    J.B = B; J.S = S; J.H = H; J.D = D;
    J.scale = scale;
    rjob_t R;
    memset(&R, 0, sizeof R);
    R.J = &J;
    R.rows = rows;
    R.n_rows = n_rows;
    R.dq = dq;
    R.tq = tq;
    pthread_mutex_init(&R.mu, NULL);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!th) return 2;
    int started = 0, failed = 0;
    for (int t = 0; t < n_threads; ++t)
        if (pthread_create(&th[t], NULL, r_worker, &R) == 0) ++started;
    if (started == 0) failed = (r_worker(&R) != NULL);
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret != NULL) failed = 1;
    }
    free(th);
    pthread_mutex_destroy(&R.mu);
    return failed ? 2 : 0;
}

/*
 * vdx_oracle_attn_bwd
 *   q, k, v, dout  bf16 bit patterns [B, S, H, D], host memory.
 *   seg_q/seg_kv   int32 [B, S] or both NULL (unmasked).
 *   dq, dk, dv     fp64 [B, S, H, D] outputs.
 *   tq, tk, tv     fp64 [B, S, H, D] or all NULL: per element, the sum of
 *                  the absolute values of the terms whose rounding makes up a
 *                  finite-precision implementation's error --
 *                    tq_id = scale sum_j (|dS_ij| + P_ij E_i) |k_jd|
 *                    tk_jd = scale sum_i (|dS_ij| + P_ij E_i) |q_id|
 *                    tv_jd = sum_i P_ij |dout_id|
 *                  with E_i = sum_j P_ij sum_d |dout_id| |v_jd| (how far
 *                  delta_i moves per unit relative error in out_i's terms).
 *                  A result computed with every term rounded once to
 *                  relative precision u lies within u * t of the exact one.
 *   n_threads      worker threads over (b, h) (<= 0 -> online CPUs).
 * Memory: two S x S fp64 matrices per thread.  Returns 0 on success, 1 on bad
 * arguments, 2 on allocation failure.
 */
ORACLE_EXPORT int vdx_oracle_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                      const uint16_t *dout, const int32_t *seg_q, const int32_t *seg_kv,
                                      int64_t B, int64_t S, int64_t H, int64_t D, double scale,
                                      double *dq, double *dk, double *dv, double *tq, double *tk,
                                      double *tv, int n_threads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return 1;
    if ((tq == NULL) != (tk == NULL) || (tq == NULL) != (tv == NULL)) return 1;
    if ((seg_q == NULL) != (seg_kv == NULL)) return 1;
    if (B < 1 || S < 1 || H < 1 || D < 1 || S > 16384) return 1;
    if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (n_threads < 1) n_threads = 1;
    bjob_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dout = dout;
    J.seg_q = seg_q; J.seg_kv = seg_kv;
    J.B = B; J.S = S; J.H = H; J.D = D;
    J.scale = scale;
    J.dq = dq; J.dk = dk; J.dv = dv;
    J.tq = tq; J.tk = tk; J.tv = tv;
    pthread_mutex_init(&J.mu, NULL);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!th) return 2;
    int started = 0, failed = 0;
    for (int t = 0; t < n_threads; ++t)
        if (pthread_create(&th[t], NULL, b_worker, &J) == 0) ++started;
    if (started == 0) failed = (b_worker(&J) != NULL);
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret != NULL) failed = 1;
    }
    free(th);
    pthread_mutex_destroy(&J.mu);
    return failed ? 2 : 0;
}
