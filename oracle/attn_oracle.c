/*
 * attn_oracle.c -- plain, slow, scalar fp64 CPU oracle for segment-masked,
 * non-causal softmax self-attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file or the library built from it; only the tests, the
 * package smoke check and the benchmark's CPU-baseline leg do.  It shares no
 * code, header, helper or constant with the HIP path.
 *
 * What it computes (the plain definition, not an algorithm replay):
 *   vidax paper (arXiv:2609.18077), section 1 "Spatiotemporal constraints in
 *   video generation": full self-attention over the flattened multi-frame
 *   patch volume;
 *   section 2 "3D RoPE, 3D VAEs, and flash attention": attention dispatches to
 *   flash-attention kernels, whose cited algorithm (reference [2],
 *   FlashAttention: "exact attention") returns exactly softmax(Q K^T) V, only
 *   without materialising the score matrix -- so the oracle is that
 *   definition written out;
 *   Appendix A, Table 4, group 2 (HunyuanVideo-1.5 row): SegmentIds decide
 *   which (query, key) pairs take part instead of a dense (B,H,Sq,Sk) mask;
 *   Table 4, group 1 (CogVideoX row): padding tokens must not be attended.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - pair (i, j) of batch b is valid iff seg_q[b,i] == seg_kv[b,j] and that
 *     ID is nonzero; ID 0 marks padding and matches nothing, itself included;
 *     NULL segment arrays mean "every pair valid";
 *   - lse is the natural log of the sum of exp of the scaled scores over the
 *     valid keys of a row;
 *   - a row with no valid key has out = +0.0 and lse = -inf;
 *   - scores are scale * (q . k) with the dot product summed in fp64 over d
 *     ascending; inputs are the exact bf16 values widened to fp64.
 *
 * Layouts: q, k, v are bf16 bit patterns [B, S, H, D]; seg arrays int32 [B, S].
 * Output is fp64 and is never rounded to bf16 here.
 *
 * Optionally it also returns, per output element, the sum of the magnitudes
 * of the terms that make it up, sens_id = sum_j P_ij |v_jd|: a finite-precision
 * result whose every probability carries its own relative error up to u lies
 * within u * sens_id of the exact one (to first order), which sets the parity
 * tolerance of elements where that exceeds the fixed bound.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_EXPORT __attribute__((visibility("default")))

/* bf16 bit pattern -> fp64, exactly (bf16 is the top half of an fp32). */
static double bf16_to_f64(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

typedef struct {
    const uint16_t *q, *k, *v;
    const int32_t *seg_q, *seg_kv;
    int64_t B, S, H, D;
    double scale;
    const int64_t *rows; /* n_rows (b, h, i) triples, or NULL for all rows */
    int64_t n_rows;
    double *out, *lse;
    double *probs;       /* optional: per-row probability vector [n_rows, S] */
    double *sens;        /* optional: sum_j P_ij |v_jd|, shaped like out */
    int64_t next;        /* shared work counter */
    pthread_mutex_t mu;
} job_t;

static int64_t tok_index(const job_t *J, int64_t b, int64_t s, int64_t h) {
    return ((b * J->S + s) * J->H + h) * J->D;
}

/* One output row: fixed (b, h, i). */
static void one_row(const job_t *J, int64_t b, int64_t h, int64_t i,
                    double *out_row, double *lse_row, double *probs_row, double *sens_row,
                    double *s_buf, unsigned char *valid) {
    const int64_t S = J->S, D = J->D;
    int any = 0;
    const int32_t c = J->seg_q ? J->seg_q[b * S + i] : 1;

    /* Valid key set J_i. */
    for (int64_t j = 0; j < S; ++j) {
        int ok;
        if (J->seg_q == NULL)
            ok = 1;
        else
            ok = (c != 0) && (J->seg_kv[b * S + j] == c);
        valid[j] = (unsigned char)ok;
        any |= ok;
    }
    if (!any) {
        for (int64_t d = 0; d < D; ++d) out_row[d] = 0.0;
        if (sens_row)
            for (int64_t d = 0; d < D; ++d) sens_row[d] = 0.0;
        *lse_row = -INFINITY;
        if (probs_row)
            for (int64_t j = 0; j < S; ++j) probs_row[j] = 0.0;
        return;
    }

    /* Scaled scores and their maximum over the valid keys. */
    const uint16_t *qi = J->q + tok_index(J, b, i, h);
    double m = -INFINITY;
    for (int64_t j = 0; j < S; ++j) {
        if (!valid[j]) continue;
        const uint16_t *kj = J->k + tok_index(J, b, j, h);
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += bf16_to_f64(qi[d]) * bf16_to_f64(kj[d]);
        s_buf[j] = J->scale * dot;
        if (s_buf[j] > m) m = s_buf[j];
    }

    /* Softmax weights relative to the maximum, their sum, and the weighted V. */
    double l = 0.0;
    for (int64_t d = 0; d < D; ++d) out_row[d] = 0.0;
    if (sens_row)
        for (int64_t d = 0; d < D; ++d) sens_row[d] = 0.0;
    for (int64_t j = 0; j < S; ++j) {
        if (!valid[j]) continue;
        const double w = exp(s_buf[j] - m);
        s_buf[j] = w;
        l += w;
        const uint16_t *vj = J->v + tok_index(J, b, j, h);
        for (int64_t d = 0; d < D; ++d) out_row[d] += w * bf16_to_f64(vj[d]);
        if (sens_row)
            for (int64_t d = 0; d < D; ++d) sens_row[d] += w * fabs(bf16_to_f64(vj[d]));
    }
    for (int64_t d = 0; d < D; ++d) out_row[d] /= l;
    if (sens_row)
        for (int64_t d = 0; d < D; ++d) sens_row[d] /= l;
    *lse_row = m + log(l);
    if (probs_row)
        for (int64_t j = 0; j < S; ++j) probs_row[j] = valid[j] ? s_buf[j] / l : 0.0;
}

static void *worker(void *arg) {
    job_t *J = (job_t *)arg;
    double *s_buf = (double *)malloc(sizeof(double) * (size_t)J->S);
    unsigned char *valid = (unsigned char *)malloc((size_t)J->S);
    if (!s_buf || !valid) {
        free(s_buf);
        free(valid);
        return (void *)1;
    }
    const int64_t total = J->rows ? J->n_rows : J->B * J->H * J->S;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t r = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (r >= total) break;
        int64_t b, h, i;
        double *out_row, *lse_row, *probs_row = NULL, *sens_row = NULL;
        if (J->rows) {
            b = J->rows[3 * r + 0];
            h = J->rows[3 * r + 1];
            i = J->rows[3 * r + 2];
            out_row = J->out + r * J->D;
            lse_row = J->lse + r;
            if (J->probs) probs_row = J->probs + r * J->S;
            if (J->sens) sens_row = J->sens + r * J->D;
        } else {
            /* r enumerates (b, h, i) with i fastest; out is [B,S,H,D], lse [B,H,S]. */
            i = r % J->S;
            h = (r / J->S) % J->H;
            b = r / (J->S * J->H);
            out_row = J->out + tok_index(J, b, i, h);
            lse_row = J->lse + (b * J->H + h) * J->S + i;
            if (J->probs) probs_row = J->probs + r * J->S;
            if (J->sens) sens_row = J->sens + tok_index(J, b, i, h);
        }
        one_row(J, b, h, i, out_row, lse_row, probs_row, sens_row, s_buf, valid);
    }
    free(s_buf);
    free(valid);
    return NULL;
}

/*
 * vdx_oracle_attn_fwd
 *   q, k, v      bf16 bit patterns, [B, S, H, D], contiguous, host memory.
 *   seg_q/seg_kv int32 [B, S] or both NULL (unmasked).
 *   scale        multiplies q . k (fp64).
 *   rows         NULL -> every row; out is [B,S,H,D] and lse is [B,H,S].
 *                else n_rows (b, h, i) triples; out is [n_rows, D], lse [n_rows].
 *   probs        optional [n_rows or B*H*S, S] softmax rows (tiny cases only).
 *   sens         optional, shaped like out: sum_j P_ij |v_jd| per element.
 *   n_threads    worker threads (<= 0 -> online CPUs).
 * Returns 0 on success, 1 on bad arguments, 2 on allocation failure.
 */
ORACLE_EXPORT int vdx_oracle_attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                      const int32_t *seg_q, const int32_t *seg_kv,
                                      int64_t B, int64_t S, int64_t H, int64_t D, double scale,
                                      const int64_t *rows, int64_t n_rows,
                                      double *out, double *lse, double *probs, double *sens,
                                      int n_threads) {
    if (!q || !k || !v || !out || !lse) return 1;
    if ((seg_q == NULL) != (seg_kv == NULL)) return 1;
    if (B < 1 || S < 1 || H < 1 || D < 1) return 1;
    if (rows) {
        if (n_rows < 0) return 1;
        for (int64_t r = 0; r < n_rows; ++r) {
            const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= S) return 1;
        }
    }
    if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (n_threads < 1) n_threads = 1;

    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v;
    J.seg_q = seg_q; J.seg_kv = seg_kv;
    J.B = B; J.S = S; J.H = H; J.D = D;
    J.scale = scale;
    J.rows = rows; J.n_rows = n_rows;
    J.out = out; J.lse = lse; J.probs = probs; J.sens = sens;
    J.next = 0;
    pthread_mutex_init(&J.mu, NULL);

    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!th) return 2;
    int started = 0, failed = 0;
    for (int t = 0; t < n_threads; ++t) {
        if (pthread_create(&th[t], NULL, worker, &J) == 0) ++started;
    }
    if (started == 0) failed = (worker(&J) != NULL);
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret != NULL) failed = 1;
    }
    free(th);
    pthread_mutex_destroy(&J.mu);
    return failed ? 2 : 0;
}

ORACLE_EXPORT int vdx_oracle_version(void) { return 1; }
