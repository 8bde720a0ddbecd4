/*
 * natten_oracle.c -- plain, slow, scalar fp64 CPU oracle for 3D neighbourhood
 * (windowed) self-attention over a t x h x w token grid.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file or the library built from it; only the tests, the
 * package smoke check and the benchmark's CPU-baseline leg do.  It shares no
 * code, header, helper or constant with the HIP path.
 *
 * What it computes (vidax paper, arXiv:2609.18077):
 *   section 2, "3D RoPE, 3D VAEs, and flash attention": models without a
 *   native TPU kernel, such as LTX-2.5's neighbourhood-attention VAE decoder,
 *   fall back to a windowed-attention primitive;
 *   Appendix A, Table 4, group 4 ("Memory, Tiling & Execution Graphs"),
 *   LTX-2.5 VAE decoder rows: local-window attention whose window spans
 *   11 x 11 x 11 grid positions for that checkpoint's stage-5 kernel, rebuilt
 *   to process one query at a time with a gather of its window.
 * The plain definition, per query token: softmax over the keys inside its
 * window of the scaled dot products, applied to the values of those keys.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - tokens of the grid are flattened (t, y, x) row-major, x fastest:
 *     s = (t * NH + y) * NW + x;
 *   - the window of a query is its neighbourhood in the sense of
 *     neighbourhood attention: along an axis of length n with window size k
 *     (odd), k_eff = min(k, n) positions starting at
 *     clamp(c - k/2, 0, n - k_eff), so the window shifts inward at the grid
 *     border and every query sees exactly k_eff,t * k_eff,h * k_eff,w keys;
 *   - no causality along t, no dilation;
 *   - scores are scale * (q . k) summed in fp64 over d ascending; lse is the
 *     natural log of the sum of exp of the scaled scores in the window.
 *
 * Layouts: q, k, v are bf16 bit patterns [B, S, H, D] with S = NT*NH*NW.
 * Output is fp64 and is never rounded to bf16 here.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_EXPORT __attribute__((visibility("default")))

static double bf16_bits_to_f64(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* First window position along an axis of length n for coordinate c. */
static int64_t window_start(int64_t c, int64_t k, int64_t n) {
    const int64_t keff = k < n ? k : n;
    int64_t s = c - k / 2;
    if (s < 0) s = 0;
    if (s > n - keff) s = n - keff;
    return s;
}

typedef struct {
    const uint16_t *q, *k, *v;
    int64_t B, NT, NH, NW, H, D, KT, KH, KW;
    double scale;
    const int64_t *rows;
    int64_t n_rows;
    double *out, *lse;
    double *sens; /* optional: sum over the window of P_ij |v_jd|, shaped like out */
    int64_t next;
    pthread_mutex_t mu;
} njob_t;

static int64_t n_tok(const njob_t *J) { return J->NT * J->NH * J->NW; }

static int64_t elem(const njob_t *J, int64_t b, int64_t s, int64_t h) {
    return ((b * n_tok(J) + s) * J->H + h) * J->D;
}

static void n_row(const njob_t *J, int64_t b, int64_t h, int64_t i, double *out_row, double *lse_row,
                  double *sens_row, double *s_buf) {
    const int64_t D = J->D;
    const int64_t x = i % J->NW, y = (i / J->NW) % J->NH, t = i / (J->NW * J->NH);
    const int64_t kt = J->KT < J->NT ? J->KT : J->NT;
    const int64_t kh = J->KH < J->NH ? J->KH : J->NH;
    const int64_t kw = J->KW < J->NW ? J->KW : J->NW;
    const int64_t t0 = window_start(t, J->KT, J->NT);
    const int64_t y0 = window_start(y, J->KH, J->NH);
    const int64_t x0 = window_start(x, J->KW, J->NW);
    const uint16_t *qi = J->q + elem(J, b, i, h);

    /* Scores over the window, enumerated (dt, dy, dx) with dx fastest. */
    double m = -INFINITY;
    int64_t n = 0;
    for (int64_t a = 0; a < kt; ++a)
        for (int64_t c = 0; c < kh; ++c)
            for (int64_t e = 0; e < kw; ++e) {
                const int64_t j = ((t0 + a) * J->NH + (y0 + c)) * J->NW + (x0 + e);
                const uint16_t *kj = J->k + elem(J, b, j, h);
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += bf16_bits_to_f64(qi[d]) * bf16_bits_to_f64(kj[d]);
                s_buf[n] = J->scale * dot;
                if (s_buf[n] > m) m = s_buf[n];
                ++n;
            }

    double l = 0.0;
    for (int64_t d = 0; d < D; ++d) out_row[d] = 0.0;
    if (sens_row)
        for (int64_t d = 0; d < D; ++d) sens_row[d] = 0.0;
    n = 0;
    for (int64_t a = 0; a < kt; ++a)
        for (int64_t c = 0; c < kh; ++c)
            for (int64_t e = 0; e < kw; ++e) {
                const int64_t j = ((t0 + a) * J->NH + (y0 + c)) * J->NW + (x0 + e);
                const double w = exp(s_buf[n] - m);
                l += w;
                const uint16_t *vj = J->v + elem(J, b, j, h);
                for (int64_t d = 0; d < D; ++d) out_row[d] += w * bf16_bits_to_f64(vj[d]);
                if (sens_row)
                    for (int64_t d = 0; d < D; ++d) sens_row[d] += w * fabs(bf16_bits_to_f64(vj[d]));
                ++n;
            }
    for (int64_t d = 0; d < D; ++d) out_row[d] /= l;
    if (sens_row)
        for (int64_t d = 0; d < D; ++d) sens_row[d] /= l;
    *lse_row = m + log(l);
}

static void *n_worker(void *arg) {
    njob_t *J = (njob_t *)arg;
    const int64_t S = n_tok(J);
    const int64_t wmax = (J->KT < J->NT ? J->KT : J->NT) * (J->KH < J->NH ? J->KH : J->NH) *
                         (J->KW < J->NW ? J->KW : J->NW);
    double *s_buf = (double *)malloc(sizeof(double) * (size_t)wmax);
    if (!s_buf) return (void *)1;
    const int64_t total = J->rows ? J->n_rows : J->B * J->H * S;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t r = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (r >= total) break;
        int64_t b, h, i;
        double *out_row, *lse_row, *sens_row = NULL;
        if (J->rows) {
            b = J->rows[3 * r + 0];
            h = J->rows[3 * r + 1];
            i = J->rows[3 * r + 2];
            out_row = J->out + r * J->D;
            lse_row = J->lse + r;
            if (J->sens) sens_row = J->sens + r * J->D;
        } else {
            i = r % S;
            h = (r / S) % J->H;
            b = r / (S * J->H);
            out_row = J->out + elem(J, b, i, h);
            lse_row = J->lse + (b * J->H + h) * S + i;
            if (J->sens) sens_row = J->sens + elem(J, b, i, h);
        }
        n_row(J, b, h, i, out_row, lse_row, sens_row, s_buf);
    }
    free(s_buf);
    return NULL;
}

/*
 * vdx_oracle_natten3d_fwd
 *   q, k, v        bf16 bit patterns, [B, S, H, D] with S = NT*NH*NW, host memory.
 *   NT, NH, NW     grid extents (t, y, x); tokens flattened (t, y, x), x fastest.
 *   KT, KH, KW     window sizes, odd and >= 1 (larger than the grid: whole axis).
 *   scale          multiplies q . k (fp64).
 *   rows           NULL -> every row; out is [B,S,H,D] and lse is [B,H,S].
 *                  else n_rows (b, h, i) triples; out is [n_rows, D], lse [n_rows].
 *   sens           optional, shaped like out: sum over the window of P_ij |v_jd|
 *                  (first-order rounding sensitivity of each output element).
 *   n_threads      worker threads (<= 0 -> online CPUs).
 * Returns 0 on success, 1 on bad arguments, 2 on allocation failure.
 */
ORACLE_EXPORT int vdx_oracle_natten3d_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                          int64_t B, int64_t NT, int64_t NH, int64_t NW, int64_t H,
                                          int64_t D, int64_t KT, int64_t KH, int64_t KW, double scale,
                                          const int64_t *rows, int64_t n_rows, double *out, double *lse,
                                          double *sens, int n_threads) {
    if (!q || !k || !v || !out || !lse) return 1;
    if (B < 1 || NT < 1 || NH < 1 || NW < 1 || H < 1 || D < 1) return 1;
    if (KT < 1 || KH < 1 || KW < 1 || KT % 2 == 0 || KH % 2 == 0 || KW % 2 == 0) return 1;
    const int64_t S = NT * NH * NW;
    if (rows) {
        if (n_rows < 0) return 1;
        for (int64_t r = 0; r < n_rows; ++r) {
            const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= S) return 1;
        }
    }
    if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (n_threads < 1) n_threads = 1;

    njob_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v;
    J.B = B; J.NT = NT; J.NH = NH; J.NW = NW; J.H = H; J.D = D;
    J.KT = KT; J.KH = KH; J.KW = KW;
    J.scale = scale;
    J.rows = rows; J.n_rows = n_rows;
    J.out = out; J.lse = lse; J.sens = sens;
    J.next = 0;
    pthread_mutex_init(&J.mu, NULL);

    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!th) return 2;
    int started = 0, failed = 0;
    for (int t = 0; t < n_threads; ++t)
        if (pthread_create(&th[t], NULL, n_worker, &J) == 0) ++started;
    if (started == 0) failed = (n_worker(&J) != NULL);
    for (int t = 0; t < started; ++t) {
        void *ret = NULL;
        pthread_join(th[t], &ret);
        if (ret != NULL) failed = 1;
    }
    free(th);
    pthread_mutex_destroy(&J.mu);
    return failed ? 2 : 0;
}
