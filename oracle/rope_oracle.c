/*
 * rope_oracle.c -- plain, slow, scalar CPU oracle for the 3D rotary position
 * embedding that video DiTs apply to attention queries and keys.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file or the library built from it; only the tests, the
 * package smoke check and the benchmark's CPU-baseline leg do.  It shares no
 * code, header, helper or constant with the HIP path.
 *
 * The pages (vidax paper, arXiv:2609.18077) fix only this much: the video
 * DiTs position their tokens with a 3D rotary position embedding over time,
 * height and width, applied to the queries and keys right before attention,
 * and the families' conventions differ and cannot be swapped for one another
 * (section 2, "3D RoPE, 3D VAEs, and flash attention"; section 3.1 names Wan
 * and CogVideoX1.5 as 3D-RoPE DiTs).  No formula is printed.  This oracle is
 * the rotary position embedding's own definition -- every feature pair is
 * rotated in its plane by an angle that depends on the token's position --
 * with each family-specific choice left to the caller:
 *   - features [0, d_t), [d_t, d_t + d_h) and [d_t + d_h, d_t + d_h + d_w) of
 *     the head dim belong to the t, y and x axes; the features after them are
 *     not rotated;
 *   - pair p of axis a's section (offset o_a, width d_a, p < d_a / 2) is the
 *     features (o_a + 2p, o_a + 2p + 1) when `interleaved` is set, else
 *     (o_a + p, o_a + p + d_a / 2);
 *   - its angle comes as c = cos_a[pos_a * (d_a / 2) + p] and
 *     s = sin_a[pos_a * (d_a / 2) + p] (fp32 tables with n_a rows), so the
 *     frequency schedule is the caller's;
 *   - the pair (x0, x1) becomes (x0 c - x1 s, x0 s + x1 c);
 *   - a token whose position lies outside the tables on any axis (a
 *     coordinate < 0 or >= n_a: text tokens, padding) is not rotated.
 * Each rotated feature is formed in fp64 (a bf16 times an fp32 value is exact
 * there, so the sum is rounded once) and then rounded once to bf16, to
 * nearest with ties to even: the rotated queries and keys are bf16 activations
 * like the ones they replace.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_EXPORT __attribute__((visibility("default")))

static double r_b2d(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* y rounded to the nearest bf16 value, ties to the one with an even last
 * significand bit.  bf16 keeps 8 significant bits; below 2^-126 its values
 * are the multiples of 2^-133.  The two neighbours lo <= |y| < lo + ulp are
 * found by scaling with ulp, and the distances to them are exact in fp64. */
static uint16_t r_d2bf16(double y) {
    const uint16_t sign = signbit(y) ? 0x8000u : 0u;
    const double a = fabs(y);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex); /* a = m 2^ex, m in [0.5, 1) */
    int ue = ex - 8;
    if (ue < -133) ue = -133;
    const double ulp = ldexp(1.0, ue);
    const double n = floor(a / ulp);
    const double lo = n * ulp, hi = lo + ulp;
    const double dlo = a - lo, dhi = hi - a;
    double r;
    if (dlo < dhi)
        r = lo;
    else if (dhi < dlo)
        r = hi;
    else
        r = (fmod(n, 2.0) == 0.0) ? lo : hi;
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7f80u); /* overflow: infinity */
    const float f = (float)r;                                     /* exact */
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    return (uint16_t)(sign | (uint16_t)((w >> 16) & 0x7fffu));
}

/*
 * vdx_oracle_rope3d
 *   x        bf16 bit patterns [B, S, H, D] (host memory).
 *   pos      int32 [B, S, 3]: (t, y, x) of every token.
 *   cos_t, sin_t, cos_h, sin_h, cos_w, sin_w
 *            fp32 tables [n_a, d_a / 2] per axis (may be NULL when d_a = 0).
 *   d_t, d_h, d_w  even section widths, d_t + d_h + d_w <= D.
 *   interleaved    1: pairs (2p, 2p + 1) of a section; 0: (p, p + d_a / 2).
 *   y        out: bf16 bit patterns [B, S, H, D], the rotated features.
 *   yd       out (or NULL): fp64 [B, S, H, D], the same before the rounding.
 * Returns 0 on success, 1 on bad arguments.
 */
ORACLE_EXPORT int vdx_oracle_rope3d(const uint16_t *x, const int32_t *pos, const float *cos_t,
                                    const float *sin_t, const float *cos_h, const float *sin_h,
                                    const float *cos_w, const float *sin_w, int64_t n_t, int64_t n_h,
                                    int64_t n_w, int64_t d_t, int64_t d_h, int64_t d_w, int interleaved,
                                    int64_t B, int64_t S, int64_t H, int64_t D, uint16_t *y, double *yd) {
    if (!x || !pos || !y || B < 1 || S < 1 || H < 1 || D < 1) return 1;
    if (d_t < 0 || d_h < 0 || d_w < 0 || d_t % 2 || d_h % 2 || d_w % 2 || d_t + d_h + d_w > D) return 1;
    if (n_t < 0 || n_h < 0 || n_w < 0) return 1;
    if ((d_t && (!cos_t || !sin_t)) || (d_h && (!cos_h || !sin_h)) || (d_w && (!cos_w || !sin_w))) return 1;
    const float *cs[3] = {cos_t, cos_h, cos_w}, *sn[3] = {sin_t, sin_h, sin_w};
    const int64_t nrow[3] = {n_t, n_h, n_w}, width[3] = {d_t, d_h, d_w};
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t s = 0; s < S; ++s) {
            const int32_t *ps = pos + (b * S + s) * 3;
            int inside = 1;
            for (int a = 0; a < 3; ++a)
                if (ps[a] < 0 || ps[a] >= nrow[a]) inside = 0;
            for (int64_t h = 0; h < H; ++h) {
                const int64_t base = ((b * S + s) * H + h) * D;
                /* start from the unrotated features */
                for (int64_t d = 0; d < D; ++d) {
                    y[base + d] = x[base + d];
                    if (yd) yd[base + d] = r_b2d(x[base + d]);
                }
                if (!inside) continue;
                int64_t off = 0;
                for (int a = 0; a < 3; ++a) {
                    const int64_t half = width[a] / 2;
                    for (int64_t p = 0; p < half; ++p) {
                        const int64_t i0 = interleaved ? off + 2 * p : off + p;
                        const int64_t i1 = interleaved ? off + 2 * p + 1 : off + p + half;
                        const double c = (double)cs[a][ps[a] * half + p];
                        const double sv = (double)sn[a][ps[a] * half + p];
                        const double x0 = r_b2d(x[base + i0]), x1 = r_b2d(x[base + i1]);
                        const double y0 = x0 * c - x1 * sv;
                        const double y1 = x0 * sv + x1 * c;
                        y[base + i0] = r_d2bf16(y0);
                        y[base + i1] = r_d2bf16(y1);
                        if (yd) {
                            yd[base + i0] = y0;
                            yd[base + i1] = y1;
                        }
                    }
                    off += width[a];
                }
            }
        }
    }
    return 0;
}

/* bf16 round-to-nearest-even of fp64 values (the rounding step above, exposed
 * so that the tests can pin it on its own). */
ORACLE_EXPORT void vdx_oracle_round_bf16(const double *v, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = r_d2bf16(v[i]);
}
