/*
 * resolvent_oracle.c -- plain fp64 CPU oracle of the resolvent operator head.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  The product path (the
 * HIP library and its Python binding) never calls it, and it shares no code,
 * header, table or constant with that path.
 *
 * What it computes follows the "Resolvent Operator" page (teerth.dev,
 * Aether-Lang/integrated/resolvent):
 *   - section "Object": the scaled logit s_ij = <q_i,k_j>/sqrt(d), the blended
 *     gate m_k = clamp(lerp(1,u_k,g),0,1), theta'_k = g*theta_k, the gate
 *     a_k = m_k e^{i theta'_k}, the path product G_ij = prod_{k=j+1..i} a_k
 *     (G_ii = 1), its modulus R_ij = prod m_k, the row normaliser
 *     Z_i = sum_{j<=i} R_ij e^{qk s_ij}, the weights
 *     W_ij = G_ij e^{qk s_ij} / Z_i^beta (0 above the diagonal) and the
 *     readout O_i = sum_{j<=i} W_ij V_j;
 *   - section "Evaluation and refusals": Z_i^beta in the log domain,
 *     W_ij = G_ij exp(qk s_ij - beta log Z_i), log Z_i from a sum shifted by
 *     its maximum over the live entries (R_ij > 0); the refusal table
 *     (non-finite q, k, u, theta or switch, overflowing g*theta_k, overflowing
 *     logit), the empty sequence, and the overflow rule away from beta = 1
 *     (a dead entry is exactly 0, a lane of G that is exactly 0 stays 0);
 *   - section "Rust API": blend, gate, path_product accumulating from k = i
 *     down to k = j+1 with a_0 never read, operator, readout, chain_label;
 *   - section "The path-product corner is a resolvent": the chain
 *     y_0 = 0, y_i = a_i y_{i-1} + b_i.
 *
 * Readings where the page leaves a step open (each is listed in the design
 * notes of the repository):
 *   lerp(1,u,g) = (1-g)*1 + g*u, evaluated without a fused multiply-add, so it
 *   is exact at g = 0 and g = 1; the clamp applies after the lerp; the maximum
 *   that shifts log Z is taken over the logits qk*s_ij of the live entries;
 *   dot products and sums run in ascending index order; every entry of u and
 *   theta (index 0 included) is checked for finiteness; a logit is checked for
 *   overflow for every j <= i when qk != 0, and qk = 0 never forms the dot
 *   product.  Built with -ffp-contract=off so that no multiply-add is fused.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_NONFINITE 1
#define ORACLE_BAD_SHAPE 2
#define ORACLE_BAD_ARG 3

/* blend(u, theta, g) -> (m, theta'): "Object", blended gate. */
void oracle_blend(double u, double theta, double g, double *m, double *theta_p) {
    double l = (1.0 - g) * 1.0 + g * u; /* lerp(1, u, g) */
    if (l < 0.0) l = 0.0;
    if (l > 1.0) l = 1.0;
    *m = l;
    *theta_p = g * theta;
}

/* gate(m, theta') = m e^{i theta'}: "Object", the gate. */
void oracle_gate(double m, double theta_p, double *re, double *im) {
    *re = m * cos(theta_p);
    *im = m * sin(theta_p);
}

/* gates(u, theta, g) -> a [n]: blend then gate at every position, as the
 * head's validation does; returns ORACLE_NONFINITE at the first non-finite
 * u, theta or g*theta (a is then partly written). */
int oracle_gates(const double *u, const double *theta, int64_t n, double g, double *a_re,
                 double *a_im) {
    for (int64_t k = 0; k < n; ++k) {
        double m, tp;
        if (!isfinite(u[k]) || !isfinite(theta[k])) return ORACLE_NONFINITE;
        oracle_blend(u[k], theta[k], g, &m, &tp);
        if (!isfinite(tp)) return ORACLE_NONFINITE;
        oracle_gate(m, tp, &a_re[k], &a_im[k]);
    }
    return ORACLE_OK;
}

/* Complex product x * a, textbook form. */
static inline void cmul(double xr, double xi, double ar, double ai, double *r, double *i) {
    *r = xr * ar - xi * ai;
    *i = xr * ai + xi * ar;
}

/* path_product(a) -> G, row-major [n, n]: "Rust API".  Row i is built from
 * G_ii = 1 by multiplying in a_i, a_{i-1}, ..., a_{j+1} in that order; entries
 * above the diagonal are 0; a_0 is never read. */
void oracle_path_product(const double *a_re, const double *a_im, int64_t n,
                         double *g_re, double *g_im) {
    for (int64_t i = 0; i < n; ++i) {
        double *gr = g_re + i * n, *gi = g_im + i * n;
        for (int64_t j = 0; j < n; ++j) { gr[j] = 0.0; gi[j] = 0.0; }
        gr[i] = 1.0;
        gi[i] = 0.0;
        for (int64_t j = i - 1; j >= 0; --j)
            cmul(gr[j + 1], gi[j + 1], a_re[j + 1], a_im[j + 1], &gr[j], &gi[j]);
    }
}

/* R_ij = prod_{k=j+1..i} m_k, same order as the path product: "Object". */
void oracle_modulus(const double *m, int64_t n, double *r) {
    for (int64_t i = 0; i < n; ++i) {
        double *ri = r + i * n;
        for (int64_t j = 0; j < n; ++j) ri[j] = 0.0;
        ri[i] = 1.0;
        for (int64_t j = i - 1; j >= 0; --j) ri[j] = ri[j + 1] * m[j + 1];
    }
}

/* chain_label(a, b): y_0 = 0, y_i = a_i y_{i-1} + b_i (the page's chain, whose
 * b_0 is 0).  With y0_from_b0 != 0 the chain starts at y_0 = b_0 instead, which
 * is the readout of the path-product corner for an arbitrary b_0. */
void oracle_chain(const double *a_re, const double *a_im, const double *b, int64_t n,
                  int32_t y0_from_b0, double *y_re, double *y_im) {
    if (n <= 0) return;
    y_re[0] = y0_from_b0 ? b[0] : 0.0;
    y_im[0] = 0.0;
    for (int64_t i = 1; i < n; ++i) {
        double r, im;
        cmul(a_re[i], a_im[i], y_re[i - 1], y_im[i - 1], &r, &im);
        y_re[i] = r + b[i];
        y_im[i] = im;
    }
}

/* readout(W, V) -> O [n, dv]: "Object", the readout; j ascending. */
void oracle_readout(const double *w_re, const double *w_im, const double *v, int64_t n,
                    int64_t dv, double *o_re, double *o_im) {
    for (int64_t i = 0; i < n; ++i)
        for (int64_t c = 0; c < dv; ++c) {
            double sr = 0.0, si = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                sr += w_re[i * n + j] * v[j * dv + c];
                si += w_im[i * n + j] * v[j * dv + c];
            }
            o_re[i * dv + c] = sr;
            o_im[i * dv + c] = si;
        }
}

/* ---- one head ---------------------------------------------------------- */

typedef struct {
    const double *q, *k, *u, *theta, *v; /* q,k [n,d]; u,theta [n]; v [n,dv] */
    int64_t n, d, dv;
    double beta, qk, g;
    double *m, *a_re, *a_im; /* per-position gates (length n) */
} head_t;

/* Validation of one head's inputs ("Evaluation and refusals": non-finite
 * query, key, magnitude, phase; blended phase g*theta_k that overflows), then
 * blend and gate for every position. */
static int head_prepare(head_t *hd) {
    const int64_t n = hd->n, d = hd->d;
    for (int64_t x = 0; x < n * d; ++x)
        if (!isfinite(hd->q[x]) || !isfinite(hd->k[x])) return ORACLE_NONFINITE;
    for (int64_t x = 0; x < n; ++x) {
        if (!isfinite(hd->u[x]) || !isfinite(hd->theta[x])) return ORACLE_NONFINITE;
        double m, tp;
        oracle_blend(hd->u[x], hd->theta[x], hd->g, &m, &tp);
        if (!isfinite(tp)) return ORACLE_NONFINITE;
        hd->m[x] = m;
        oracle_gate(m, tp, &hd->a_re[x], &hd->a_im[x]);
    }
    return ORACLE_OK;
}

/* Weights of row i, W_ij for j = 0..i, into w_re/w_im; scratch needs 4*(i+1)
 * doubles.  Returns ORACLE_NONFINITE when a logit overflows. */
static int row_weights(const head_t *hd, int64_t i, double *w_re, double *w_im,
                       double *scratch) {
    const int64_t d = hd->d;
    double *gr = scratch, *gi = scratch + (i + 1), *r = scratch + 2 * (i + 1),
           *L = scratch + 3 * (i + 1);
    /* path product and modulus of row i, k = i down to j+1 */
    gr[i] = 1.0;
    gi[i] = 0.0;
    r[i] = 1.0;
    for (int64_t j = i - 1; j >= 0; --j) {
        cmul(gr[j + 1], gi[j + 1], hd->a_re[j + 1], hd->a_im[j + 1], &gr[j], &gi[j]);
        r[j] = r[j + 1] * hd->m[j + 1];
    }
    /* logits qk * s_ij; qk = 0 removes q and k without forming the dot */
    const double rootd = sqrt((double)d);
    for (int64_t j = 0; j <= i; ++j) {
        if (hd->qk == 0.0) {
            L[j] = 0.0;
            continue;
        }
        const double *qi = hd->q + i * d, *kj = hd->k + j * d;
        double dot = 0.0;
        for (int64_t e = 0; e < d; ++e) dot += qi[e] * kj[e];
        double s = dot / rootd;
        L[j] = hd->qk * s;
        if (!isfinite(L[j])) return ORACLE_NONFINITE;
    }
    /* log Z_i from the live entries, shifted by their maximum logit */
    double M = -INFINITY;
    for (int64_t j = 0; j <= i; ++j)
        if (r[j] > 0.0 && L[j] > M) M = L[j];
    double S = 0.0;
    for (int64_t j = 0; j <= i; ++j)
        if (r[j] > 0.0) S += r[j] * exp(L[j] - M);
    const double logZ = M + log(S);
    /* W_ij = G_ij exp(qk s_ij - beta log Z_i); a dead entry is exactly 0 and a
     * lane of G that is exactly 0 stays 0 */
    for (int64_t j = 0; j <= i; ++j) {
        if (r[j] == 0.0) {
            w_re[j] = 0.0;
            w_im[j] = 0.0;
            continue;
        }
        double E = exp(L[j] - hd->beta * logZ);
        w_re[j] = (gr[j] == 0.0) ? 0.0 : gr[j] * E;
        w_im[j] = (gi[j] == 0.0) ? 0.0 : gi[j] * E;
    }
    return ORACLE_OK;
}

static int check_switches(double beta, double qk, double g) {
    return (isfinite(beta) && isfinite(qk) && isfinite(g)) ? ORACLE_OK : ORACLE_NONFINITE;
}

/* operator(q, k, u, theta, seq, head_dim, switches) -> W [n, n]: "Rust API".
 * Empty in, empty out; head_dim = 0 with n > 0 is a shape error. */
int oracle_operator(const double *q, const double *k, const double *u, const double *theta,
                    int64_t n, int64_t d, double beta, double qk, double g, double *w_re,
                    double *w_im) {
    if (n < 0 || d < 0) return ORACLE_BAD_SHAPE;
    if (n == 0) return ORACLE_OK;
    if (d == 0) return ORACLE_BAD_SHAPE;
    int st = check_switches(beta, qk, g);
    if (st) return st;
    head_t hd = {q, k, u, theta, NULL, n, d, 0, beta, qk, g, NULL, NULL, NULL};
    double *buf = (double *)malloc(sizeof(double) * (size_t)(3 * n + 4 * n));
    if (!buf) return ORACLE_BAD_ARG;
    hd.m = buf;
    hd.a_re = buf + n;
    hd.a_im = buf + 2 * n;
    double *scratch = buf + 3 * n;
    st = head_prepare(&hd);
    for (int64_t i = 0; i < n && st == ORACLE_OK; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            w_re[i * n + j] = 0.0;
            w_im[i * n + j] = 0.0;
        }
        st = row_weights(&hd, i, w_re + i * n, w_im + i * n, scratch);
    }
    free(buf);
    return st;
}

/* Readout of selected rows of one head: o_re/o_im [nrows, dv].  The refusal
 * checks cover every input of the head and the logits of the rows computed. */
static int head_rows(head_t *hd, const int64_t *rows, int64_t nrows, double *o_re,
                     double *o_im, int nthreads) {
    const int64_t n = hd->n, dv = hd->dv;
    int status = ORACLE_OK;
#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
#endif
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(6 * n));
        int local = w ? ORACLE_OK : ORACLE_BAD_ARG;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t x = 0; x < nrows; ++x) {
            if (local != ORACLE_OK) continue;
            const int64_t i = rows[x];
            double *w_re = w, *w_im = w + n, *scratch = w + 2 * n;
            int st = row_weights(hd, i, w_re, w_im, scratch);
            if (st != ORACLE_OK) {
                local = st;
                continue;
            }
            for (int64_t c = 0; c < dv; ++c) {
                double sr = 0.0, si = 0.0;
                for (int64_t j = 0; j <= i; ++j) {
                    sr += w_re[j] * hd->v[j * dv + c];
                    si += w_im[j] * hd->v[j * dv + c];
                }
                o_re[x * dv + c] = sr;
                o_im[x * dv + c] = si;
            }
        }
        free(w);
        if (local != ORACLE_OK) {
#ifdef _OPENMP
#pragma omp critical
#endif
            if (status == ORACLE_OK) status = local;
        }
    }
    return status;
}

/* Forward pass, selected rows of one head (b, h): q,k [n,d], v [n,dv],
 * u,theta [n]; rows[x] in [0, n); o_re/o_im [nrows, dv]. */
int oracle_forward_rows(const double *q, const double *k, const double *u,
                        const double *theta, const double *v, int64_t n, int64_t d,
                        int64_t dv, double beta, double qk, double g, const int64_t *rows,
                        int64_t nrows, double *o_re, double *o_im, int32_t nthreads) {
    if (n < 0 || d < 0 || dv < 0 || nrows < 0) return ORACLE_BAD_SHAPE;
    if (n == 0) return ORACLE_OK;
    if (d == 0) return ORACLE_BAD_SHAPE;
    int st = check_switches(beta, qk, g);
    if (st) return st;
    for (int64_t x = 0; x < nrows; ++x)
        if (rows[x] < 0 || rows[x] >= n) return ORACLE_BAD_ARG;
    head_t hd = {q, k, u, theta, v, n, d, dv, beta, qk, g, NULL, NULL, NULL};
    double *buf = (double *)malloc(sizeof(double) * (size_t)(3 * n));
    if (!buf) return ORACLE_BAD_ARG;
    hd.m = buf;
    hd.a_re = buf + n;
    hd.a_im = buf + 2 * n;
    st = head_prepare(&hd);
    if (st == ORACLE_OK) st = head_rows(&hd, rows, nrows, o_re, o_im, nthreads);
    free(buf);
    return st;
}

/* Forward pass over B*H heads: q,k [B,H,n,d], v [B,H,n,dv], u,theta [B,H,n],
 * o_re/o_im [B,H,n,dv]. */
int oracle_forward(const double *q, const double *k, const double *u, const double *theta,
                   const double *v, int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv,
                   double beta, double qk, double g, double *o_re, double *o_im,
                   int32_t nthreads) {
    if (B < 0 || H < 0 || n < 0 || d < 0 || dv < 0) return ORACLE_BAD_SHAPE;
    if (B == 0 || H == 0 || n == 0) return ORACLE_OK;
    if (d == 0) return ORACLE_BAD_SHAPE;
    int st = check_switches(beta, qk, g);
    if (st) return st;
    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!rows) return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) rows[i] = i;
    for (int64_t bh = 0; bh < B * H && st == ORACLE_OK; ++bh)
        st = oracle_forward_rows(q + bh * n * d, k + bh * n * d, u + bh * n, theta + bh * n,
                                 v + bh * n * dv, n, d, dv, beta, qk, g, rows, n,
                                 o_re + bh * n * dv, o_im + bh * n * dv, nthreads);
    free(rows);
    return st;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
