/*
 * Driver for the sanitizer build of the fp64 oracle (test infrastructure):
 * calls every entry point of oracle/resolvent_oracle.c on the kinds of inputs
 * the pin tests use -- small heads over a switch grid with interior and
 * extreme values, clamped and exactly closed gates, the empty sequence,
 * head_dim 0, non-finite inputs of each refused class, row subsets and
 * several threads -- with every output buffer sized exactly.  Built with
 * -fsanitize=address,undefined; any report fails the run.  The values are
 * not checked here (the pin tests do that); a status that contradicts the
 * refusal table of "Evaluation and refusals" exits nonzero.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_blend(double u, double theta, double g, double *m, double *theta_p);
void oracle_gate(double m, double theta_p, double *re, double *im);
int oracle_gates(const double *u, const double *theta, int64_t n, double g, double *a_re,
                 double *a_im);
void oracle_path_product(const double *a_re, const double *a_im, int64_t n, double *g_re,
                         double *g_im);
void oracle_modulus(const double *m, int64_t n, double *r);
void oracle_chain(const double *a_re, const double *a_im, const double *b, int64_t n,
                  int32_t y0_from_b0, double *y_re, double *y_im);
void oracle_readout(const double *w_re, const double *w_im, const double *v, int64_t n,
                    int64_t dv, double *o_re, double *o_im);
int oracle_operator(const double *q, const double *k, const double *u, const double *theta,
                    int64_t n, int64_t d, double beta, double qk, double g, double *w_re,
                    double *w_im);
int oracle_forward_rows(const double *q, const double *k, const double *u, const double *theta,
                        const double *v, int64_t n, int64_t d, int64_t dv, double beta,
                        double qk, double g, const int64_t *rows, int64_t nr, double *o_re,
                        double *o_im, int32_t nthreads);
int oracle_forward(const double *q, const double *k, const double *u, const double *theta,
                   const double *v, int64_t B, int64_t H, int64_t n, int64_t d, int64_t dv,
                   double beta, double qk, double g, double *o_re, double *o_im,
                   int32_t nthreads);
int oracle_max_threads(void);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double unif(double lo, double hi) { /* xorshift64*, uniform in [lo, hi) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    const uint64_t x = state * 0x2545F4914F6CDD1Dull;
    return lo + (hi - lo) * (double)(x >> 11) * (1.0 / 9007199254740992.0);
}
static double *fill(int64_t cnt, double lo, double hi) {
    double *p = malloc(sizeof(double) * (size_t)(cnt > 0 ? cnt : 1));
    for (int64_t i = 0; i < cnt; ++i) p[i] = unif(lo, hi);
    return p;
}
static double *zeros(int64_t cnt) { return calloc((size_t)(cnt > 0 ? cnt : 1), sizeof(double)); }

static int failures = 0;
static void expect(int got, int want, const char *what) {
    if (got != want) {
        printf("status %d, expected %d: %s\n", got, want, what);
        ++failures;
    }
}

static void one_head(int64_t n, int64_t d, int64_t dv) {
    static const double grid[][3] = {{1, 1, 0},     {0, 1, 0},       {0, 0, 1},   {0.5, 0.7, 0.5},
                                     {0.3, -1.3, 1.4}, {1.7, 0.4, -0.3}, {1, 1, 1}, {0, 0, 0}};
    double *q = fill(n * d, -2, 2), *k = fill(n * d, -2, 2), *v = fill(n * dv, -1, 1);
    double *u = fill(n, -0.5, 1.5), *th = fill(n, -4, 4);
    if (n > 3) u[n / 2] = 0.0; /* a closed gate at g = 1 */
    double *wr = zeros(n * n), *wi = zeros(n * n), *orr = zeros(n * dv), *oi = zeros(n * dv);
    int64_t *rows = malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) rows[i] = n - 1 - i;
    for (size_t s = 0; s < sizeof grid / sizeof grid[0]; ++s) {
        const double b = grid[s][0], qk = grid[s][1], g = grid[s][2];
        expect(oracle_operator(q, k, u, th, n, d, b, qk, g, wr, wi), 0, "operator");
        oracle_readout(wr, wi, v, n, dv, orr, oi);
        expect(oracle_forward_rows(q, k, u, th, v, n, d, dv, b, qk, g, rows, n, orr, oi, 1), 0,
               "forward_rows, 1 thread");
        expect(oracle_forward_rows(q, k, u, th, v, n, d, dv, b, qk, g, rows, n / 2, orr, oi, 3), 0,
               "forward_rows, 3 threads, half the rows");
    }
    double *ar = zeros(n), *ai = zeros(n), *gr = zeros(n * n), *gi = zeros(n * n);
    expect(oracle_gates(u, th, n, 0.8, ar, ai), 0, "gates");
    oracle_path_product(ar, ai, n, gr, gi);
    oracle_modulus(u, n, gr);
    oracle_chain(ar, ai, v, n, 0, orr, oi);
    oracle_chain(ar, ai, v, n, 1, orr, oi);
    if (n > 0) { /* each refused class, index 0 included */
        const double bad[2] = {NAN, INFINITY};
        for (int x = 0; x < 2; ++x) {
            double keep = q[0];
            q[0] = bad[x];
            expect(oracle_operator(q, k, u, th, n, d, 1, 1, 1, wr, wi), 1, "non-finite q");
            q[0] = keep;
            keep = k[n * d - 1];
            k[n * d - 1] = bad[x];
            expect(oracle_forward_rows(q, k, u, th, v, n, d, dv, 1, 1, 1, rows, n, orr, oi, 2), 1,
                   "non-finite k");
            k[n * d - 1] = keep;
            keep = u[0];
            u[0] = bad[x];
            expect(oracle_gates(u, th, n, 0.5, ar, ai), 1, "non-finite u");
            u[0] = keep;
            keep = th[n - 1];
            th[n - 1] = bad[x];
            expect(oracle_operator(q, k, u, th, n, d, 1, 1, 1, wr, wi), 1, "non-finite theta");
            th[n - 1] = keep;
            expect(oracle_operator(q, k, u, th, n, d, bad[x], 1, 1, wr, wi), 1, "non-finite beta");
        }
    }
    free(q); free(k); free(v); free(u); free(th); free(wr); free(wi); free(orr); free(oi);
    free(rows); free(ar); free(ai); free(gr); free(gi);
}

int main(void) {
    double m, tp, re, im;
    oracle_blend(0.3, 1.0, 1.0, &m, &tp);
    oracle_gate(m, tp, &re, &im);
    oracle_gate(1.0, 3.141592653589793, &re, &im);
    static const int64_t shapes[][3] = {{0, 4, 4}, {1, 1, 1}, {2, 3, 2}, {3, 2, 5},
                                        {5, 4, 4}, {8, 3, 1}, {17, 8, 3}, {40, 16, 6}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        one_head(shapes[s][0], shapes[s][1], shapes[s][2]);
    { /* head_dim 0 with positions: a shape error, outputs untouched */
        double u[3] = {1, 1, 1}, th[3] = {0, 0, 0}, w[9], x[1] = {0};
        expect(oracle_operator(x, x, u, th, 3, 0, 1, 1, 1, w, w), 2, "head_dim 0");
    }
    { /* batched forward, several threads */
        const int64_t B = 2, H = 2, n = 33, d = 8, dv = 5;
        double *q = fill(B * H * n * d, -1, 1), *k = fill(B * H * n * d, -1, 1);
        double *v = fill(B * H * n * dv, -1, 1), *u = fill(B * H * n, 0, 1);
        double *th = fill(B * H * n, -3, 3);
        double *orr = zeros(B * H * n * dv), *oi = zeros(B * H * n * dv);
        expect(oracle_forward(q, k, u, th, v, B, H, n, d, dv, 0.5, 0.7, 0.5, orr, oi, 4), 0,
               "forward");
        free(q); free(k); free(v); free(u); free(th); free(orr); free(oi);
    }
    printf("oracle cases done, %d failures, %d threads available\n", failures,
           oracle_max_threads());
    return failures != 0;
}
