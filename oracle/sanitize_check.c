/*
 * sanitize_check.c — drives the C oracle (la_oracle.c) under AddressSanitizer
 * and UndefinedBehaviorSanitizer on the host (TEST INFRASTRUCTURE: built and
 * run by tests/test_oracle_sanitized.py only).
 *
 * Cases: a multi-slice prefill from a random state against the same tokens fed
 * one decode step at a time (the recurrence is one loop in both, so the
 * results are bitwise equal); an empty sequence leaves the state untouched; an
 * infinite slope (lambda = 0) and a zero slope (lambda = 1); rejected
 * arguments.  Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int la_oracle_prefill(const double *q, const double *k, const double *v, const double *slopes,
                      double *state, double *out, int64_t B, int64_t H, int64_t N, int64_t d);
int la_oracle_decode_step(const double *q, const double *k, const double *v,
                          const double *slopes, double *state, double *out, int64_t B,
                          int64_t H, int64_t d);

static uint64_t rng = 0x9e3779b97f4a7c15ull;

static double urand(void)   /* xorshift64, uniform in [-1, 1) */
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}

static double *fill(size_t n)
{
    double *p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = urand();
    return p;
}

static int check(int ok, const char *what)
{
    if (!ok) fprintf(stderr, "sanitize_check: %s failed\n", what);
    return ok ? 0 : 1;
}

int main(void)
{
    enum { B = 2, H = 3, N = 37, D = 5 };
    const size_t act = (size_t)B * H * N * D, st = (size_t)B * H * D * D;
    double *q = fill(act), *k = fill(act), *v = fill(act), *s0 = fill(st);
    double slopes[H] = {0.0, 0.25, INFINITY};           /* lambda = 1, e^-0.25, 0 */
    int bad = 0;

    /* prefill from s0 */
    double *sp = malloc(st * sizeof(double)), *op = malloc(act * sizeof(double));
    memcpy(sp, s0, st * sizeof(double));
    bad += check(la_oracle_prefill(q, k, v, slopes, sp, op, B, H, N, D) >= 1, "prefill status");

    /* the same tokens one decode step at a time */
    double *sd = malloc(st * sizeof(double)), *od = malloc(act * sizeof(double));
    double *qt = malloc((size_t)B * H * D * sizeof(double)), *kt = malloc((size_t)B * H * D * sizeof(double));
    double *vt = malloc((size_t)B * H * D * sizeof(double)), *ot = malloc((size_t)B * H * D * sizeof(double));
    memcpy(sd, s0, st * sizeof(double));
    for (int t = 0; t < N; ++t) {
        for (int bh = 0; bh < B * H; ++bh)
            for (int i = 0; i < D; ++i) {
                const size_t src = ((size_t)bh * N + t) * D + i, dst = (size_t)bh * D + i;
                qt[dst] = q[src];
                kt[dst] = k[src];
                vt[dst] = v[src];
            }
        bad += check(la_oracle_decode_step(qt, kt, vt, slopes, sd, ot, B, H, D) >= 1, "decode status");
        for (int bh = 0; bh < B * H; ++bh)
            for (int i = 0; i < D; ++i) od[((size_t)bh * N + t) * D + i] = ot[(size_t)bh * D + i];
    }
    bad += check(memcmp(op, od, act * sizeof(double)) == 0, "prefill == decode steps (outputs)");
    bad += check(memcmp(sp, sd, st * sizeof(double)) == 0, "prefill == decode steps (states)");

    /* lambda = 0: the last token alone, o_t = (q_t . k_t) v_t */
    {
        const int h = 2, b = 1, t = N - 1;
        const size_t row = ((size_t)(b * H + h) * N + t) * D;
        double qk = 0.0;
        for (int i = 0; i < D; ++i) qk += q[row + i] * k[row + i];
        double err = 0.0;
        for (int j = 0; j < D; ++j) err = fmax(err, fabs(op[row + j] - qk * v[row + j]));
        bad += check(err < 1e-12, "lambda = 0 closed form");
    }

    /* empty sequence: the state is untouched */
    double *se = malloc(st * sizeof(double));
    memcpy(se, s0, st * sizeof(double));
    bad += check(la_oracle_prefill(q, k, v, slopes, se, NULL, B, H, 0, D) >= 1, "empty status");
    bad += check(memcmp(se, s0, st * sizeof(double)) == 0, "empty sequence keeps the state");

    /* rejected arguments */
    bad += check(la_oracle_prefill(NULL, k, v, slopes, se, NULL, B, H, N, D) == -1, "null q");
    bad += check(la_oracle_prefill(q, k, v, slopes, se, NULL, B, H, -1, D) == -1, "negative N");
    bad += check(la_oracle_prefill(q, k, v, slopes, se, NULL, B, H, N, 0) == -1, "d = 0");

    free(q); free(k); free(v); free(s0); free(sp); free(op); free(sd); free(od);
    free(qt); free(kt); free(vt); free(ot); free(se);
    if (!bad) printf("sanitize_check: all checks passed\n");
    return bad ? 1 : 0;
}
