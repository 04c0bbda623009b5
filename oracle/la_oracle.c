/*
 * la_oracle.c — fp64 CPU oracle for decayed causal linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this.  It shares no code, header or
 * table with the GPU library: it is a second, independent statement of what
 * the layer computes, written to be checked by eye.
 *
 * What it computes (the plain recurrent definition, no blocking):
 *   per (b, h), with lambda = exp(-slope[h]) in fp64 and S = S_init[b,h]:
 *     for t = 0 .. N-1:
 *       S[i][j] = lambda * S[i][j] + k[t][i] * v[t][j]     (all i, j < d)
 *       o[t][j] = sum_i q[t][i] * S[i][j]
 *   i.e. o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s + lambda^(t+1) q_t S_init,
 *   and the final state is S_{N-1}.
 *
 * Source: Ling and Ring 2.6 Technical Report (translation on
 * garden.houmin.site), §4.1.1 "Context Parallel for Lightning Attention":
 * linear attention is evaluated as an RNN-style recurrence that carries a
 * per-(batch, head) D x D state ([B,H,D,D]); Fig. 2 places the kernel
 * between RoPE and the grouped RMSNorm, so nothing inside it normalises or
 * scales q.k.  The per-head exponential decay lambda_h = exp(-s_h) with
 * s_h = 2^(-8(h+1)/H) is the Lightning Attention decay the layer is built
 * for; the pages do not print it (readings listed with the design notes).
 *
 * Layouts: q, k, v, o are [B][H][N][d] row-major fp64; state is [B][H][d][d]
 * with i (the k index) slow and j (the v index) fast.  slopes is [H].
 * Parallel over the B*H independent slices with OpenMP.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One (b, h) slice: the recurrence above, token by token. */
static void recurrent_slice(const double *q, const double *k, const double *v,
                            double lambda, double *S, double *o,
                            int64_t N, int64_t d)
{
    for (int64_t t = 0; t < N; ++t) {
        const double *qt = q + t * d, *kt = k + t * d, *vt = v + t * d;
        /* state update: S = lambda * S + k_t^T v_t */
        for (int64_t i = 0; i < d; ++i) {
            double *Si = S + i * d;
            for (int64_t j = 0; j < d; ++j)
                Si[j] = lambda * Si[j] + kt[i] * vt[j];
        }
        /* read-out: o_t = q_t S */
        if (o) {
            double *ot = o + t * d;
            for (int64_t j = 0; j < d; ++j) ot[j] = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                const double qi = qt[i];
                const double *Si = S + i * d;
                for (int64_t j = 0; j < d; ++j) ot[j] += qi * Si[j];
            }
        }
    }
}

/*
 * Prefill over N tokens.  state: [B,H,d,d], IN = S_init, OUT = S_{N-1}.
 * out: [B,H,N,d] or NULL (state only).  Returns the number of OpenMP threads
 * used (>= 1), or -1 on bad arguments.
 */
/* Threads the oracle's parallel loops use from now on (n >= 1); timing aid
 * only, the results do not depend on it. */
void la_oracle_set_threads(int n)
{
    if (n >= 1) omp_set_num_threads(n);
}

int la_oracle_prefill(const double *q, const double *k, const double *v,
                      const double *slopes, double *state, double *out,
                      int64_t B, int64_t H, int64_t N, int64_t d)
{
    if (!q || !k || !v || !slopes || !state || B < 0 || H < 0 || N < 0 || d < 1)
        return -1;
    int threads = 1;
    const int64_t BH = B * H;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            threads = omp_get_num_threads();
#endif
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < BH; ++bh) {
            const double lambda = exp(-slopes[bh % H]);
            const int64_t off = bh * N * d;
            recurrent_slice(q + off, k + off, v + off, lambda, state + bh * d * d,
                            out ? out + off : NULL, N, d);
        }
    }
    return threads;
}

/*
 * One decode step for B*H sequences: q, k, v, out are [B,H,d]; state is
 * [B,H,d,d] updated in place (S = lambda S + k^T v, then o = q S).
 */
int la_oracle_decode_step(const double *q, const double *k, const double *v,
                          const double *slopes, double *state, double *out,
                          int64_t B, int64_t H, int64_t d)
{
    return la_oracle_prefill(q, k, v, slopes, state, out, B, H, 1, d);
}
