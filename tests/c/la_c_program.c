/*
 * la_c_program.c - the lightning_attn C ABI used from plain C with the HIP
 * runtime's C API (no Python, no torch): device buffers from hipMalloc, every
 * call enqueued on a created stream.  Built by the package build on the CPU,
 * run by tests/test_gpu_c_program.py on the GPU.
 *
 * Checks (self-consistency, no oracle needed):
 *   1. la_prefill over N + M tokens equals la_prefill over N tokens followed
 *      by M la_decode_step calls, within the bf16 bar (max over (b, h) of the
 *      relative L2 error 2e-2), outputs and final state;
 *   2. la_prefill_varlen over two packed sequences equals two la_prefill
 *      calls, bitwise;
 *   3. argument errors: d = 96 -> LA_ERR_UNSUPPORTED, a null state ->
 *      LA_ERR_INVALID_ARG, la_status_string for every code;
 *   4. la_prefill_varlen_plan answers 0 or 1 for a valid shape and rejects a
 *      null result pointer;
 *   5. la_prefill_ws (the sequence split through a caller's workspace, sized
 *      by la_prefill_workspace_bytes) against la_prefill on a long sequence,
 *      within the bf16 bar, outputs and final state;
 *   6. la_prefill_varlen_from_zero with null states (outputs only) against
 *      la_prefill_varlen on zero states, bitwise.
 * Exit status 0 when every check holds; the first failure is printed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lightning_attn.h"

#define B 1
#define H 4
#define D 64
#define N 150   /* prefill tokens (two full blocks and a ragged tail) */
#define M 6     /* decode steps after it */

static int fail(const char *what)
{
    fprintf(stderr, "la_c_program: %s\n", what);
    return 1;
}

#define HIP_OK(x) do { if ((x) != hipSuccess) return fail(#x); } while (0)

static uint64_t rng = 0x2545f4914f6cdd1dull;

static float urand(void)   /* xorshift64*, uniform in [-1, 1) */
{
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (float)((rng * 0x2545f4914f6cdd1dull) >> 40) / 8388608.0f - 1.0f;
}

static uint16_t to_bf16(float f)   /* round to nearest even */
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* max over (b, h) slices of ||x - r|| / ||r|| over `len` values per slice */
static double max_rel_l2(const float *x, const float *r, int slices, int len)
{
    double worst = 0.0;
    for (int s = 0; s < slices; ++s) {
        double num = 0.0, den = 0.0;
        for (int i = 0; i < len; ++i) {
            const double dlt = (double)x[s * len + i] - r[s * len + i];
            num += dlt * dlt;
            den += (double)r[s * len + i] * r[s * len + i];
        }
        const double e = den > 0 ? sqrt(num / den) : sqrt(num);
        if (e > worst) worst = e;
    }
    return worst;
}

int main(void)
{
    const int T = N + M;
    const size_t act = (size_t)B * H * T * D, st = (size_t)B * H * D * D;
    uint16_t *hq = malloc(act * 2), *hk = malloc(act * 2), *hv = malloc(act * 2);
    float *hs = malloc(st * 4), slopes[H];
    for (size_t i = 0; i < act; ++i) {
        hq[i] = to_bf16(urand() * 0.125f);
        hk[i] = to_bf16(urand() * 0.125f);
        hv[i] = to_bf16(urand());
    }
    for (size_t i = 0; i < st; ++i) hs[i] = 0.1f * urand();
    for (int h = 0; h < H; ++h) slopes[h] = (float)pow(2.0, -8.0 * (h + 1) / H);

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    void *q, *k, *v, *out, *out2;
    float *dslopes, *state, *state2;
    HIP_OK(hipMalloc(&q, act * 2));
    HIP_OK(hipMalloc(&k, act * 2));
    HIP_OK(hipMalloc(&v, act * 2));
    HIP_OK(hipMalloc(&out, act * 2));
    HIP_OK(hipMalloc(&out2, act * 2));
    HIP_OK(hipMalloc((void **)&dslopes, H * 4));
    HIP_OK(hipMalloc((void **)&state, st * 4));
    HIP_OK(hipMalloc((void **)&state2, st * 4));
    HIP_OK(hipMemcpy(q, hq, act * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k, hk, act * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v, hv, act * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dslopes, slopes, H * 4, hipMemcpyHostToDevice));

    /* 1a. one prefill over all T tokens (layout [B][H][T][D]) */
    HIP_OK(hipMemcpy(state, hs, st * 4, hipMemcpyHostToDevice));
    if (la_prefill(q, k, v, dslopes, out, state, B, H, T, D, stream) != LA_OK)
        return fail("la_prefill over T tokens");

    /* 1b. the first N tokens of every head, then M decode steps; the inputs
     *     are re-laid out per call ([B][H][N][D], then [B][H][D] per step) */
    uint16_t *pq = malloc((size_t)B * H * N * D * 2), *pk = malloc((size_t)B * H * N * D * 2),
             *pv = malloc((size_t)B * H * N * D * 2);
    for (int bh = 0; bh < B * H; ++bh) {
        memcpy(pq + (size_t)bh * N * D, hq + (size_t)bh * T * D, (size_t)N * D * 2);
        memcpy(pk + (size_t)bh * N * D, hk + (size_t)bh * T * D, (size_t)N * D * 2);
        memcpy(pv + (size_t)bh * N * D, hv + (size_t)bh * T * D, (size_t)N * D * 2);
    }
    void *q2, *k2, *v2, *o2;
    HIP_OK(hipMalloc(&q2, (size_t)B * H * N * D * 2));
    HIP_OK(hipMalloc(&k2, (size_t)B * H * N * D * 2));
    HIP_OK(hipMalloc(&v2, (size_t)B * H * N * D * 2));
    HIP_OK(hipMalloc(&o2, (size_t)B * H * N * D * 2));
    HIP_OK(hipMemcpy(q2, pq, (size_t)B * H * N * D * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k2, pk, (size_t)B * H * N * D * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v2, pv, (size_t)B * H * N * D * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(state2, hs, st * 4, hipMemcpyHostToDevice));
    if (la_prefill(q2, k2, v2, dslopes, o2, state2, B, H, N, D, stream) != LA_OK)
        return fail("la_prefill over N tokens");
    uint16_t *tq = malloc((size_t)B * H * D * 2), *tk = malloc((size_t)B * H * D * 2),
             *tv = malloc((size_t)B * H * D * 2), *to = malloc((size_t)B * H * D * 2);
    uint16_t *dec_out = malloc((size_t)B * H * M * D * 2);
    void *sq, *sk, *sv, *so;
    HIP_OK(hipMalloc(&sq, (size_t)B * H * D * 2));
    HIP_OK(hipMalloc(&sk, (size_t)B * H * D * 2));
    HIP_OK(hipMalloc(&sv, (size_t)B * H * D * 2));
    HIP_OK(hipMalloc(&so, (size_t)B * H * D * 2));
    for (int t = 0; t < M; ++t) {
        for (int bh = 0; bh < B * H; ++bh) {
            memcpy(tq + (size_t)bh * D, hq + ((size_t)bh * T + N + t) * D, D * 2);
            memcpy(tk + (size_t)bh * D, hk + ((size_t)bh * T + N + t) * D, D * 2);
            memcpy(tv + (size_t)bh * D, hv + ((size_t)bh * T + N + t) * D, D * 2);
        }
        HIP_OK(hipMemcpyAsync(sq, tq, (size_t)B * H * D * 2, hipMemcpyHostToDevice, stream));
        HIP_OK(hipMemcpyAsync(sk, tk, (size_t)B * H * D * 2, hipMemcpyHostToDevice, stream));
        HIP_OK(hipMemcpyAsync(sv, tv, (size_t)B * H * D * 2, hipMemcpyHostToDevice, stream));
        if (la_decode_step(sq, sk, sv, dslopes, state2, so, B, H, D, stream) != LA_OK)
            return fail("la_decode_step");
        HIP_OK(hipMemcpyAsync(to, so, (size_t)B * H * D * 2, hipMemcpyDeviceToHost, stream));
        HIP_OK(hipStreamSynchronize(stream));
        for (int bh = 0; bh < B * H; ++bh)
            memcpy(dec_out + ((size_t)bh * M + t) * D, to + (size_t)bh * D, D * 2);
    }
    HIP_OK(hipStreamSynchronize(stream));

    /* compare the last M tokens' outputs and the final states */
    uint16_t *full = malloc(act * 2);
    float *fs = malloc(st * 4), *fs2 = malloc(st * 4);
    HIP_OK(hipMemcpy(full, out, act * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(fs, state, st * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(fs2, state2, st * 4, hipMemcpyDeviceToHost));
    float *a = malloc((size_t)B * H * M * D * 4), *r = malloc((size_t)B * H * M * D * 4);
    for (int bh = 0; bh < B * H; ++bh)
        for (int t = 0; t < M; ++t)
            for (int i = 0; i < D; ++i) {
                a[((size_t)bh * M + t) * D + i] = from_bf16(dec_out[((size_t)bh * M + t) * D + i]);
                r[((size_t)bh * M + t) * D + i] = from_bf16(full[((size_t)bh * T + N + t) * D + i]);
            }
    const double eo = max_rel_l2(a, r, B * H, M * D), es = max_rel_l2(fs2, fs, B * H, D * D);
    printf("prefill(N) + %d decode steps vs prefill(N+%d): out %.3e, state %.3e\n", M, M, eo, es);
    if (!(eo <= 2e-2) || !(es <= 2e-2)) return fail("decode continuation differs from prefill");

    /* 2. packed: sequences of 70 and 86 tokens ([H][T][D], B = 1) against
     *    separate dense calls over each sequence */
    {
        const int64_t cu_h[3] = {0, 70, T};
        int64_t *cu;
        HIP_OK(hipMalloc((void **)&cu, 3 * 8));
        HIP_OK(hipMemcpy(cu, cu_h, 3 * 8, hipMemcpyHostToDevice));
        float *sts;
        HIP_OK(hipMalloc((void **)&sts, 2 * st * 4));
        HIP_OK(hipMemcpy(sts, hs, st * 4, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy((char *)sts + st * 4, hs, st * 4, hipMemcpyHostToDevice));
        if (la_prefill_varlen(q, k, v, dslopes, cu, 2, out2, sts, H, T, D, stream) != LA_OK)
            return fail("la_prefill_varlen");
        uint16_t *packed = malloc(act * 2);
        float *pst = malloc(2 * st * 4);
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipMemcpy(packed, out2, act * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(pst, sts, 2 * st * 4, hipMemcpyDeviceToHost));
        for (int sq_i = 0; sq_i < 2; ++sq_i) {
            const int a0 = (int)cu_h[sq_i], n = (int)(cu_h[sq_i + 1] - cu_h[sq_i]);
            uint16_t *xq = malloc((size_t)H * n * D * 2), *xk = malloc((size_t)H * n * D * 2),
                     *xv = malloc((size_t)H * n * D * 2), *xo = malloc((size_t)H * n * D * 2);
            for (int h = 0; h < H; ++h) {
                memcpy(xq + (size_t)h * n * D, hq + ((size_t)h * T + a0) * D, (size_t)n * D * 2);
                memcpy(xk + (size_t)h * n * D, hk + ((size_t)h * T + a0) * D, (size_t)n * D * 2);
                memcpy(xv + (size_t)h * n * D, hv + ((size_t)h * T + a0) * D, (size_t)n * D * 2);
            }
            HIP_OK(hipMemcpy(q2, xq, (size_t)H * n * D * 2, hipMemcpyHostToDevice));
            HIP_OK(hipMemcpy(k2, xk, (size_t)H * n * D * 2, hipMemcpyHostToDevice));
            HIP_OK(hipMemcpy(v2, xv, (size_t)H * n * D * 2, hipMemcpyHostToDevice));
            HIP_OK(hipMemcpy(state2, hs, st * 4, hipMemcpyHostToDevice));
            if (la_prefill(q2, k2, v2, dslopes, o2, state2, 1, H, n, D, stream) != LA_OK)
                return fail("la_prefill per sequence");
            HIP_OK(hipStreamSynchronize(stream));
            HIP_OK(hipMemcpy(xo, o2, (size_t)H * n * D * 2, hipMemcpyDeviceToHost));
            HIP_OK(hipMemcpy(fs2, state2, st * 4, hipMemcpyDeviceToHost));
            for (int h = 0; h < H; ++h)
                if (memcmp(xo + (size_t)h * n * D, packed + ((size_t)h * T + a0) * D,
                           (size_t)n * D * 2) != 0)
                    return fail("packed output differs from the per-sequence call");
            if (memcmp(fs2, pst + (size_t)sq_i * st, st * 4) != 0)
                return fail("packed state differs from the per-sequence call");
            free(xq); free(xk); free(xv); free(xo);
        }
        printf("packed prefill of 2 sequences == per-sequence prefill (bitwise)\n");
        free(packed); free(pst);
        HIP_OK(hipFree(cu));
        HIP_OK(hipFree(sts));
    }

    /* 3. argument errors are reported on the host, nothing is launched */
    if (la_prefill(q, k, v, dslopes, out, state, B, H, T, 96, stream) != LA_ERR_UNSUPPORTED)
        return fail("d = 96 not reported as unsupported");
    if (la_prefill(q, k, v, dslopes, out, NULL, B, H, T, D, stream) != LA_ERR_INVALID_ARG)
        return fail("null state not reported");
    for (int c = 0; c <= 3; ++c)
        if (!la_status_string(c) || !la_status_string(c)[0]) return fail("la_status_string");
    if (la_abi_version() != LA_ABI_VERSION) return fail("ABI version");

    /* 4. the packed prefill's work split for a shape (no GPU work) */
    {
        int walks = -1;
        if (la_prefill_varlen_plan(74, 64, 262144, 128, &walks) != LA_OK || (walks != 0 && walks != 1))
            return fail("la_prefill_varlen_plan");
        if (la_prefill_varlen_plan(74, 64, 262144, 128, NULL) != LA_ERR_INVALID_ARG)
            return fail("la_prefill_varlen_plan with a null result");
        printf("packed prefill of 74 sequences x 64 heads: %s\n",
               walks ? "one workgroup per head and 32 columns walks the sequences"
                     : "one workgroup per sequence, head and 32 columns");
    }

    /* 5. the sequence split through a caller's workspace: one long sequence */
    {
        const int64_t NL = 20000;
        const size_t la = (size_t)H * NL * D;
        uint16_t *lq = malloc(la * 2), *lk = malloc(la * 2), *lv = malloc(la * 2);
        for (size_t i = 0; i < la; ++i) {
            lq[i] = to_bf16(urand() * 0.125f);
            lk[i] = to_bf16(urand() * 0.125f);
            lv[i] = to_bf16(urand());
        }
        void *xq, *xk, *xv, *xo, *xo2, *work = NULL;
        float *xs, *xs2;
        HIP_OK(hipMalloc(&xq, la * 2));
        HIP_OK(hipMalloc(&xk, la * 2));
        HIP_OK(hipMalloc(&xv, la * 2));
        HIP_OK(hipMalloc(&xo, la * 2));
        HIP_OK(hipMalloc(&xo2, la * 2));
        HIP_OK(hipMalloc((void **)&xs, (size_t)H * D * D * 4));
        HIP_OK(hipMalloc((void **)&xs2, (size_t)H * D * D * 4));
        HIP_OK(hipMemcpy(xq, lq, la * 2, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(xk, lk, la * 2, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(xv, lv, la * 2, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(xs, hs, (size_t)H * D * D * 4, hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(xs2, hs, (size_t)H * D * D * 4, hipMemcpyHostToDevice));
        int64_t wsb = -1;
        if (la_prefill_workspace_bytes(1, H, NL, D, &wsb) != LA_OK || wsb < 0)
            return fail("la_prefill_workspace_bytes");
        if (wsb > 0) HIP_OK(hipMalloc(&work, (size_t)wsb));     /* hipMalloc: 256-byte aligned */
        if (la_prefill_ws(xq, xk, xv, dslopes, xo, xs, 1, H, NL, D, work, wsb, stream) != LA_OK)
            return fail("la_prefill_ws");
        if (la_prefill(xq, xk, xv, dslopes, xo2, xs2, 1, H, NL, D, stream) != LA_OK)
            return fail("la_prefill over the long sequence");
        HIP_OK(hipStreamSynchronize(stream));
        uint16_t *ho = malloc(la * 2), *ho2 = malloc(la * 2);
        float *fo = malloc(la * 4), *fo2 = malloc(la * 4), *hs1 = malloc((size_t)H * D * D * 4),
              *hs2 = malloc((size_t)H * D * D * 4);
        HIP_OK(hipMemcpy(ho, xo, la * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(ho2, xo2, la * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(hs1, xs, (size_t)H * D * D * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(hs2, xs2, (size_t)H * D * D * 4, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < la; ++i) {
            fo[i] = from_bf16(ho[i]);
            fo2[i] = from_bf16(ho2[i]);
        }
        const double e5o = max_rel_l2(fo, fo2, H, (int)(NL * D)), e5s = max_rel_l2(hs1, hs2, H, D * D);
        printf("la_prefill_ws (%lld workspace bytes) vs la_prefill over %lld tokens: out %.3e, state %.3e\n",
               (long long)wsb, (long long)NL, e5o, e5s);
        if (!(e5o <= 2e-2) || !(e5s <= 2e-2)) return fail("la_prefill_ws differs from la_prefill");
        if (work) HIP_OK(hipFree(work));
        HIP_OK(hipFree(xq)); HIP_OK(hipFree(xk)); HIP_OK(hipFree(xv)); HIP_OK(hipFree(xo));
        HIP_OK(hipFree(xo2)); HIP_OK(hipFree(xs)); HIP_OK(hipFree(xs2));
        free(lq); free(lk); free(lv); free(ho); free(ho2); free(fo); free(fo2); free(hs1); free(hs2);
    }

    /* 6. fresh sequences, outputs only: null states against zero states */
    {
        const int64_t cu_h[4] = {0, 70, 71, T};
        int64_t *cu;
        float *zst;
        HIP_OK(hipMalloc((void **)&cu, 4 * 8));
        HIP_OK(hipMemcpy(cu, cu_h, 4 * 8, hipMemcpyHostToDevice));
        HIP_OK(hipMalloc((void **)&zst, 3 * st * 4));
        HIP_OK(hipMemset(zst, 0, 3 * st * 4));
        if (la_prefill_varlen(q, k, v, dslopes, cu, 3, out, zst, H, T, D, stream) != LA_OK)
            return fail("la_prefill_varlen on zero states");
        if (la_prefill_varlen_from_zero(q, k, v, dslopes, cu, 3, out2, NULL, H, T, D,
                                        (int64_t)T * D, D, (int64_t)T * D, D, stream) != LA_OK)
            return fail("la_prefill_varlen_from_zero with null states");
        HIP_OK(hipStreamSynchronize(stream));
        uint16_t *o1 = malloc(act * 2), *o2h = malloc(act * 2);
        HIP_OK(hipMemcpy(o1, out, act * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(o2h, out2, act * 2, hipMemcpyDeviceToHost));
        if (memcmp(o1, o2h, act * 2) != 0) return fail("outputs-only packed prefill differs");
        printf("packed prefill from zero, null states == zero states (bitwise)\n");
        free(o1); free(o2h);
        HIP_OK(hipFree(cu));
        HIP_OK(hipFree(zst));
    }

    HIP_OK(hipStreamDestroy(stream));
    printf("la_c_program: all checks passed\n");
    return 0;
}
