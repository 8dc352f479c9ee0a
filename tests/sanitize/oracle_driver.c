/*
 * Exercise of the C oracle (oracle/gdn2_oracle.c) built with AddressSanitizer
 * and UndefinedBehaviorSanitizer.
 *
 * The forward and backward routines run over shapes that reach every branch
 * of their indexing: empty batches and sequences, lengths below, at and past
 * the backward's 64-token checkpoint spans, all prologue flag combinations,
 * column blocks that do and do not divide dv, one and two threads.  Each call
 * must return 0 with finite outputs, and the forward over T tokens must equal
 * two forwards over the halves with the state carried between them (to
 * rounding).  The sanitizers abort the process on any memory or
 * undefined-behaviour error; exit status 0 means every case held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdn2_oracle_f64(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, const float* q, const float* k,
                    const float* v, const float* alpha, const float* b, const float* w, const float* S0, double* o,
                    double* S_out, int nthreads, int64_t col_block, int flags);
int gdn2_oracle_bwd_f64(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, const float* q, const float* k,
                        const float* v, const float* alpha, const float* b, const float* w, const float* S0,
                        const float* dO, const float* dS_T, double* dq, double* dk_out, double* dv_out,
                        double* dalpha, double* db, double* dw, double* dS0, int nthreads, int flags);

static int g_bad = 0;
static uint64_t g_rng = 0x9e3779b97f4a7c15ull;

/* uniform in [lo, hi): a 64-bit linear congruential step, top 24 bits */
static float uni(float lo, float hi)
{
    g_rng = g_rng * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * (float)((g_rng >> 40) * (1.0 / 16777216.0));
}

static float* fill(int64_t n, float lo, float hi)
{
    float* p = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i) p[i] = uni(lo, hi);
    return p;
}

static double* zeros(int64_t n) { return (double*)calloc((size_t)(n > 0 ? n : 1), sizeof(double)); }

static void finite(const char* what, const double* x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) {
            fprintf(stderr, "FAIL %s: non-finite at %lld\n", what, (long long)i);
            ++g_bad;
            return;
        }
}

static void check(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int flags, int64_t col_block, int nthr)
{
    const int64_t nk = B * T * H * dk, nv = B * T * H * dv, ns = B * H * dk * dv;
    const int logits = flags & 1;
    float* q = fill(nk, -1.f, 1.f);
    float* k = fill(nk, -1.f, 1.f);
    float* v = fill(nv, -1.f, 1.f);
    float* alpha = fill(nk, logits ? 1.f : 0.5f, logits ? 4.f : 1.f);
    float* b = fill(nk, logits ? -2.f : 0.f, logits ? 2.f : 1.f);
    float* w = fill(nv, 0.f, 1.f);
    float* S0 = fill(ns, -0.5f, 0.5f);
    float* dO = fill(nv, -1.f, 1.f);
    float* dST = fill(ns, -1.f, 1.f);
    double* o = zeros(nv);
    double* S = zeros(ns);
    char tag[96];
    snprintf(tag, sizeof tag, "B%lld T%lld H%lld dk%lld dv%lld flags %d cb %lld thr %d", (long long)B, (long long)T,
             (long long)H, (long long)dk, (long long)dv, flags, (long long)col_block, nthr);

    if (gdn2_oracle_f64(B, T, H, dk, dv, q, k, v, alpha, b, w, S0, o, S, nthr, col_block, flags) != 0) {
        fprintf(stderr, "FAIL forward %s: status\n", tag);
        ++g_bad;
    }
    finite(tag, o, nv);
    finite(tag, S, ns);

    /* the same tokens in two calls, [0, T1) then [T1, T), state carried in fp32 */
    if (B == 1 && T >= 2) {
        const int64_t T1 = T / 2, T2 = T - T1;
        double* o1 = zeros(T1 * H * dv);
        double* o2 = zeros(T2 * H * dv);
        double* S1 = zeros(ns);
        double* S2 = zeros(ns);
        float* S1f = (float*)malloc((size_t)ns * sizeof(float));
        gdn2_oracle_f64(1, T1, H, dk, dv, q, k, v, alpha, b, w, S0, o1, S1, nthr, col_block, flags);
        for (int64_t i = 0; i < ns; ++i) S1f[i] = (float)S1[i];
        gdn2_oracle_f64(1, T2, H, dk, dv, q + T1 * H * dk, k + T1 * H * dk, v + T1 * H * dv, alpha + T1 * H * dk,
                        b + T1 * H * dk, w + T1 * H * dv, S1f, o2, S2, nthr, col_block, flags);
        double err = 0, ref = 0;
        for (int64_t i = 0; i < ns; ++i) {
            err += (S2[i] - S[i]) * (S2[i] - S[i]);
            ref += S[i] * S[i];
        }
        for (int64_t i = 0; i < T2 * H * dv; ++i) {
            const double d = o2[i] - o[T1 * H * dv + i];
            err += d * d;
            ref += o[T1 * H * dv + i] * o[T1 * H * dv + i];
        }
        if (err > 1e-10 * (ref + 1e-30)) {   /* the carried state is rounded to fp32 once */
            fprintf(stderr, "FAIL split %s: rel %g\n", tag, sqrt(err / (ref + 1e-30)));
            ++g_bad;
        }
        free(o1); free(o2); free(S1); free(S2); free(S1f);
    }

    double* dq = zeros(nk); double* dk_ = zeros(nk); double* dv_ = zeros(nv);
    double* da = zeros(nk); double* db = zeros(nk); double* dw = zeros(nv); double* dS0 = zeros(ns);
    if (gdn2_oracle_bwd_f64(B, T, H, dk, dv, q, k, v, alpha, b, w, S0, dO, dST, dq, dk_, dv_, da, db, dw, dS0, nthr,
                            flags) != 0) {
        fprintf(stderr, "FAIL backward %s: status\n", tag);
        ++g_bad;
    }
    finite(tag, dq, nk); finite(tag, dk_, nk); finite(tag, dv_, nv);
    finite(tag, da, nk); finite(tag, db, nk); finite(tag, dw, nv); finite(tag, dS0, ns);
    /* no initial state and no final-state gradient */
    gdn2_oracle_bwd_f64(B, T, H, dk, dv, q, k, v, alpha, b, w, NULL, dO, NULL, dq, dk_, dv_, da, db, dw, dS0, nthr,
                        flags);

    free(q); free(k); free(v); free(alpha); free(b); free(w); free(S0); free(dO); free(dST);
    free(o); free(S); free(dq); free(dk_); free(dv_); free(da); free(db); free(dw); free(dS0);
}

int main(void)
{
    const int64_t Ts[] = {0, 1, 5, 63, 64, 65, 130};
    for (size_t i = 0; i < sizeof Ts / sizeof Ts[0]; ++i)
        for (int flags = 0; flags < 8; ++flags) {
            if ((flags & 2) && !(flags & 1)) continue;   /* NEG_EIGVAL needs GATE_LOGITS */
            check(1, Ts[i], 2, 8, 12, flags, 5, 1);
        }
    check(0, 10, 2, 8, 8, 0, 8, 1);
    check(2, 70, 3, 16, 16, 7, 16, 2);
    check(2, 33, 1, 4, 6, 1, 100, 2);
    /* bad sizes are refused */
    if (gdn2_oracle_f64(-1, 1, 1, 1, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 0) != -1) ++g_bad;
    if (gdn2_oracle_bwd_f64(1, 1, 1, 0, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                            NULL, NULL, NULL, NULL, 1, 0) != -1)
        ++g_bad;
    printf("oracle driver: %d failed cases\n", g_bad);
    return g_bad == 0 ? 0 : 1;
}
